// Selective scan backward: dispatch over (dtype, state count), the chunk combine of the adjoint,
// and the kernel that adds the per-block / per-chunk partial sums into dA, dD, ddelta_bias, dB, dC.
#include "device_common.h"
#include "internal.h"

namespace ss2d {

template <typename T, int NS, typename TU>
hipError_t scan_bwd_launch(const ScanBwdParams& p, hipStream_t s);

namespace {

// One thread per (row, state): walk the chunks from the last to the first.  On entry
// lam_carry[row][c] is chunk c's adjoint at its start computed from zero; on exit it is the
// adjoint flowing into chunk c from all later chunks.
__global__ __launch_bounds__(256) void lambda_combine_kernel(const ScanBwdParams p) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rows = p.batch * p.dim;
  if (i >= rows * p.N) return;
  const int64_t row = i / p.N;
  const int n = int(i % p.N);
  const float A = p.A[(row % p.dim) * p.N + n];
  float m = 0.0f;
  for (int c = p.n_chunks - 1; c >= 0; --c) {
    float* slot = p.lam_carry + (row * p.n_chunks + c) * p.N + n;
    const float loc = *slot;
    *slot = m;
    m = fmaf(fast_exp2(A * p.chunk_sum[row * p.n_chunks + c]), m, loc);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void reduce_bc_kernel(const BwdReduceArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_block = a.batch * a.G * a.N * a.L;
  if (i >= per_block) return;
  float sb = 0.0f, sc = 0.0f;
  for (int64_t k = 0; k < a.dblocks; ++k) {
    sb += a.dB_part[k * per_block + i];
    sc += a.dC_part[k * per_block + i];
  }
  const int64_t nl = int64_t(a.N) * a.L;
  const int64_t o = a.bc_out_stride ? (i / nl) * a.bc_out_stride + i % nl : i;
  Elem<T>::store(static_cast<T*>(a.dB), o, sb * kLn2);  // dB terms were formed with delta / ln 2
  Elem<T>::store(static_cast<T*>(a.dC), o, sc);
}

// The same for partial sums in 4-step blocks of all states ((b, g) block, t / 4, n, t % 4): one
// thread per (block, 4-step group, state) adds four steps at once, so a wavefront reads whole
// lines of every partial-sum block.
template <typename T>
__global__ __launch_bounds__(256) void reduce_bc_blocked_kernel(const BwdReduceArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // (bg, t / 4, n)
  const int64_t per_block = a.batch * a.G * a.N * a.L;
  if (i * 4 >= per_block) return;
  float4 sb = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sc = sb;
  for (int64_t k = 0; k < a.dblocks; ++k) {
    // read once: past the caches
    typedef float F4 __attribute__((ext_vector_type(4)));
    const F4 vb = __builtin_nontemporal_load(reinterpret_cast<const F4*>(a.dB_part + k * per_block + 4 * i));
    const F4 vc = __builtin_nontemporal_load(reinterpret_cast<const F4*>(a.dC_part + k * per_block + 4 * i));
    sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
    sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
  }
  const int64_t groups = a.L / 4;
  const int64_t n = i % a.N, t = ((i / a.N) % groups) * 4, bg = i / (a.N * groups);
  const int64_t o = bg * (a.bc_out_stride ? a.bc_out_stride : int64_t(a.N) * a.L) + n * a.L + t;
  // dB terms were formed with delta / ln 2
  Elem<T>::store4(static_cast<T*>(a.dB), o, make_float4(sb.x * kLn2, sb.y * kLn2, sb.z * kLn2, sb.w * kLn2));
  Elem<T>::store4(static_cast<T*>(a.dC), o, sc);
}

// 64 outputs per workgroup (dA entries, then (dD, dbias) pairs); its four wavefronts take every
// fourth image, and their sums are added in a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void reduce_params_kernel(const BwdReduceArgs a) {
  __shared__ float red[4][kWave][2];
  const int lane = int(threadIdx.x) % kWave, w = int(threadIdx.x) / kWave;
  const int64_t i = int64_t(blockIdx.x) * kWave + lane;
  const int64_t rows = a.batch * a.dim, nA = a.dim * a.N;
  float s0 = 0.0f, s1 = 0.0f;
  if (i < nA) {
    const int64_t d = i / a.N, n = i % a.N;
    for (int c = 0; c < a.n_chunks; ++c) {
#pragma unroll 4
      for (int64_t b = w; b < a.batch; b += 4) s0 += a.dA_part[(int64_t(c) * rows + b * a.dim + d) * a.N + n];
    }
  } else if (i < nA + a.dim) {
    const int64_t d = i - nA;
    for (int c = 0; c < a.n_chunks; ++c) {
#pragma unroll 4
      for (int64_t b = w; b < a.batch; b += 4) {
        s0 += a.dD_part[int64_t(c) * rows + b * a.dim + d];
        s1 += a.dbias_part[int64_t(c) * rows + b * a.dim + d];
      }
    }
  }
  red[w][lane][0] = s0;
  red[w][lane][1] = s1;
  __syncthreads();
  if (w != 0) return;
  const float t0 = (red[0][lane][0] + red[1][lane][0]) + (red[2][lane][0] + red[3][lane][0]);
  const float t1 = (red[0][lane][1] + red[1][lane][1]) + (red[2][lane][1] + red[3][lane][1]);
  if (i < nA) {
    a.dA[i] = t0 * kLn2;  // dA terms were formed with delta / ln 2
  } else if (i < nA + a.dim) {
    const int64_t d = i - nA;
    if (a.dD) a.dD[d] = t0;
    if (a.dbias) a.dbias[d] = t1;
  }
}

template <typename T, typename TU>
hipError_t launch_dtype(const ScanBwdParams& p, hipStream_t s) {
  if (p.N <= 1) return scan_bwd_launch<T, 1, TU>(p, s);
  if (p.N <= 4) return scan_bwd_launch<T, 4, TU>(p, s);
  if (p.N <= 8) return scan_bwd_launch<T, 8, TU>(p, s);
  if (p.N <= 16) return scan_bwd_launch<T, 16, TU>(p, s);
  if (p.N <= 32) return scan_bwd_launch<T, 32, TU>(p, s);
  return scan_bwd_launch<T, 64, TU>(p, s);
}

}  // namespace

hipError_t launch_scan_bwd(const ScanBwdParams& p, hipStream_t s) {
  if (p.dtype == 0) return launch_dtype<float, float>(p, s);
  return p.u_f32 ? launch_dtype<bf16, float>(p, s) : launch_dtype<bf16, bf16>(p, s);
}

hipError_t launch_lambda_combine(const ScanBwdParams& p, hipStream_t s) {
  const int64_t n = p.batch * p.dim * p.N;
  if (n == 0) return hipSuccess;
  lambda_combine_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdReduceArgs& a, hipStream_t s) {
  const int64_t nbc = a.batch * a.G * a.N * a.L;
  if (nbc > 0 && a.bc_blocked) {
    const int64_t threads = nbc / 4;
    if (a.dtype == 0)
      reduce_bc_blocked_kernel<float><<<dim3(uint32_t((threads + 255) / 256)), dim3(256), 0, s>>>(a);
    else
      reduce_bc_blocked_kernel<bf16><<<dim3(uint32_t((threads + 255) / 256)), dim3(256), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (nbc > 0) {
    if (a.dtype == 0)
      reduce_bc_kernel<float><<<dim3(uint32_t((nbc + 255) / 256)), dim3(256), 0, s>>>(a);
    else
      reduce_bc_kernel<bf16><<<dim3(uint32_t((nbc + 255) / 256)), dim3(256), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t np = a.dim * a.N + a.dim;
  if (np > 0) reduce_params_kernel<<<dim3(uint32_t((np + kWave - 1) / kWave)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ss2d
