// Dense fp32 products of the Δ/B/C producer (the per-route x_proj and dt_proj of the scanned
// sequence, the `Mamba` module's projections on "Vision Mamba structure and principle", section
// 2) and of its gradient, on the matrix cores: v_mfma_f32_32x32x2f32, fp32 operands and
// accumulation (no rounding of any operand).
//
// One workgroup computes a 64 x 64 tile of C with four wavefronts (2 x 2 blocks of 32 x 32, 16
// accumulators per lane).  K advances in chunks of 32: each thread loads 8 elements of the A tile
// and 8 of the B tile (strided views, addresses clamped and out-of-range values zeroed by a
// select, so the loads carry no branch), the tiles go through LDS k-major, and each wavefront
// issues 16 MFMAs per chunk.  Lane layout of the instruction (checked on the device): lane l
// supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator v of lane l is
// C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTM = 64, kTN = 64, kTK = 32, kThreads = 256, kPad = 4;

// Address of element (r, c) of an operand view, batch (b0, b1); ncols = the column extent (for
// reversed columns).  Segment pointers are picked by selects (no dynamic indexing of the
// argument block).
__device__ __forceinline__ const float* opnd_addr(const GemmOpnd& o, int64_t r, int64_t c, int64_t ncols, int64_t b0,
                                                  int64_t b1) {
  const bool s1 = r >= o.split1, s2 = r >= o.split2;
  const float* p = s2 ? o.p[2] : (s1 ? o.p[1] : o.p[0]);
  const int64_t sr = s2 ? o.s_r[2] : (s1 ? o.s_r[1] : o.s_r[0]);
  const int64_t sb0 = s2 ? o.s_b0[2] : (s1 ? o.s_b0[1] : o.s_b0[0]);
  const int64_t sb1 = s2 ? o.s_b1[2] : (s1 ? o.s_b1[1] : o.s_b1[0]);
  const int64_t r0 = s2 ? o.split2 : (s1 ? o.split1 : 0);
  const int64_t cc = o.rev_c ? ncols - 1 - c : c;
  return p + b0 * sb0 + b1 * sb1 + (r - r0) * sr + cc * o.s_c;
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ float As[kTK][kTM + kPad];  // k-major: As[kk][i]
  __shared__ float Bs[kTK][kTN + kPad];  // Bs[kk][j]
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t m0 = int64_t(blockIdx.y) * kTM, n0 = int64_t(blockIdx.x) * kTN;
  int64_t b1, b0_begin, b0_end, split = 0;
  if (g.sum_b0) {
    split = blockIdx.z % g.b0_splits;
    b1 = blockIdx.z / g.b0_splits;
    const int64_t per = (g.nb0 + g.b0_splits - 1) / g.b0_splits;
    b0_begin = split * per;
    b0_end = b0_begin + per < g.nb0 ? b0_begin + per : g.nb0;
  } else {
    b0_begin = blockIdx.z % g.nb0;
    b0_end = b0_begin + 1;
    b1 = blockIdx.z / g.nb0;
  }
  // each thread's 8 elements of a tile: unit-stride index fastest across threads
  const bool a_kfast = g.a.s_c == 1, b_nfast = g.b.s_c == 1;
  floatx16 acc = {};
  for (int64_t b0 = b0_begin; b0 < b0_end; ++b0) {
    for (int64_t k0 = 0; k0 < g.K; k0 += kTK) {
      float va[8], vb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = t + kThreads * q;
        const int ia = a_kfast ? e / kTK : e % kTM, ka = a_kfast ? e % kTK : e / kTM;
        const int64_t ri = m0 + ia, ck = k0 + ka;
        const bool ina = ri < g.M && ck < g.K;
        const float x = *opnd_addr(g.a, ina ? ri : 0, ina ? ck : 0, g.K, b0, b1);
        va[q] = ina ? x : 0.0f;
        const int kb = b_nfast ? e / kTN : e % kTK, jb = b_nfast ? e % kTN : e / kTK;
        const int64_t rk = k0 + kb, cj = n0 + jb;
        const bool inb = rk < g.K && cj < g.N;
        const float y = *opnd_addr(g.b, inb ? rk : 0, inb ? cj : 0, g.N, b0, b1);
        vb[q] = inb ? y : 0.0f;
      }
      __syncthreads();  // the previous chunk's MFMAs have read the tiles
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = t + kThreads * q;
        const int ia = a_kfast ? e / kTK : e % kTM, ka = a_kfast ? e % kTK : e / kTM;
        const int kb = b_nfast ? e / kTN : e % kTK, jb = b_nfast ? e % kTN : e / kTK;
        As[ka][ia] = va[q];
        Bs[kb][jb] = vb[q];
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kTK / 2; ++s) {
        const float a = As[2 * s + lane / 32][wm * 32 + lane % 32];
        const float b = Bs[2 * s + lane / 32][wn * 32 + lane % 32];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
    }
  }
  const int64_t cb0 = g.sum_b0 ? 0 : b0_begin;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t i = m0 + wm * 32 + (v / 4) * 8 + (lane / 32) * 4 + v % 4;
    const int64_t j = n0 + wn * 32 + lane % 32;
    if (i < g.M && j < g.N) {
      float* c = const_cast<float*>(opnd_addr(g.c, i, j, g.N, cb0, b1)) + split * g.c_split;
      *c = g.accumulate ? *c + acc[v] : acc[v];
    }
  }
}

__global__ __launch_bounds__(256) void sum_parts_kernel(const float* part, float* out, int64_t n, int64_t n_parts) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int64_t k = 0; k < n_parts; ++k) s += part[k * n + i];
  out[i] = s;
}

// 32 x 32 tile of one plane: fp32 copy in grid order and, through LDS, transposed
template <typename T>
__global__ __launch_bounds__(256) void cast_transpose_kernel(const T* x, float* xf, float* xfT, int64_t C, int H,
                                                             int W) {
  __shared__ float tile[32][33];
  const int tw = (W + 31) / 32, th = (H + 31) / 32;
  int64_t bid = blockIdx.x;
  const int t = int(bid % (int64_t(tw) * th));
  const int64_t plane = bid / (int64_t(tw) * th);
  const int h0 = (t / tw) * 32, w0 = (t % tw) * 32;
  const int64_t base = plane * int64_t(H) * W;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = h0 + ty + 8 * r, w = w0 + tx;
    if (h < H && w < W) {
      const float v = Elem<T>::load(x, base + int64_t(h) * W + w);
      xf[base + int64_t(h) * W + w] = v;
      tile[ty + 8 * r][tx] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int w = w0 + ty + 8 * r, h = h0 + tx;
    if (h < H && w < W) xfT[base + int64_t(w) * H + h] = tile[tx][ty + 8 * r];
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int64_t tm = (g.M + kTM - 1) / kTM, tn = (g.N + kTN - 1) / kTN;
  const int64_t z = g.sum_b0 ? g.b0_splits * g.nb1 : g.nb0 * g.nb1;
  if (tm > 65535 || z > 65535 || tn > int64_t(INT32_MAX) || z <= 0) return hipErrorInvalidValue;
  if (g.sum_b0 && (g.b0_splits <= 0 || g.b0_splits > g.nb0)) return hipErrorInvalidValue;
  gemm_kernel<<<dim3(uint32_t(tn), uint32_t(tm), uint32_t(z)), dim3(kThreads), 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* part, float* out, int64_t n, int64_t n_parts, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  sum_parts_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s>>>(part, out, n, n_parts);
  return hipGetLastError();
}

hipError_t launch_cast_transpose(const void* x, float* xf, float* xfT, int64_t batch, int64_t C, int64_t H,
                                 int64_t W, int dtype, hipStream_t s) {
  const int64_t blocks = batch * C * ((H + 31) / 32) * ((W + 31) / 32);
  if (blocks == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  if (dtype == 0)
    cast_transpose_kernel<float><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(static_cast<const float*>(x), xf, xfT,
                                                                             C, int(H), int(W));
  else
    cast_transpose_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(static_cast<const bf16*>(x), xf, xfT, C,
                                                                            int(H), int(W));
  return hipGetLastError();
}

}  // namespace ss2d
