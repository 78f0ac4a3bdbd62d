// Selective scan forward: dispatch over (dtype, state count) and the chunk-combine kernel.
// The kernel itself is in scan_fwd_kernel.h; its instantiations live in scan_fwd_inst_*.hip so
// that they compile in parallel.
#include "device_common.h"
#include "internal.h"

namespace ss2d {

template <typename T, int NS, typename TU>
hipError_t scan_fwd_launch(const ScanFwdParams& p, hipStream_t s);

namespace {

// One thread per (row, state): walk the chunks in order.
__global__ __launch_bounds__(256) void chunk_combine_kernel(const ScanFwdParams p) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rows = p.batch * p.dim;
  if (i >= rows * p.N) return;
  const int64_t row = i / p.N;
  const int n = int(i % p.N);
  const int64_t d = row % p.dim;
  const float A = p.A[d * p.N + n];
  float h = 0.0f;
  for (int c = 0; c < p.n_chunks; ++c) {
    float* slot = p.ckpt + (((int64_t(c) * p.chunk_len) / p.ckpt_every) * rows + row) * p.N + n;
    if (c > 0) h = fmaf(fast_exp2(A * p.chunk_sum[row * p.n_chunks + c - 1]), h, *slot);
    *slot = h;
  }
}


template <typename T, typename TU>
hipError_t launch_dtype(const ScanFwdParams& p, hipStream_t s) {
  if (p.N <= 1) return scan_fwd_launch<T, 1, TU>(p, s);
  if (p.N <= 4) return scan_fwd_launch<T, 4, TU>(p, s);
  if (p.N <= 8) return scan_fwd_launch<T, 8, TU>(p, s);
  if (p.N <= 16) return scan_fwd_launch<T, 16, TU>(p, s);
  if (p.N <= 32) return scan_fwd_launch<T, 32, TU>(p, s);
  return scan_fwd_launch<T, 64, TU>(p, s);
}

}  // namespace

hipError_t launch_scan_fwd(const ScanFwdParams& p, hipStream_t s) {
  if (p.dtype == 0) return launch_dtype<float, float>(p, s);
  return p.u_f32 ? launch_dtype<bf16, float>(p, s) : launch_dtype<bf16, bf16>(p, s);
}

hipError_t launch_chunk_combine(const ScanFwdParams& p, hipStream_t s) {
  const int64_t n = p.batch * p.dim * p.N;
  if (n == 0) return hipSuccess;
  chunk_combine_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace ss2d
