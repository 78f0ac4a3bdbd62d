// One recurrent step of the selective scan from a carried state (`selective_scan_ref`'s loop
// body for one t, as the `Mamba` module's token-by-token inference path on the "Vision Mamba
// structure and principle" page, section 2, advances its ssm_state):
//   delta = softplus(delta_raw + bias);  h <- exp(delta A) h + delta B x  (in place)
//   y = <C, h> + D x;  out = y * silu(z)
// P lanes per row (b, d), one per (padded) state, so the state is read and written coalesced;
// y is summed over the row's lanes with xor shuffles.  Memory-bound: 8 bytes of state traffic
// per (row, state).
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

template <typename T, int P>
__global__ __launch_bounds__(256) void scan_step_kernel(const StepParams p) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gid / P;
  const int n = int(gid % P);
  const bool valid = row < p.batch * p.dim;
  const int64_t r = valid ? row : 0;
  const int64_t b = r / p.dim, d = r % p.dim, g = d / (p.dim / p.G);
  const bool has_n = valid && n < p.N;
  const float x = Elem<T>::load(static_cast<const T*>(p.x), r);
  const float w = (Elem<T>::load(static_cast<const T*>(p.delta), r) + (p.delta_bias ? p.delta_bias[d] : 0.0f)) * kLog2e;
  const float lam = p.softplus ? softplus_log2<sizeof(T) == 4>(w) : w;  // delta / ln 2
  float part = 0.0f;
  if (has_n) {
    const int64_t si = r * p.N + n;
    const int64_t bi = (b * p.G + g) * p.N + n;
    const float bn = Elem<T>::load(static_cast<const T*>(p.Bm), bi);
    const float cn = Elem<T>::load(static_cast<const T*>(p.Cm), bi);
    const float h = fmaf(fast_exp2(lam * p.A[d * p.N + n]), p.state[si], lam * kLn2 * bn * x);
    p.state[si] = h;
    part = cn * h;
  }
#pragma unroll
  for (int m = P / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, kWave);
  if (valid && n == 0) {
    float y = part;
    if (p.Dskip) y = fmaf(p.Dskip[d], x, y);
    if (p.z) y *= silu(Elem<T>::load(static_cast<const T*>(p.z), r));
    Elem<T>::store(static_cast<T*>(p.out), r, y);
  }
}

template <typename T, int P>
hipError_t launch_p(const StepParams& p, hipStream_t s) {
  const int64_t threads = p.batch * p.dim * P;
  scan_step_kernel<T, P><<<dim3(uint32_t((threads + 255) / 256)), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const StepParams& p, hipStream_t s) {
  const int P = padded_states(p.N);
  if (P == 1) return launch_p<T, 1>(p, s);
  if (P == 4) return launch_p<T, 4>(p, s);
  if (P == 8) return launch_p<T, 8>(p, s);
  if (P == 16) return launch_p<T, 16>(p, s);
  if (P == 32) return launch_p<T, 32>(p, s);
  return launch_p<T, 64>(p, s);
}

}  // namespace

hipError_t launch_scan_step(const StepParams& p, hipStream_t s) {
  if (p.batch * p.dim == 0) return hipSuccess;
  return p.dtype == 0 ? launch_t<float>(p, s) : launch_t<bf16>(p, s);
}

}  // namespace ss2d
