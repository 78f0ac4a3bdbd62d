// Issue-rate probe for the vector ALU of gfx950 (measurement support, not part of the SS2D
// library): how many SIMD cycles a wave64 FMA, a v_exp_f32 and the scan's per-(step, state)
// instruction mix take, so that the scan kernels' arithmetic roofline rests on a measurement.
//
// Every wavefront runs `iters` iterations of a block of independent dependency chains (eight
// per lane, so that issue, not latency, limits it) entirely in registers, and lane 0 records
// the shader-clock counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime) before and after the loop.  From them: cycles per block for this wavefront,
// and the clock it ran at.  With k wavefronts per SIMD sharing one vector unit, cycles per
// instruction per SIMD = cycles per block / (instructions per block * k).
//
// kind 0: FMA      x = fma(x, c1, c2)                       8 v_fmac per chain step
// kind 1: exp      x = exp2(-x)                              8 v_exp_f32 per chain step
// kind 2: scan mix a = exp2(lam * A_n); h_n = fma(a, h_n, du * B_n); acc = fma(C_n, h_n, acc)
//                  for 8 states: 8 x (v_mul, v_exp, v_mul, v_fma, v_fma) per step, the
//                  instructions the scan issues per (element, state), plus one v_fma per step
//                  that varies lam and du (so nothing is loop-invariant)
// Outputs: stamps[4 w + {0,1,2,3}] = clock start, clock end, real start, real end of wave w;
// sink receives one value per lane (never read; it keeps the chains live).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int kKind>
__global__ __launch_bounds__(64) void valu_probe_kernel(int64_t iters, uint64_t* stamps, float* sink) {
  const int lane = threadIdx.x;
  float x[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) x[i] = 0.25f + 0.01f * float(i + lane % 7);
  float A[kChains], B[kChains], C[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    A[i] = -0.5f - 0.125f * float(i);
    B[i] = 0.03f * float(i + 1);
    C[i] = 0.5f - 0.05f * float(i);
  }
  float lam = 0.05f + 0.001f * float(lane), du = 0.1f, acc = 0.0f;
  __syncthreads();
  const uint64_t c0 = clock64();
  const uint64_t r0 = wall_clock64();
  for (int64_t it = 0; it < iters; ++it) {
    if constexpr (kKind == 0) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < kChains; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
    } else if constexpr (kKind == 1) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < kChains; ++i) x[i] = ex2(-x[i]);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kChains; ++i) {
          const float a = ex2(lam * A[i]);
          x[i] = fmaf(a, x[i], du * B[i]);
          acc = fmaf(C[i], x[i], acc);
        }
        lam = fmaf(acc, 1e-6f, lam);  // one per step, as the scan's per-step work
        du = acc;
      }
    }
  }
  const uint64_t c1 = clock64();
  const uint64_t r1 = wall_clock64();
  float v = acc;
#pragma unroll
  for (int i = 0; i < kChains; ++i) v += x[i];
  const int64_t w = blockIdx.x;
  sink[w * 64 + lane] = v;
  if (lane == 0) {
    stamps[4 * w] = c0;
    stamps[4 * w + 1] = c1;
    stamps[4 * w + 2] = r0;
    stamps[4 * w + 3] = r1;
  }
}

}  // namespace

extern "C" {

// VALU instructions per loop iteration and lane for each kind (what the cycle counts divide by)
int valu_probe_insts_per_iter(int kind) {
  if (kind == 0 || kind == 1) return 8 * kChains;
  if (kind == 2) return 8 * (5 * kChains + 1);
  return 0;
}

// Launches `waves` wavefronts of 64 lanes on `stream`.  stamps: 4 * waves uint64; sink: 64 * waves
// floats (device buffers owned by the caller).  Returns 0, 1 for invalid arguments, 3 for a launch
// error.
int valu_probe_run(int kind, int64_t waves, int64_t iters, uint64_t* stamps, float* sink, hipStream_t stream) {
  if (waves < 1 || waves > 0x7fffffff || iters < 1 || !stamps || !sink || kind < 0 || kind > 2) return 1;
  const dim3 grid{uint32_t(waves)}, block{64};
  if (kind == 0)
    valu_probe_kernel<0><<<grid, block, 0, stream>>>(iters, stamps, sink);
  else if (kind == 1)
    valu_probe_kernel<1><<<grid, block, 0, stream>>>(iters, stamps, sink);
  else
    valu_probe_kernel<2><<<grid, block, 0, stream>>>(iters, stamps, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
