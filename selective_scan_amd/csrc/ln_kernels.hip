// The VSS block's back half after the SS2D merge: LayerNorm over the channels of each pixel,
// then the gate (the VSS block description in "Vision Mamba structure and principle",
// section 1: the SS2D features are layer-normalised and multiplied by the other branch, whose
// activation is SiLU).  Forward and backward; all arithmetic in fp32 on the fp32 merged map,
// one rounding to the I/O type at the end.
//
// A workgroup takes 64 consecutive pixels of one image, one per lane, and eight wavefronts that
// split the channels (channel c goes to wavefront c % 8): every load of a channel's 64 pixels
// is one contiguous 256-byte segment.  The per-pixel statistics are summed over the eight
// wavefronts in LDS.  The mean and variance use sums shifted by the pixel's first channel, so
// that a large mean does not cancel the variance's digits.  Up to 256 channels a lane keeps its
// channels' values in registers between the statistics and the outputs, so each input is read
// once; wider maps are read again (from L2).
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
static_assert(kLnPixels == kWave, "one pixel per lane");

struct PixelBlock {
  int64_t base;  // offset of (image, channel 0, pixel) in a (batch, C, L) map
  bool active;   // the pixel exists (the last block of an image may be partial)
};

__device__ __forceinline__ PixelBlock pixel_block(const LnArgs& a) {
  const int64_t per = (a.L + kLnPixels - 1) / kLnPixels;
  const int64_t img = blockIdx.x / per;
  const int64_t p = (blockIdx.x % per) * kLnPixels + threadIdx.x % kWave;
  PixelBlock pb;
  pb.active = p < a.L;
  pb.base = img * a.C * a.L + (pb.active ? p : 0);
  return pb;
}

// Adds the wavefronts' values of this lane's pixel in a fixed order.
__device__ __forceinline__ float pixel_sum(float (*red)[kLnPixels], float v) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  red[wv][lane] = v;
  __syncthreads();
  float s = red[0][lane];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) s += red[k][lane];
  __syncthreads();  // red may be reused
  return s;
}

// LayerNorm scale and shift of the (at most 8 kPer) channels in LDS, so that the per-channel
// reads in the output pass are LDS reads rather than global loads (whose waits would also wait
// for the pass's own stores).  Ordered before use by the barriers of the statistics.
template <int kPer>
struct LnParams {
  float w[kPer > 0 ? kWaves * kPer : 1], b[kPer > 0 ? kWaves * kPer : 1];
};
template <int kPer>
__device__ __forceinline__ void stage_params(const LnArgs& a, LnParams<kPer>& p) {
  if constexpr (kPer > 0) {
    for (int c = threadIdx.x; c < a.C; c += kThreads) {
      p.w[c] = a.w ? a.w[c] : 1.0f;
      p.b[c] = a.b ? a.b[c] : 0.0f;
    }
  }
}

// Shifted sums of the pixel's channels over the wavefronts (each value less the pixel's
// first channel, so that a large mean does not cancel the variance's digits): the mean and
// 1/std.  s1 = sum (m - shift), s2 = sum (m - shift)^2 of this lane's channels.
__device__ __forceinline__ void finish_stats(const LnArgs& a, float (*r1)[kLnPixels], float (*r2)[kLnPixels],
                                             float shift, float s1, float s2, float& mu, float& rstd) {
  s1 = pixel_sum(r1, s1);
  s2 = pixel_sum(r2, s2);
  const float inv = 1.0f / float(a.C);
  const float d = s1 * inv;
  const float var = fmaxf(fmaf(-d, d, s2 * inv), 0.0f);
  mu = shift + d;
  rstd = rsqrtf(var + a.eps);
}

// kPer > 0: the C <= 8 kPer channels of a lane are held in registers between the passes (the
// map is read once); kPer = 0: the map is read again for each pass (wide channel counts).
// Loads are unconditional (channel index clamped, inactive pixels read pixel 0) so that they are
// all in flight together; out-of-range values are masked by selects.
template <typename T, int kPer, bool kZ>
__global__ __launch_bounds__(kThreads) void ln_gate_fwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  __shared__ LnParams<kPer> prm;
  const PixelBlock pb = pixel_block(a);
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const float* m = a.M + pb.base;
  const T* zg = kZ ? static_cast<const T*>(a.z) + pb.base : nullptr;
  const float shift = m[0];
  float s1 = 0.0f, s2 = 0.0f;
  constexpr int kArr = kPer > 0 ? kPer : 1;
  float mv[kArr], zv[kArr] = {};
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i, cc = c < a.C ? c : a.C - 1;
      mv[i] = m[cc * a.L];
      if constexpr (kZ) zv[i] = Elem<T>::load(zg, cc * a.L);  // the gate's loads overlap the statistics
    }
    stage_params<kPer>(a, prm);  // while the loads are in flight
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float v = (wv + int64_t(kWaves) * i < a.C) ? mv[i] - shift : 0.0f;
      s1 += v;
      s2 = fmaf(v, v, s2);
    }
  } else {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves) {
      const float v = m[c * a.L] - shift;
      s1 += v;
      s2 = fmaf(v, v, s2);
    }
  }
  float mu, rstd;
  finish_stats(a, r1, r2, shift, s1, s2, mu, rstd);
  if (!pb.active) return;
  T* og = static_cast<T*>(a.out) + pb.base;
  auto emit = [&](int64_t c, float mval, float zval) {
    float y = (mval - mu) * rstd;
    if constexpr (kPer > 0)
      y = fmaf(y, prm.w[c], prm.b[c]);
    else
      y = fmaf(y, a.w ? a.w[c] : 1.0f, a.b ? a.b[c] : 0.0f);
    if constexpr (kZ) y *= silu(zval);
    Elem<T>::store(og, c * a.L, y);
  };
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i;
      if (c < a.C) emit(c, mv[i], zv[i]);
    }
  } else {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves) emit(c, m[c * a.L], kZ ? Elem<T>::load(zg, c * a.L) : 0.0f);
  }
}

// Sum over the 64 lanes (pixels) of a wavefront, returned wave-uniform: within each row of 16
// lanes by DPP shifts (row_shr 1, 2, 4, 8 with zero fill; lane 15 of the row ends with the row's
// sum), then the four rows' last lanes added in a fixed order.
__device__ __forceinline__ float dpp_shr_add(float v, int ctrl_shift) {
  int src = __builtin_bit_cast(int, v), sh;
  switch (ctrl_shift) {
    case 1: sh = __builtin_amdgcn_update_dpp(0, src, 0x111, 0xF, 0xF, true); break;
    case 2: sh = __builtin_amdgcn_update_dpp(0, src, 0x112, 0xF, 0xF, true); break;
    case 4: sh = __builtin_amdgcn_update_dpp(0, src, 0x114, 0xF, 0xF, true); break;
    default: sh = __builtin_amdgcn_update_dpp(0, src, 0x118, 0xF, 0xF, true); break;
  }
  return v + __builtin_bit_cast(float, sh);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_shr_add(v, 1);
  v = dpp_shr_add(v, 2);
  v = dpp_shr_add(v, 4);
  v = dpp_shr_add(v, 8);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
  return ((r0 + r1) + r2) + r3;
}

// One pass gathers everything the pixel needs: with dy = dout silu(z) (dout without a gate),
// g = dy w, and m' = m - shift, the sums of m', m'^2, g and g m' give the mean, 1/std and the
// two means of the gradient formula (sum g xhat = rstd (sum g m' - (mu - shift) sum g)).
// The second pass writes dM, dz and the per-channel partials of dw and db.
template <typename T, int kPer, bool kZ>
__global__ __launch_bounds__(kThreads) void ln_gate_bwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  __shared__ LnParams<kPer> prm;
  const PixelBlock pb = pixel_block(a);
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave), lane = threadIdx.x % kWave;
  const float* m = a.M + pb.base;
  const T* zg = kZ ? static_cast<const T*>(a.z) + pb.base : nullptr;
  const T* gg = static_cast<const T*>(a.dout) + pb.base;
  auto wt = [&](int64_t c) {
    if constexpr (kPer > 0) return prm.w[c];
    else return a.w ? a.w[c] : 1.0f;
  };
  auto bs = [&](int64_t c) {
    if constexpr (kPer > 0) return prm.b[c];
    else return a.b ? a.b[c] : 0.0f;
  };
  const float shift = m[0];
  float s1 = 0.0f, s2 = 0.0f, sg = 0.0f, sgm = 0.0f;
  constexpr int kArr = kPer > 0 ? kPer : 1;
  float mv[kArr], gv[kArr], zv[kArr] = {};
  auto gather = [&](int64_t c, float mval, float gout, float zval) {
    const float dy = kZ ? gout * silu(zval) : gout;
    const float g = dy * wt(c);
    const float v = mval - shift;
    s1 += v;
    s2 = fmaf(v, v, s2);
    sg += g;
    sgm = fmaf(g, v, sgm);
  };
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i, cc = c < a.C ? c : a.C - 1;
      mv[i] = m[cc * a.L];
      gv[i] = Elem<T>::load(gg, cc * a.L);
      if constexpr (kZ) zv[i] = Elem<T>::load(zg, cc * a.L);
    }
  }
  stage_params<kPer>(a, prm);  // while the loads are in flight
  __syncthreads();
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i;
      if (c < a.C) gather(c, mv[i], gv[i], zv[i]);
    }
  } else {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves)
      gather(c, m[c * a.L], Elem<T>::load(gg, c * a.L), kZ ? Elem<T>::load(zg, c * a.L) : 0.0f);
  }
  float mu, rstd;
  finish_stats(a, r1, r2, shift, s1, s2, mu, rstd);
  const float inv = 1.0f / float(a.C);
  const float tg = pixel_sum(r1, sg), tgm = pixel_sum(r2, sgm);
  const float mg = tg * inv;
  const float mgx = rstd * (tgm - (mu - shift) * tg) * inv;
  float* dmg = a.dM + pb.base;
  T* dzg = kZ ? static_cast<T*>(a.dz) + pb.base : nullptr;
  float* part = a.part + int64_t(blockIdx.x) * 2 * a.C;
  auto emit = [&](int64_t c, float mval, float gout, float zval) {
    const int64_t o = c * a.L;
    float pw = 0.0f, pbias = 0.0f;
    if (pb.active) {
      const float xh = (mval - mu) * rstd;
      float dy = gout;
      if constexpr (kZ) {
        const float sz = sigmoid(zval);
        dy *= zval * sz;
        const float y = fmaf(xh, wt(c), bs(c));
        Elem<T>::store(dzg, o, gout * y * sz * (1.0f + zval * (1.0f - sz)));
      }
      const float g = dy * wt(c);
      dmg[o] = rstd * (g - mg - xh * mgx);
      pw = dy * xh;
      pbias = dy;
    }
    pw = wave_sum(pw);
    pbias = wave_sum(pbias);
    if (lane == 0) {
      part[c] = pw;
      part[a.C + c] = pbias;
    }
  };
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i;
      if (c < a.C) emit(c, mv[i], gv[i], zv[i]);
    }
  } else {
    for (int64_t c = wv; c < a.C; c += kWaves) {
      const bool act = pb.active;
      emit(c, act ? m[c * a.L] : 0.0f, act ? Elem<T>::load(gg, c * a.L) : 0.0f,
           (kZ && act) ? Elem<T>::load(zg, c * a.L) : 0.0f);
    }
  }
}

// dw[c], db[c] (one workgroup per channel): the sum over the backward's workgroups of their
// partials, in a fixed order.
__global__ __launch_bounds__(kThreads) void ln_reduce_kernel(LnArgs a, int64_t rows) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  const int64_t c = blockIdx.x;
  float sw = 0.0f, sb = 0.0f;
  for (int64_t r = threadIdx.x; r < rows; r += kThreads) {
    sw += a.part[r * 2 * a.C + c];
    sb += a.part[r * 2 * a.C + a.C + c];
  }
  sw = wave_sum(sw);
  sb = wave_sum(sb);
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (lane == 0) {
    r1[wv][0] = sw;
    r2[wv][0] = sb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float tw = r1[0][0], tb = r2[0][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      tw += r1[k][0];
      tb += r2[k][0];
    }
    if (a.dw) a.dw[c] = tw;
    if (a.db) a.db[c] = tb;
  }
}

// channels per lane held in registers: up to 32 (C <= 256), else the map is re-read
constexpr int kRegPer = 32;

template <template <typename, int, bool> class K>
hipError_t launch_ln(const LnArgs& a, hipStream_t s) {
  const int64_t blocks = ln_part_rows(a.batch, a.L);
  if (blocks == 0 || a.C == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  const dim3 g{uint32_t(blocks)}, b{kThreads};
  const bool regs = a.C <= int64_t(kWaves) * kRegPer, z = a.z != nullptr;
  if (a.dtype == 0) {
    if (regs) z ? K<float, kRegPer, true>::run(a, g, b, s) : K<float, kRegPer, false>::run(a, g, b, s);
    else z ? K<float, 0, true>::run(a, g, b, s) : K<float, 0, false>::run(a, g, b, s);
  } else {
    if (regs) z ? K<bf16, kRegPer, true>::run(a, g, b, s) : K<bf16, kRegPer, false>::run(a, g, b, s);
    else z ? K<bf16, 0, true>::run(a, g, b, s) : K<bf16, 0, false>::run(a, g, b, s);
  }
  return hipGetLastError();
}

template <typename T, int kPer, bool kZ>
struct FwdK {
  static void run(const LnArgs& a, dim3 g, dim3 b, hipStream_t s) { ln_gate_fwd_kernel<T, kPer, kZ><<<g, b, 0, s>>>(a); }
};
template <typename T, int kPer, bool kZ>
struct BwdK {
  static void run(const LnArgs& a, dim3 g, dim3 b, hipStream_t s) { ln_gate_bwd_kernel<T, kPer, kZ><<<g, b, 0, s>>>(a); }
};

}  // namespace

hipError_t launch_ln_gate_fwd(const LnArgs& a, hipStream_t s) { return launch_ln<FwdK>(a, s); }

hipError_t launch_ln_gate_bwd(const LnArgs& a, hipStream_t s) { return launch_ln<BwdK>(a, s); }

hipError_t launch_ln_reduce(const LnArgs& a, hipStream_t s) {
  if (a.C == 0 || (!a.dw && !a.db)) return hipSuccess;
  if (a.C > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  ln_reduce_kernel<<<dim3(uint32_t(a.C)), dim3(kThreads), 0, s>>>(a, ln_part_rows(a.batch, a.L));
  return hipGetLastError();
}

}  // namespace ss2d
