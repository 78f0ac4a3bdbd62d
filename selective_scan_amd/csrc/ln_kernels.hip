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
template <typename T, int kPer>
__global__ __launch_bounds__(kThreads) void ln_gate_fwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  const PixelBlock pb = pixel_block(a);
  const int wv = threadIdx.x / kWave;
  const float* m = a.M + pb.base;
  const float shift = pb.active ? m[0] : 0.0f;
  float s1 = 0.0f, s2 = 0.0f;
  float mv[kPer > 0 ? kPer : 1];
  if (pb.active) {
    if constexpr (kPer > 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t c = wv + int64_t(kWaves) * i;
        mv[i] = c < a.C ? m[c * a.L] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (wv + int64_t(kWaves) * i < a.C) {
          const float v = mv[i] - shift;
          s1 += v;
          s2 = fmaf(v, v, s2);
        }
      }
    } else {
#pragma unroll 4
      for (int64_t c = wv; c < a.C; c += kWaves) {
        const float v = m[c * a.L] - shift;
        s1 += v;
        s2 = fmaf(v, v, s2);
      }
    }
  }
  float mu, rstd;
  finish_stats(a, r1, r2, shift, s1, s2, mu, rstd);
  if (!pb.active) return;
  const T* zg = a.z ? static_cast<const T*>(a.z) + pb.base : nullptr;
  T* og = static_cast<T*>(a.out) + pb.base;
  auto emit = [&](int64_t c, float mval) {
    const int64_t o = c * a.L;
    float y = (mval - mu) * rstd;
    y = fmaf(y, a.w ? a.w[c] : 1.0f, a.b ? a.b[c] : 0.0f);
    if (zg) y *= silu(Elem<T>::load(zg, o));
    Elem<T>::store(og, o, y);
  };
  if constexpr (kPer > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t c = wv + int64_t(kWaves) * i;
      if (c < a.C) emit(c, mv[i]);
    }
  } else {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves) emit(c, m[c * a.L]);
  }
}

// Sum over the 64 lanes (pixels) of a wavefront; every lane receives it.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m /= 2) v += __shfl_xor(v, m, kWave);
  return v;
}

// One pass gathers everything the pixel needs: with dy = dout silu(z) (dout without a gate),
// g = dy w, and m' = m - shift, the sums of m', m'^2, g and g m' give the mean, 1/std and the
// two means of the gradient formula (sum g xhat = rstd (sum g m' - (mu - shift) sum g)).
// The second pass writes dM, dz and the per-channel partials of dw and db.
template <typename T, int kPer>
__global__ __launch_bounds__(kThreads) void ln_gate_bwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  const PixelBlock pb = pixel_block(a);
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const float* m = a.M + pb.base;
  const T* zg = a.z ? static_cast<const T*>(a.z) + pb.base : nullptr;
  const T* gg = static_cast<const T*>(a.dout) + pb.base;
  const float shift = pb.active ? m[0] : 0.0f;
  float s1 = 0.0f, s2 = 0.0f, sg = 0.0f, sgm = 0.0f;
  constexpr int kArr = kPer > 0 ? kPer : 1;
  float mv[kArr], gv[kArr], zv[kArr];
  auto gather = [&](int64_t c, float mval, float gout, float zval) {
    const float dy = zg ? gout * silu(zval) : gout;
    const float g = dy * (a.w ? a.w[c] : 1.0f);
    const float v = mval - shift;
    s1 += v;
    s2 = fmaf(v, v, s2);
    sg += g;
    sgm = fmaf(g, v, sgm);
  };
  if (pb.active) {
    if constexpr (kPer > 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t c = wv + int64_t(kWaves) * i;
        const bool in = c < a.C;
        mv[i] = in ? m[c * a.L] : 0.0f;
        gv[i] = in ? Elem<T>::load(gg, c * a.L) : 0.0f;
        zv[i] = (in && zg) ? Elem<T>::load(zg, c * a.L) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t c = wv + int64_t(kWaves) * i;
        if (c < a.C) gather(c, mv[i], gv[i], zv[i]);
      }
    } else {
#pragma unroll 4
      for (int64_t c = wv; c < a.C; c += kWaves)
        gather(c, m[c * a.L], Elem<T>::load(gg, c * a.L), zg ? Elem<T>::load(zg, c * a.L) : 0.0f);
    }
  }
  float mu, rstd;
  finish_stats(a, r1, r2, shift, s1, s2, mu, rstd);
  const float inv = 1.0f / float(a.C);
  const float tg = pixel_sum(r1, sg), tgm = pixel_sum(r2, sgm);
  const float mg = tg * inv;
  const float mgx = rstd * (tgm - (mu - shift) * tg) * inv;
  float* dmg = a.dM + pb.base;
  T* dzg = a.z ? static_cast<T*>(a.dz) + pb.base : nullptr;
  float* part = a.part + int64_t(blockIdx.x) * 2 * a.C;
  auto emit = [&](int64_t c, float mval, float gout, float zval) {
    const int64_t o = c * a.L;
    float pw = 0.0f, pbias = 0.0f;
    if (pb.active) {
      const float xh = (mval - mu) * rstd;
      float dy = gout;
      if (zg) {
        const float sz = sigmoid(zval);
        dy *= zval * sz;
        const float y = fmaf(xh, a.w ? a.w[c] : 1.0f, a.b ? a.b[c] : 0.0f);
        Elem<T>::store(dzg, o, gout * y * sz * (1.0f + zval * (1.0f - sz)));
      }
      const float g = dy * (a.w ? a.w[c] : 1.0f);
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
           (act && zg) ? Elem<T>::load(zg, c * a.L) : 0.0f);
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

template <template <typename, int> class K>
hipError_t launch_ln(const LnArgs& a, hipStream_t s) {
  const int64_t blocks = ln_part_rows(a.batch, a.L);
  if (blocks == 0 || a.C == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  const dim3 g{uint32_t(blocks)}, b{kThreads};
  const bool regs = a.C <= int64_t(kWaves) * kRegPer;
  if (a.dtype == 0)
    regs ? K<float, kRegPer>::run(a, g, b, s) : K<float, 0>::run(a, g, b, s);
  else
    regs ? K<bf16, kRegPer>::run(a, g, b, s) : K<bf16, 0>::run(a, g, b, s);
  return hipGetLastError();
}

template <typename T, int kPer>
struct FwdK {
  static void run(const LnArgs& a, dim3 g, dim3 b, hipStream_t s) { ln_gate_fwd_kernel<T, kPer><<<g, b, 0, s>>>(a); }
};
template <typename T, int kPer>
struct BwdK {
  static void run(const LnArgs& a, dim3 g, dim3 b, hipStream_t s) { ln_gate_bwd_kernel<T, kPer><<<g, b, 0, s>>>(a); }
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
