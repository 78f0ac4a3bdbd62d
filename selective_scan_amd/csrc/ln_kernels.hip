// The VSS block's back half after the SS2D merge: LayerNorm over the channels of each pixel,
// then the gate (the VSS block description in "Vision Mamba structure and principle",
// section 1: the SS2D features are layer-normalised and multiplied by the other branch, whose
// activation is SiLU).  Forward and backward; all arithmetic in fp32 on the fp32 merged map,
// one rounding to the I/O type at the end.
//
// A workgroup takes 64 consecutive pixels of one image, one per lane, and four wavefronts that
// split the channels (channel c goes to wavefront c % 4): every load of a channel's 64 pixels
// is one contiguous 256-byte segment.  The per-pixel statistics are summed over the four
// wavefronts in LDS.  The mean and variance use sums shifted by the pixel's first channel, so
// that a large mean does not cancel the variance's digits; the map is then read a second time
// (from L2) for the outputs.
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

constexpr int kThreads = 256;
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

// Adds the four wavefronts' values of this lane's pixel in a fixed order.
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

// Mean and 1/std of the pixel's channels.
__device__ __forceinline__ void pixel_stats(const LnArgs& a, const PixelBlock& pb, float (*r1)[kLnPixels],
                                            float (*r2)[kLnPixels], float& mu, float& rstd) {
  const float* m = a.M + pb.base;
  const int wv = threadIdx.x / kWave;
  const float shift = pb.active ? m[0] : 0.0f;
  float s1 = 0.0f, s2 = 0.0f;
  if (pb.active) {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves) {
      const float v = m[c * a.L] - shift;
      s1 += v;
      s2 = fmaf(v, v, s2);
    }
  }
  const int lane = threadIdx.x % kWave;
  r1[wv][lane] = s1;
  r2[wv][lane] = s2;
  __syncthreads();
  s1 = r1[0][lane];
  s2 = r2[0][lane];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    s1 += r1[k][lane];
    s2 += r2[k][lane];
  }
  __syncthreads();
  const float inv = 1.0f / float(a.C);
  const float d = s1 * inv;
  const float var = fmaxf(fmaf(-d, d, s2 * inv), 0.0f);
  mu = shift + d;
  rstd = rsqrtf(var + a.eps);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void ln_gate_fwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  const PixelBlock pb = pixel_block(a);
  float mu, rstd;
  pixel_stats(a, pb, r1, r2, mu, rstd);
  if (!pb.active) return;
  const float* m = a.M + pb.base;
  const T* zg = a.z ? static_cast<const T*>(a.z) + pb.base : nullptr;
  T* og = static_cast<T*>(a.out) + pb.base;
#pragma unroll 4
  for (int64_t c = threadIdx.x / kWave; c < a.C; c += kWaves) {
    const int64_t o = c * a.L;
    float y = (m[o] - mu) * rstd;
    y = fmaf(y, a.w ? a.w[c] : 1.0f, a.b ? a.b[c] : 0.0f);
    if (zg) y *= silu(Elem<T>::load(zg, o));
    Elem<T>::store(og, o, y);
  }
}

// Sum over the 64 lanes (pixels) of a wavefront; every lane receives it.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m /= 2) v += __shfl_xor(v, m, kWave);
  return v;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void ln_gate_bwd_kernel(LnArgs a) {
  __shared__ float r1[kWaves][kLnPixels], r2[kWaves][kLnPixels];
  const PixelBlock pb = pixel_block(a);
  float mu, rstd;
  pixel_stats(a, pb, r1, r2, mu, rstd);
  const float* m = a.M + pb.base;
  const T* zg = a.z ? static_cast<const T*>(a.z) + pb.base : nullptr;
  const T* gg = static_cast<const T*>(a.dout) + pb.base;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  // dy = dout * silu(z) (dout without a gate), g = dy * w: the pixel's mean of g and of g * xhat
  float sg = 0.0f, sgx = 0.0f;
  if (pb.active) {
#pragma unroll 4
    for (int64_t c = wv; c < a.C; c += kWaves) {
      const int64_t o = c * a.L;
      const float xh = (m[o] - mu) * rstd;
      float dy = Elem<T>::load(gg, o);
      if (zg) dy *= silu(Elem<T>::load(zg, o));
      const float g = dy * (a.w ? a.w[c] : 1.0f);
      sg += g;
      sgx = fmaf(g, xh, sgx);
    }
  }
  const float inv = 1.0f / float(a.C);
  const float mg = pixel_sum(r1, sg) * inv, mgx = pixel_sum(r2, sgx) * inv;
  float* dmg = a.dM + pb.base;
  T* dzg = a.z ? static_cast<T*>(a.dz) + pb.base : nullptr;
  float* part = a.part + int64_t(blockIdx.x) * 2 * a.C;
  for (int64_t c = wv; c < a.C; c += kWaves) {
    const int64_t o = c * a.L;
    float pw = 0.0f, pbias = 0.0f;
    if (pb.active) {
      const float xh = (m[o] - mu) * rstd;
      const float gout = Elem<T>::load(gg, o);
      float dy = gout;
      if (zg) {
        const float zv = Elem<T>::load(zg, o), sz = sigmoid(zv);
        dy *= zv * sz;
        const float y = fmaf(xh, a.w ? a.w[c] : 1.0f, a.b ? a.b[c] : 0.0f);
        Elem<T>::store(dzg, o, gout * y * sz * (1.0f + zv * (1.0f - sz)));
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

}  // namespace

hipError_t launch_ln_gate_fwd(const LnArgs& a, hipStream_t s) {
  const int64_t blocks = ln_part_rows(a.batch, a.L);
  if (blocks == 0 || a.C == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  if (a.dtype == 0)
    ln_gate_fwd_kernel<float><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  else
    ln_gate_fwd_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ln_gate_bwd(const LnArgs& a, hipStream_t s) {
  const int64_t blocks = ln_part_rows(a.batch, a.L);
  if (blocks == 0 || a.C == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  if (a.dtype == 0)
    ln_gate_bwd_kernel<float><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  else
    ln_gate_bwd_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ln_reduce(const LnArgs& a, hipStream_t s) {
  if (a.C == 0 || (!a.dw && !a.db)) return hipSuccess;
  if (a.C > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  ln_reduce_kernel<<<dim3(uint32_t(a.C)), dim3(kThreads), 0, s>>>(a, ln_part_rows(a.batch, a.L));
  return hipGetLastError();
}

}  // namespace ss2d
