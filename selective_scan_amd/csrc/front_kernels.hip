// The SS2D input front: depthwise k x k convolution + SiLU before the cross-scan, forward and
// backward (the VSS block's "depthwise convolution and activation, SiLU by default", ahead of
// SS2D, on the "Vision Mamba structure and principle" page, section 1).
//
// 32 x 32 output tiles of one (b, c) plane per workgroup (256 threads, four passes of 8 rows).
// The forward stages the input tile with an r-pixel halo in LDS and writes the result in grid
// order and, through an LDS transpose, in the column-major route order.  The backward stages x
// with a 2r halo, recomputes pre and dpre = dxc silu'(pre) on the tile plus an r halo, and from
// those forms dx and the tile's partial sums of the filter and bias gradients.
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

constexpr int kT = 32, kTy = 8, kR = kFrontMaxK / 2;

struct Tile {
  int64_t b, c, t;  // image, channel, tile index within the plane
  int h0, w0;
};

__device__ __forceinline__ Tile front_tile(const FrontArgs& a) {
  const int tw = int((a.W + kT - 1) / kT), th = int((a.H + kT - 1) / kT);
  int64_t bid = blockIdx.x;
  Tile t;
  t.t = bid % (int64_t(tw) * th);
  t.h0 = int(t.t / tw) * kT;
  t.w0 = int(t.t % tw) * kT;
  bid /= int64_t(tw) * th;
  t.c = bid % a.C;
  t.b = bid / a.C;
  return t;
}

template <typename T>
__global__ __launch_bounds__(256) void front_fwd_kernel(FrontArgs a) {
  __shared__ float xin[kT + 2 * kR][kT + 2 * kR + 1];
  __shared__ float tout[kT][kT + 1];
  __shared__ float wk[kFrontMaxK * kFrontMaxK];
  const Tile tl = front_tile(a);
  const int H = int(a.H), W = int(a.W), k = a.k, r = k / 2, span = kT + 2 * r;
  const int64_t plane = (tl.b * a.C + tl.c) * a.H * a.W;
  const T* xg = static_cast<const T*>(a.x) + plane;
  for (int e = threadIdx.x; e < span * span; e += 256) {
    const int i = e / span, j = e % span, h = tl.h0 - r + i, w = tl.w0 - r + j;
    xin[i][j] = (h >= 0 && h < H && w >= 0 && w < W) ? Elem<T>::load(xg, int64_t(h) * W + w) : 0.0f;
  }
  if (int(threadIdx.x) < k * k) wk[threadIdx.x] = a.w[tl.c * k * k + threadIdx.x];
  const float bias = a.bias ? a.bias[tl.c] : 0.0f;
  __syncthreads();
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  T* xc = static_cast<T*>(a.xc) + plane;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int hh = ty + kTy * rr, h = tl.h0 + hh, w = tl.w0 + tx;
    float pre = bias;
    for (int i = 0; i < k; ++i)
      for (int j = 0; j < k; ++j) pre = fmaf(wk[i * k + j], xin[hh + i][tx + j], pre);
    const float v = silu(pre);
    if (h < H && w < W) {
      Elem<T>::store(xc, int64_t(h) * W + w, v);
      tout[hh][tx] = Elem<T>::load(xc, int64_t(h) * W + w);  // the stored (rounded) value
    }
  }
  __syncthreads();
  T* xcT = static_cast<T*>(a.xcT) + plane;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int ww = ty + kTy * rr, w = tl.w0 + ww, h = tl.h0 + tx;
    if (h < H && w < W) Elem<T>::store(xcT, int64_t(w) * H + h, tout[tx][ww]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void front_bwd_kernel(FrontArgs a) {
  __shared__ float xin[kT + 4 * kR][kT + 4 * kR + 1];  // x, halo 2r
  __shared__ float dp[kT + 2 * kR][kT + 2 * kR + 1];   // dpre, halo r
  __shared__ float wk[kFrontMaxK * kFrontMaxK];
  __shared__ float red[4][kFrontMaxK * kFrontMaxK + 1];  // per wavefront
  const Tile tl = front_tile(a);
  const int H = int(a.H), W = int(a.W), k = a.k, r = k / 2, kk = k * k;
  const int64_t plane = (tl.b * a.C + tl.c) * a.H * a.W;
  const T* xg = static_cast<const T*>(a.x) + plane;
  const int sx = kT + 4 * r, sd = kT + 2 * r;
  constexpr int kKK = kFrontMaxK * kFrontMaxK;  // partial-sum slots: filter taps (row stride 7), then the bias
  for (int e = threadIdx.x; e < sx * sx; e += 256) {
    const int i = e / sx, j = e % sx, h = tl.h0 - 2 * r + i, w = tl.w0 - 2 * r + j;
    xin[i][j] = (h >= 0 && h < H && w >= 0 && w < W) ? Elem<T>::load(xg, int64_t(h) * W + w) : 0.0f;
  }
  if (int(threadIdx.x) < kk) wk[threadIdx.x] = a.w[tl.c * kk + threadIdx.x];
  const float bias = a.bias ? a.bias[tl.c] : 0.0f;
  __syncthreads();
  const float* dxc = a.dxc + plane;
  for (int e = threadIdx.x; e < sd * sd; e += 256) {
    const int i = e / sd, j = e % sd, h = tl.h0 - r + i, w = tl.w0 - r + j;
    float d = 0.0f;
    if (h >= 0 && h < H && w >= 0 && w < W) {
      float pre = bias;
      for (int ii = 0; ii < k; ++ii)
        for (int jj = 0; jj < k; ++jj) pre = fmaf(wk[ii * k + jj], xin[i + ii][j + jj], pre);
      const float sg = sigmoid(pre);
      d = dxc[int64_t(h) * W + w] * sg * (1.0f + pre * (1.0f - sg));
    }
    dp[i][j] = d;
  }
  __syncthreads();
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  float acc[kFrontMaxK * kFrontMaxK + 1];
#pragma unroll
  for (int e = 0; e <= kFrontMaxK * kFrontMaxK; ++e) acc[e] = 0.0f;
  T* dx = static_cast<T*>(a.dx) + plane;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int hh = ty + kTy * rr, h = tl.h0 + hh, w = tl.w0 + tx;
    if (h < H && w < W) {
      float g = 0.0f;
      for (int i = 0; i < k; ++i)
        for (int j = 0; j < k; ++j) g = fmaf(wk[i * k + j], dp[hh + 2 * r - i][tx + 2 * r - j], g);
      Elem<T>::store(dx, int64_t(h) * W + w, g);
      const float dv = dp[hh + r][tx + r];
#pragma unroll
      for (int i = 0; i < kFrontMaxK; ++i)
#pragma unroll
        for (int j = 0; j < kFrontMaxK; ++j)
          if (i < k && j < k) acc[i * kFrontMaxK + j] = fmaf(dv, xin[hh + r + i][tx + r + j], acc[i * kFrontMaxK + j]);
      acc[kKK] += dv;
    }
  }
  // tile sums (fixed 7 x 7 + 1 layout): over each wavefront by xor shuffles, then over the four
  // wavefronts in LDS
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
#pragma unroll
  for (int e = 0; e <= kKK; ++e) {
    const int i = e / kFrontMaxK, j = e % kFrontMaxK;
    if (e < kKK && (i >= k || j >= k)) continue;
    float v = acc[e];
#pragma unroll
    for (int m = kWave / 2; m >= 1; m /= 2) v += __shfl_xor(v, m, kWave);
    if (lane == 0) red[wv][e] = v;
  }
  __syncthreads();
  if (int(threadIdx.x) <= kKK) {
    const int e = threadIdx.x, i = e / kFrontMaxK, j = e % kFrontMaxK;
    if (e == kKK || (i < k && j < k)) {
      const float v = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
      a.part[((tl.b * a.C + tl.c) * front_tiles(a.H, a.W) + tl.t) * (kKK + 1) + e] = v;
    }
  }
}

// dw[c, i, j] and dbias[c]: sums over images and tiles, in that order, of the tile partials
// (slot i * 7 + j for tap (i, j), slot 49 for the bias)
__global__ __launch_bounds__(256) void front_reduce_kernel(FrontArgs a) {
  constexpr int kKK = kFrontMaxK * kFrontMaxK;
  const int kk = a.k * a.k;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= a.C * (kk + 1)) return;
  const int64_t c = idx / (kk + 1);
  const int e = int(idx % (kk + 1));
  const int slot = e < kk ? (e / a.k) * kFrontMaxK + e % a.k : kKK;
  const int64_t tiles = front_tiles(a.H, a.W);
  float s = 0.0f;
  for (int64_t b = 0; b < a.batch; ++b)
    for (int64_t t = 0; t < tiles; ++t) s += a.part[((b * a.C + c) * tiles + t) * (kKK + 1) + slot];
  if (e < kk)
    a.dw[c * kk + e] = s;
  else if (a.dbias)
    a.dbias[c] = s;
}

}  // namespace

hipError_t launch_front_fwd(const FrontArgs& a, hipStream_t s) {
  const int64_t blocks = a.batch * a.C * front_tiles(a.H, a.W);
  if (blocks == 0) return hipSuccess;
  if (a.dtype == 0)
    front_fwd_kernel<float><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a);
  else
    front_fwd_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_front_bwd(const FrontArgs& a, hipStream_t s) {
  const int64_t blocks = a.batch * a.C * front_tiles(a.H, a.W);
  if (blocks == 0) return hipSuccess;
  if (a.dtype == 0)
    front_bwd_kernel<float><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a);
  else
    front_bwd_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_front_reduce(const FrontArgs& a, hipStream_t s) {
  const int64_t n = a.C * (int64_t(a.k) * a.k + 1);
  if (n == 0) return hipSuccess;
  front_reduce_kernel<<<dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ss2d
