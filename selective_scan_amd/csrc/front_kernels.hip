// The SS2D input front: depthwise k x k convolution + SiLU before the cross-scan, forward and
// backward (the VSS block's depthwise convolution and activation, SiLU by default, ahead of
// SS2D: "Vision Mamba structure and principle", section 1).
//
// Planes whose halo'd copies fit 64 KB of LDS (every VMamba stage map) take one workgroup per
// (image, channel) plane: the plane is staged once in LDS with a zero halo of r = k/2 pixels and
// every output pixel reads its k x k window from there.  Larger maps go by 32 x 32 tiles, each
// staging its own halo.  The filter size is a template parameter (k = 1, 3, 5, 7), so the taps
// sit in registers and the window loops unroll.
//
// Forward: xc = silu(pre), in fp32, in grid order and, through an LDS transpose, in the
// column-major order of the second and fourth routes (the routes scan it and the merge adds
// its skip term without a rounding to the I/O type in between).
// Backward: pre and dpre = dxc silu'(pre) are recomputed into LDS; dx is the transposed
// convolution of dpre; each plane (or tile) leaves one row of partial sums of the filter and
// bias gradients, which the reduce kernel adds per channel in a fixed order.
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 32, kTy = 8;                                       // tile path
constexpr int kKK = kFrontMaxK * kFrontMaxK, kSlots = kKK + 1;        // partial-sum row
constexpr int kWaves = kThreads / kWave;

// Slot of partial sum e (taps in row-major order, then the bias) in the fixed 7 x 7 + 1 row.
template <int K>
__device__ __forceinline__ int slot_of(int e) {
  return e < K * K ? (e / K) * kFrontMaxK + e % K : kKK;
}

// Walks p = threadIdx.x, + 256, ... over a rows x cols array in row-major order, keeping
// (row, col) of p without a division per step.
struct Walk {
  int row, col, dq, dr, cols;
  __device__ Walk(int cols_) : cols(cols_) {
    row = int(threadIdx.x) / cols;
    col = int(threadIdx.x) - row * cols;
    dq = kThreads / cols;
    dr = kThreads - dq * cols;
  }
  __device__ __forceinline__ void next() {
    row += dq;
    col += dr;
    if (col >= cols) {
      col -= cols;
      ++row;
    }
  }
};

// Zeroes the r-pixel border of an (H + 2r) x (W + 2r) LDS array (row stride ld = W + 2r).
template <int R>
__device__ __forceinline__ void zero_halo(float* s, int H, int W) {
  if constexpr (R > 0) {
    const int ld = W + 2 * R, nrow = 2 * R * ld, n = nrow + 2 * R * H;
    for (int e = threadIdx.x; e < n; e += kThreads) {
      if (e < nrow) {
        const int i = e / ld, j = e - i * ld;
        s[(i < R ? i : H + i) * ld + j] = 0.0f;
      } else {
        const int q = e - nrow, i = q / (2 * R), j = q - i * (2 * R);
        s[(i + R) * ld + (j < R ? j : W + j)] = 0.0f;
      }
    }
  }
}

// Copies an H x W plane into the interior of a halo'd LDS array (pixel (h, w) at
// (h + R) * ld + w + R); vec: H*W % 4 == 0 and the plane 4-element aligned.  The vector path
// issues kBatch loads per thread before writing any of them: loads past the plane read a valid
// address instead and their values go to the spare LDS word `trash`, so that neither the loads
// nor the writes sit behind a branch (a load moved into a conditional block would be waited for
// on its own, one round trip per load).
constexpr int kBatch = 4;
template <int R, typename T>
__device__ __forceinline__ void stage_plane(float* s, float* trash, const T* g, int H, int W, bool vec) {
  const int ld = W + 2 * R, L = H * W;
  if (vec) {
    for (int p0 = 4 * int(threadIdx.x); p0 < L; p0 += 4 * kThreads * kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + 4 * kThreads * u;
        v[u] = Elem<T>::load4(g, p < L ? p : p0);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + 4 * kThreads * u;
        const bool in = p < L;
        const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        int h = in ? p / W : 0, w = in ? p - h * W : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *(in ? s + (h + R) * ld + w + R : trash) = vv[j];
          if (++w == W) {
            w = 0;
            ++h;
          }
        }
      }
    }
  } else {
    Walk pw(W);
    for (int p = threadIdx.x; p < L; p += kThreads, pw.next()) s[(pw.row + R) * ld + pw.col + R] = Elem<T>::load(g, p);
  }
}

template <int K>
__device__ __forceinline__ void load_taps(const FrontArgs& a, int64_t c, float (&wk)[K * K], float& bias) {
#pragma unroll
  for (int e = 0; e < K * K; ++e) wk[e] = a.w[c * (K * K) + e];
  bias = a.bias ? a.bias[c] : 0.0f;
}

// pre-activation at the window whose top-left corner is s[0] (row stride ld)
template <int K>
__device__ __forceinline__ float window(const float* s, int ld, const float (&wk)[K * K], float bias) {
  float pre = bias;
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int j = 0; j < K; ++j) pre = fmaf(wk[i * K + j], s[i * ld + j], pre);
  return pre;
}

// Sums acc[e] over the workgroup: xor shuffles within each wavefront, then the four wavefronts
// in a fixed order; thread e (< N) returns sum e.
template <int N>
__device__ __forceinline__ float block_sum(float (&acc)[N], float (*red)[kSlots]) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    float v = acc[e];
#pragma unroll
    for (int m = kWave / 2; m >= 1; m /= 2) v += __shfl_xor(v, m, kWave);
    if (lane == 0) red[wv][e] = v;
  }
  __syncthreads();
  float s = 0.0f;
  if (int(threadIdx.x) < N) {
    s = red[0][threadIdx.x];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) s += red[k][threadIdx.x];
  }
  return s;
}

// ---- whole-plane kernels ---------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(kThreads) void front_fwd_plane_kernel(FrontArgs a, int vec) {
  constexpr int R = K / 2;
  extern __shared__ float smem[];
  const int H = int(a.H), W = int(a.W), L = H * W, ld = W + 2 * R, ldt = H + 1;
  float* xin = smem;                      // x with the zero halo
  float* tout = smem + (H + 2 * R) * ld;  // the output, pixel (h, w) at w * ldt + h
  float* trash = tout + W * ldt;          // one spare word
  const int64_t plane = blockIdx.x, c = plane % a.C;
  zero_halo<R>(xin, H, W);
  stage_plane<R>(xin, trash, static_cast<const T*>(a.x) + plane * L, H, W, vec != 0);
  float wk[K * K], bias;
  load_taps<K>(a, c, wk, bias);
  __syncthreads();
  float* xc = a.xc + plane * L;
  Walk pw(W);
  for (int p = threadIdx.x; p < L; p += kThreads, pw.next()) {
    const float v = silu(window<K>(xin + pw.row * ld + pw.col, ld, wk, bias));
    xc[p] = v;
    tout[pw.col * ldt + pw.row] = v;
  }
  __syncthreads();
  float* xcT = a.xcT + plane * L;
  if (vec) {
    for (int q = 4 * int(threadIdx.x); q < L; q += 4 * kThreads) {
      int w = q / H, h = q - w * H;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = tout[w * ldt + h];
        if (++h == H) {
          h = 0;
          ++w;
        }
      }
      *reinterpret_cast<float4*>(xcT + q) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    Walk qw(H);  // q = w * H + h: row w, column h
    for (int q = threadIdx.x; q < L; q += kThreads, qw.next()) xcT[q] = tout[qw.row * ldt + qw.col];
  }
}

template <int K, typename T>
__global__ __launch_bounds__(kThreads) void front_bwd_plane_kernel(FrontArgs a, int vec) {
  constexpr int R = K / 2, KK = K * K;
  extern __shared__ float smem[];
  __shared__ float red[kWaves][kSlots];
  const int H = int(a.H), W = int(a.W), L = H * W, ld = W + 2 * R;
  float* xin = smem;                    // x with the zero halo
  float* dp = smem + (H + 2 * R) * ld;  // dpre with the zero halo
  float* trash = dp + (H + 2 * R) * ld; // one spare word
  const int64_t plane = blockIdx.x, c = plane % a.C;
  zero_halo<R>(xin, H, W);
  zero_halo<R>(dp, H, W);
  stage_plane<R>(xin, trash, static_cast<const T*>(a.x) + plane * L, H, W, vec != 0);
  stage_plane<R>(dp, trash, a.dxc + plane * L, H, W, vec != 0);  // dxc first; dpre replaces it in place
  float wk[KK], bias;
  load_taps<K>(a, c, wk, bias);
  __syncthreads();
  {
    Walk pw(W);
    for (int p = threadIdx.x; p < L; p += kThreads, pw.next()) {
      const float pre = window<K>(xin + pw.row * ld + pw.col, ld, wk, bias);
      const float sg = sigmoid(pre);
      float& d = dp[(pw.row + R) * ld + pw.col + R];
      d = d * sg * (1.0f + pre * (1.0f - sg));
    }
  }
  __syncthreads();
  float acc[KK + 1];
#pragma unroll
  for (int e = 0; e <= KK; ++e) acc[e] = 0.0f;
  T* dx = static_cast<T*>(a.dx) + plane * L;
  Walk pw(W);
  for (int p = threadIdx.x; p < L; p += kThreads, pw.next()) {
    // dx[h, w] = sum_{i,j} w[i, j] dpre[h + R - i, w + R - j]
    const float* d0 = dp + (pw.row + 2 * R) * ld + pw.col + 2 * R;
    float g = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) g = fmaf(wk[i * K + j], d0[-(i * ld + j)], g);
    Elem<T>::store(dx, p, g);
    // dw[i, j] += dpre[h, w] x[h + i - R, w + j - R]
    const float dv = dp[(pw.row + R) * ld + pw.col + R];
    const float* x0 = xin + pw.row * ld + pw.col;
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) acc[i * K + j] = fmaf(dv, x0[i * ld + j], acc[i * K + j]);
    acc[KK] += dv;
  }
  const float s = block_sum<KK + 1>(acc, red);
  if (int(threadIdx.x) <= KK) a.part[plane * kSlots + slot_of<K>(threadIdx.x)] = s;
}

// ---- 32 x 32 tile kernels (maps too large for one workgroup's LDS) ---------------------------

struct Tile {
  int64_t plane, c, t;  // (image, channel) plane, channel, tile index within the plane
  int h0, w0;
};

__device__ __forceinline__ Tile front_tile(const FrontArgs& a) {
  const int tw = int((a.W + kT - 1) / kT), th = int((a.H + kT - 1) / kT);
  const int64_t bid = blockIdx.x, per = int64_t(tw) * th;
  Tile t;
  t.t = bid % per;
  t.h0 = int(t.t / tw) * kT;
  t.w0 = int(t.t % tw) * kT;
  t.plane = bid / per;
  t.c = t.plane % a.C;
  return t;
}

// x of the tile with a halo of `halo` pixels (zero outside the map), row stride kT + 2 halo + 1
template <typename T>
__device__ __forceinline__ void stage_tile(float* s, const T* g, int H, int W, int h0, int w0, int halo) {
  const int span = kT + 2 * halo, ld = span + 1;
  for (int e = threadIdx.x; e < span * span; e += kThreads) {
    const int i = e / span, j = e - i * span, h = h0 - halo + i, w = w0 - halo + j;
    s[i * ld + j] = (h >= 0 && h < H && w >= 0 && w < W) ? Elem<T>::load(g, int64_t(h) * W + w) : 0.0f;
  }
}

template <int K, typename T>
__global__ __launch_bounds__(kThreads) void front_fwd_tile_kernel(FrontArgs a) {
  constexpr int R = K / 2, ld = kT + 2 * R + 1;
  __shared__ float xin[(kT + 2 * R) * ld];
  __shared__ float tout[kT][kT + 1];
  const Tile tl = front_tile(a);
  const int H = int(a.H), W = int(a.W);
  const int64_t base = tl.plane * a.H * a.W;
  stage_tile(xin, static_cast<const T*>(a.x) + base, H, W, tl.h0, tl.w0, R);
  float wk[K * K], bias;
  load_taps<K>(a, tl.c, wk, bias);
  __syncthreads();
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  float* xc = a.xc + base;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int hh = ty + kTy * rr, h = tl.h0 + hh, w = tl.w0 + tx;
    const float v = silu(window<K>(xin + hh * ld + tx, ld, wk, bias));
    if (h < H && w < W) {
      xc[int64_t(h) * W + w] = v;
      tout[hh][tx] = v;
    }
  }
  __syncthreads();
  float* xcT = a.xcT + base;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int ww = ty + kTy * rr, w = tl.w0 + ww, h = tl.h0 + tx;
    if (h < H && w < W) xcT[int64_t(w) * H + h] = tout[tx][ww];
  }
}

template <int K, typename T>
__global__ __launch_bounds__(kThreads) void front_bwd_tile_kernel(FrontArgs a) {
  constexpr int R = K / 2, KK = K * K, ldx = kT + 4 * R + 1, ldd = kT + 2 * R + 1;
  __shared__ float xin[(kT + 4 * R) * ldx];  // x, halo 2R
  __shared__ float dp[(kT + 2 * R) * ldd];   // dpre, halo R
  __shared__ float red[kWaves][kSlots];
  const Tile tl = front_tile(a);
  const int H = int(a.H), W = int(a.W);
  const int64_t base = tl.plane * a.H * a.W;
  stage_tile(xin, static_cast<const T*>(a.x) + base, H, W, tl.h0, tl.w0, 2 * R);
  float wk[KK], bias;
  load_taps<K>(a, tl.c, wk, bias);
  __syncthreads();
  const float* dxc = a.dxc + base;
  constexpr int sd = kT + 2 * R;
  for (int e = threadIdx.x; e < sd * sd; e += kThreads) {
    const int i = e / sd, j = e - i * sd, h = tl.h0 - R + i, w = tl.w0 - R + j;
    float d = 0.0f;
    if (h >= 0 && h < H && w >= 0 && w < W) {
      const float pre = window<K>(xin + i * ldx + j, ldx, wk, bias);
      const float sg = sigmoid(pre);
      d = dxc[int64_t(h) * W + w] * sg * (1.0f + pre * (1.0f - sg));
    }
    dp[i * ldd + j] = d;
  }
  __syncthreads();
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  float acc[KK + 1];
#pragma unroll
  for (int e = 0; e <= KK; ++e) acc[e] = 0.0f;
  T* dx = static_cast<T*>(a.dx) + base;
#pragma unroll
  for (int rr = 0; rr < kT / kTy; ++rr) {
    const int hh = ty + kTy * rr, h = tl.h0 + hh, w = tl.w0 + tx;
    if (h < H && w < W) {
      const float* d0 = dp + (hh + 2 * R) * ldd + tx + 2 * R;
      float g = 0.0f;
#pragma unroll
      for (int i = 0; i < K; ++i)
#pragma unroll
        for (int j = 0; j < K; ++j) g = fmaf(wk[i * K + j], d0[-(i * ldd + j)], g);
      Elem<T>::store(dx, int64_t(h) * W + w, g);
      const float dv = dp[(hh + R) * ldd + tx + R];
      const float* x0 = xin + (hh + R) * ldx + tx + R;
#pragma unroll
      for (int i = 0; i < K; ++i)
#pragma unroll
        for (int j = 0; j < K; ++j) acc[i * K + j] = fmaf(dv, x0[i * ldx + j], acc[i * K + j]);
      acc[KK] += dv;
    }
  }
  const float s = block_sum<KK + 1>(acc, red);
  if (int(threadIdx.x) <= KK) a.part[(tl.plane * front_tiles(a.H, a.W) + tl.t) * kSlots + slot_of<K>(threadIdx.x)] = s;
}

// dw[c, :, :] and dbias[c] (one workgroup per channel): the sum over images and partial-sum
// rows of the backward's partials, in a fixed order.
template <int K>
__global__ __launch_bounds__(kThreads) void front_reduce_kernel(FrontArgs a, int64_t rows) {
  constexpr int KK = K * K;
  __shared__ float red[kWaves][kSlots];
  const int64_t c = blockIdx.x, n = a.batch * rows;
  float acc[KK + 1];
#pragma unroll
  for (int e = 0; e <= KK; ++e) acc[e] = 0.0f;
  for (int64_t q = threadIdx.x; q < n; q += kThreads) {
    const int64_t b = q / rows, t = q - b * rows;
    const float* src = a.part + ((b * a.C + c) * rows + t) * kSlots;
#pragma unroll
    for (int e = 0; e <= KK; ++e) acc[e] += src[slot_of<K>(e)];
  }
  const float s = block_sum<KK + 1>(acc, red);
  const int e = threadIdx.x;
  if (e < KK)
    a.dw[c * KK + e] = s;
  else if (e == KK && a.dbias)
    a.dbias[c] = s;
}

// 4-element vector access: whole planes of a multiple of 4 pixels, x aligned for its type,
// the fp32 arrays (the forward's outputs, the backward's dxc) to 16 bytes
bool vec_plane(const FrontArgs& a, bool forward) {
  if ((a.H * a.W) % 4 != 0) return false;
  if (reinterpret_cast<uintptr_t>(a.x) & (a.dtype == 0 ? 15 : 7)) return false;
  const uintptr_t f32 = forward ? (reinterpret_cast<uintptr_t>(a.xc) | reinterpret_cast<uintptr_t>(a.xcT))
                                : reinterpret_cast<uintptr_t>(a.dxc);
  return (f32 & 15) == 0;
}

template <int K, typename T>
hipError_t fwd_k(const FrontArgs& a, hipStream_t s) {
  if (front_plane_path(a.H, a.W, K)) {
    const int64_t blocks = a.batch * a.C;
    if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
    const size_t lds = size_t(((a.H + K - 1) * (a.W + K - 1) + a.W * (a.H + 1) + 1) * 4);
    front_fwd_plane_kernel<K, T><<<dim3(uint32_t(blocks)), dim3(kThreads), lds, s>>>(
        a, vec_plane(a, true) ? 1 : 0);
  } else {
    const int64_t blocks = a.batch * a.C * front_tiles(a.H, a.W);
    if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
    front_fwd_tile_kernel<K, T><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int K, typename T>
hipError_t bwd_k(const FrontArgs& a, hipStream_t s) {
  if (front_plane_path(a.H, a.W, K)) {
    const int64_t blocks = a.batch * a.C;
    if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
    const size_t lds = size_t((2 * (a.H + K - 1) * (a.W + K - 1) + 1) * 4);
    front_bwd_plane_kernel<K, T><<<dim3(uint32_t(blocks)), dim3(kThreads), lds, s>>>(a, vec_plane(a, false) ? 1 : 0);
  } else {
    const int64_t blocks = a.batch * a.C * front_tiles(a.H, a.W);
    if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
    front_bwd_tile_kernel<K, T><<<dim3(uint32_t(blocks)), dim3(kThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

template <template <int, typename> class F>
hipError_t dispatch(const FrontArgs& a, hipStream_t s) {
  const bool f32 = a.dtype == 0;
  switch (a.k) {
    case 1: return f32 ? F<1, float>::run(a, s) : F<1, bf16>::run(a, s);
    case 3: return f32 ? F<3, float>::run(a, s) : F<3, bf16>::run(a, s);
    case 5: return f32 ? F<5, float>::run(a, s) : F<5, bf16>::run(a, s);
    case 7: return f32 ? F<7, float>::run(a, s) : F<7, bf16>::run(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int K, typename T>
struct FwdOp {
  static hipError_t run(const FrontArgs& a, hipStream_t s) { return fwd_k<K, T>(a, s); }
};
template <int K, typename T>
struct BwdOp {
  static hipError_t run(const FrontArgs& a, hipStream_t s) { return bwd_k<K, T>(a, s); }
};

}  // namespace

hipError_t launch_front_fwd(const FrontArgs& a, hipStream_t s) {
  if (a.batch * a.C * a.H * a.W == 0) return hipSuccess;
  return dispatch<FwdOp>(a, s);
}

hipError_t launch_front_bwd(const FrontArgs& a, hipStream_t s) {
  if (a.batch * a.C * a.H * a.W == 0) return hipSuccess;
  return dispatch<BwdOp>(a, s);
}

hipError_t launch_front_reduce(const FrontArgs& a, hipStream_t s) {
  if (a.C == 0) return hipSuccess;
  if (a.C > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  const int64_t rows = front_part_rows(a.H, a.W, a.k);
  const dim3 g{uint32_t(a.C)}, b{kThreads};
  switch (a.k) {
    case 1: front_reduce_kernel<1><<<g, b, 0, s>>>(a, rows); break;
    case 3: front_reduce_kernel<3><<<g, b, 0, s>>>(a, rows); break;
    case 5: front_reduce_kernel<5><<<g, b, 0, s>>>(a, rows); break;
    case 7: front_reduce_kernel<7><<<g, b, 0, s>>>(a, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ss2d
