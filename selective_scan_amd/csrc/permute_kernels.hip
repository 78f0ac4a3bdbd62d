// Route permutations of SS2D: cross-scan (map -> four route orders), cross-merge (four route
// orders -> map, summed in fp32), and the per-pixel gate of the merged map (forward and
// backward).  Routes, after the SS2D section of the VMamba paper (Fig. 2): k = 0 row-major,
// k = 1 column-major, k = 2 / 3 the same traversals from the last pixel back to the first.
//
// Each workgroup owns a 32 x 32 pixel tile of one (b, c) plane.  Row-major routes are read and
// written along w; column-major routes along h, through a padded LDS tile so that both the
// global reads and the global writes stay contiguous.
#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

constexpr int kT = 32;   // tile edge (pixels)
constexpr int kTy = 8;   // rows of threads: 256 threads = 32 x 8, four passes of 8 rows

struct TileCoord {
  int64_t b, c;
  int h0, w0;
};

__device__ __forceinline__ TileCoord tile_coord(int64_t C, int tiles_h, int tiles_w) {
  int64_t bid = blockIdx.x;
  TileCoord t;
  const int tw = int(bid % tiles_w);
  bid /= tiles_w;
  const int th = int(bid % tiles_h);
  bid /= tiles_h;
  t.c = bid % C;
  t.b = bid / C;
  t.h0 = th * kT;
  t.w0 = tw * kT;
  return t;
}

template <typename W>
__global__ __launch_bounds__(256) void route_scatter_kernel(const W* __restrict__ x, ScanOutputs o, int64_t C,
                                                            int H, int Wd, int tiles_h, int tiles_w) {
  __shared__ W tile[kT][kT + 1];
  const TileCoord tc = tile_coord(C, tiles_h, tiles_w);
  const int64_t L = int64_t(H) * Wd;
  const W* xp = x + (tc.b * C + tc.c) * L;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
#pragma unroll
  for (int r = 0; r < kT / kTy; ++r) {
    const int h = tc.h0 + ty + kTy * r, w = tc.w0 + tx;
    if (h < H && w < Wd) tile[ty + kTy * r][tx] = xp[int64_t(h) * Wd + w];
  }
  __syncthreads();
  const int64_t off = tc.b * o.batch_stride + tc.c * L;
  W* o0 = static_cast<W*>(o.out[0]);
  W* o1 = static_cast<W*>(o.out[1]);
  W* o2 = static_cast<W*>(o.out[2]);
  W* o3 = static_cast<W*>(o.out[3]);
  if (o0 || o2) {
#pragma unroll
    for (int r = 0; r < kT / kTy; ++r) {
      const int h = tc.h0 + ty + kTy * r, w = tc.w0 + tx;
      if (h < H && w < Wd) {
        const W v = tile[ty + kTy * r][tx];
        const int64_t p = int64_t(h) * Wd + w;
        if (o0) o0[off + p] = v;
        if (o2) o2[off + L - 1 - p] = v;
      }
    }
  }
  if (o1 || o3) {
#pragma unroll
    for (int r = 0; r < kT / kTy; ++r) {
      const int w = tc.w0 + ty + kTy * r, h = tc.h0 + tx;
      if (h < H && w < Wd) {
        const W v = tile[tx][ty + kTy * r];
        const int64_t q = int64_t(w) * H + h;
        if (o1) o1[off + q] = v;
        if (o3) o3[off + L - 1 - q] = v;
      }
    }
  }
}

template <typename R>
__device__ __forceinline__ float ld_route(const R* p, int64_t i) {
  return Elem<R>::load(p, i);
}

template <typename T, typename R>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, int tiles_h, int tiles_w) {
  __shared__ float t1[kT][kT + 1];
  __shared__ float t3[kT][kT + 1];
  const int64_t C = a.C;
  const int H = int(a.H), Wd = int(a.W);
  const TileCoord tc = tile_coord(C, tiles_h, tiles_w);
  const int64_t L = int64_t(H) * Wd;
  const R* r0 = static_cast<const R*>(a.routes) + (tc.b * 4 * C + tc.c) * L;
  const R* r1 = r0 + C * L;
  const R* r2 = r1 + C * L;
  const R* r3 = r2 + C * L;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
#pragma unroll
  for (int r = 0; r < kT / kTy; ++r) {
    const int w = tc.w0 + ty + kTy * r, h = tc.h0 + tx;
    if (h < H && w < Wd) {
      const int64_t q = int64_t(w) * H + h;
      t1[ty + kTy * r][tx] = ld_route(r1, q);
      t3[ty + kTy * r][tx] = ld_route(r3, L - 1 - q);
    }
  }
  __syncthreads();
  const int64_t plane = (tc.b * C + tc.c) * L;
  float dsum = 0.0f;
  if (a.Dskip) dsum = ((a.Dskip[tc.c] + a.Dskip[C + tc.c]) + a.Dskip[2 * C + tc.c]) + a.Dskip[3 * C + tc.c];
  const T* xg = static_cast<const T*>(a.x);
  const T* zg = static_cast<const T*>(a.z);
  T* yg = static_cast<T*>(a.y);
#pragma unroll
  for (int r = 0; r < kT / kTy; ++r) {
    const int h = tc.h0 + ty + kTy * r, w = tc.w0 + tx;
    if (h < H && w < Wd) {
      const int64_t p = int64_t(h) * Wd + w;
      float v = ld_route(r0, p) + t1[tx][ty + kTy * r];
      v = v + ld_route(r2, L - 1 - p);
      v = v + t3[tx][ty + kTy * r];
      if (a.Dskip && xg) v = fmaf(dsum, Elem<T>::load(xg, plane + p), v);
      if (a.merged_f32) a.merged_f32[plane + p] = v;
      if (zg) v *= silu(Elem<T>::load(zg, plane + p));
      if (yg) Elem<T>::store(yg, plane + p, v);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(GateBwdArgs a, int tiles_h, int tiles_w) {
  __shared__ float tile[kT][kT + 1];
  const int64_t C = a.C;
  const int H = int(a.H), Wd = int(a.W);
  const TileCoord tc = tile_coord(C, tiles_h, tiles_w);
  const int64_t L = int64_t(H) * Wd;
  const int64_t plane = (tc.b * C + tc.c) * L;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  const T* zg = static_cast<const T*>(a.z);
  const T* dg = static_cast<const T*>(a.dout);
  T* dzg = static_cast<T*>(a.dz);
#pragma unroll
  for (int r = 0; r < kT / kTy; ++r) {
    const int h = tc.h0 + ty + kTy * r, w = tc.w0 + tx;
    if (h < H && w < Wd) {
      const int64_t p = plane + int64_t(h) * Wd + w;
      const float g = Elem<T>::load(dg, p);
      float dm = g;
      if (zg) {
        const float z = Elem<T>::load(zg, p);
        const float s = sigmoid(z);
        dm = g * z * s;
        const float m = a.merged[p];
        Elem<T>::store(dzg, p, g * m * s * (1.0f + z * (1.0f - s)));
      }
      a.dM[p] = dm;
      tile[ty + kTy * r][tx] = dm;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kT / kTy; ++r) {
    const int w = tc.w0 + ty + kTy * r, h = tc.h0 + tx;
    if (h < H && w < Wd) a.dMT[plane + int64_t(w) * H + h] = tile[tx][ty + kTy * r];
  }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_zero_kernel<<<dim3(uint32_t(cdiv(n, 256))), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const void* x, const ScanOutputs& o, int64_t batch, int64_t C, int64_t H,
                                int64_t W, int elem_bytes, hipStream_t s) {
  const int th = int(cdiv(H, kT)), tw = int(cdiv(W, kT));
  const int64_t blocks = batch * C * th * tw;
  if (blocks == 0) return hipSuccess;
  if (elem_bytes == 2)
    route_scatter_kernel<uint16_t><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(x), o, C, int(H), int(W), th, tw);
  else
    route_scatter_kernel<uint32_t><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(
        static_cast<const uint32_t*>(x), o, C, int(H), int(W), th, tw);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int th = int(cdiv(a.H, kT)), tw = int(cdiv(a.W, kT));
  const int64_t blocks = a.batch * a.C * th * tw;
  if (blocks == 0) return hipSuccess;
  const dim3 g{uint32_t(blocks)}, b{256};
  if (a.dtype == 0) {
    merge_kernel<float, float><<<g, b, 0, s>>>(a, th, tw);
  } else if (a.routes_f32) {
    merge_kernel<bf16, float><<<g, b, 0, s>>>(a, th, tw);
  } else {
    merge_kernel<bf16, bf16><<<g, b, 0, s>>>(a, th, tw);
  }
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  const int th = int(cdiv(a.H, kT)), tw = int(cdiv(a.W, kT));
  const int64_t blocks = a.batch * a.C * th * tw;
  if (blocks == 0) return hipSuccess;
  if (a.dtype == 0)
    gate_bwd_kernel<float><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a, th, tw);
  else
    gate_bwd_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(a, th, tw);
  return hipGetLastError();
}

}  // namespace ss2d
