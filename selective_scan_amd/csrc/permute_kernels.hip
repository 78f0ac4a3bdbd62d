// Route permutations of SS2D: cross-scan (map -> four route orders), cross-merge (four route
// orders -> map, summed in fp32), and the per-pixel gate of the merged map (forward and
// backward).  Routes, after the SS2D section of the VMamba paper (Fig. 2): k = 0 row-major,
// k = 1 column-major, k = 2 / 3 the same traversals from the last pixel back to the first.
//
// Each workgroup owns a 32 x 32 pixel tile of one (b, c) plane.  Row-major routes are read and
// written along w; column-major routes along h, through a padded LDS tile so that both the
// global reads and the global writes stay contiguous.
#include <type_traits>

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
      if (a.Dskip && xg)
        v = fmaf(dsum, a.x_f32 ? static_cast<const float*>(a.x)[plane + p] : Elem<T>::load(xg, plane + p), v);
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

// ---- plane-resident variants: one workgroup per (b, c) plane ---------------------------------
// Used when the plane (and, for the merge, its two column-major routes in fp32) fits in LDS.
// Global reads and writes are 4 consecutive elements per thread, contiguous across threads.

constexpr int kPlaneThreads = 256;

// xT[b, c, w*H + h] = x[b, c, h*W + w]  (the column-major route order, not reversed).
// Four consecutive linear indices per thread (L % 4 == 0); rows may wrap inside a group of four.
// kMulti: `pp` consecutive planes per workgroup (small planes: one plane would leave most of the
// workgroup idle); the planes are contiguous, and a quad never straddles two of them.
template <typename W, bool kMulti>
__global__ __launch_bounds__(kPlaneThreads) void transpose_plane_kernel(const W* __restrict__ x, W* __restrict__ xT,
                                                                         int H, int Wd, int64_t planes, int pp) {
  extern __shared__ __align__(16) unsigned char smem[];
  W* tile = reinterpret_cast<W*>(smem);  // [plane][h][w], row stride Wd + 1
  const int L = H * Wd;
  const int64_t p0 = kMulti ? int64_t(blockIdx.x) * pp : int64_t(blockIdx.x);
  const W* xp = x + p0 * L;
  W* op = xT + p0 * L;
  const int ld = Wd + 1, pls = H * ld;
  // elements of this workgroup (they fit the LDS, so 32-bit indices suffice)
  const int Li = kMulti ? int((planes - p0 < pp ? planes - p0 : pp) * L) : L;
  // read the plane in grid order: 4 consecutive pixels per thread, four loads issued before any
  // LDS write (a load used right away costs one round trip each); quads past the plane re-read
  // quad 0 and are not stored
  using Raw = typename std::conditional<sizeof(W) == 2, uint2, uint4>::type;
  constexpr int kBatch = 4;
  for (int q0 = 4 * int(threadIdx.x); q0 < Li; q0 += 4 * kPlaneThreads * kBatch) {
    Raw raw[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int q = q0 + 4 * kPlaneThreads * e;
      raw[e] = *reinterpret_cast<const Raw*>(xp + (q < Li ? q : 0));
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int q = q0 + 4 * kPlaneThreads * e;
      if (q >= Li) break;
      W v[4];
      if constexpr (sizeof(W) == 2) {
        v[0] = W(raw[e].x & 0xffff); v[1] = W(raw[e].x >> 16); v[2] = W(raw[e].y & 0xffff); v[3] = W(raw[e].y >> 16);
      } else {
        v[0] = W(raw[e].x); v[1] = W(raw[e].y); v[2] = W(raw[e].z); v[3] = W(raw[e].w);
      }
      // one division per index: the quad's pixels follow in row order (wrapping rows)
      const int pl = kMulti ? q / L : 0, r = q - pl * L;
      int h = r / Wd, w = r - h * Wd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[pl * pls + h * ld + w] = v[j];
        if (++w == Wd) { w = 0; ++h; }
      }
    }
  }
  __syncthreads();
  // write in column-major order: t = w*H + h, 4 consecutive t per thread (L % 4 == 0)
  for (int t = 4 * int(threadIdx.x); t < Li; t += 4 * kPlaneThreads) {
    W v[4];
    const int pl = kMulti ? t / L : 0, r = t - pl * L;
    int w = r / H, h = r - w * H;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = tile[pl * pls + h * ld + w];
      if (++h == H) { h = 0; ++w; }
    }
    if (sizeof(W) == 2) {
      uint2 raw;
      raw.x = uint32_t(v[0]) | (uint32_t(v[1]) << 16);
      raw.y = uint32_t(v[2]) | (uint32_t(v[3]) << 16);
      *reinterpret_cast<uint2*>(op + t) = raw;
    } else {
      *reinterpret_cast<uint4*>(op + t) = make_uint4(uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3]));
    }
  }
}

// The SS2D merge, one plane per workgroup: y = (((r0 + r1) + r2) + r3) [+ Dsum * x] [* silu(z)],
// summed in fp32.  Routes are of type R (fp32, or the I/O type T), grid tensors of type T.  The
// skip term (kSkip), the gate (kZ) and an fp32 x (kXF32) are template parameters, and each loop
// issues up to kMergeBatch iterations' loads before using any of them: a load behind a branch,
// or used right away, costs a round trip of its own.
// kThreads: 256, or 64 (one wavefront) for planes of up to 1024 pixels, which would leave most
// of 256 threads idle.
constexpr int kMergeBatch = 4;
template <typename T, typename R, bool kSkip, bool kZ, bool kXF32, int kThreads>
__global__ __launch_bounds__(kThreads) void merge_plane_kernel(MergeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = int(a.H), Wd = int(a.W);
  const int L = H * Wd;                    // the plane fits the LDS: 32-bit indices
  const int ld = H + 1;                    // [w][h] with an odd row stride: conflict-free column reads
  float* t1 = reinterpret_cast<float*>(smem);
  float* t3 = t1 + Wd * ld;
  const int64_t plane = int64_t(blockIdx.x);  // b * C + c
  const int64_t b = plane / a.C, c = plane % a.C;
  const R* r0 = static_cast<const R*>(a.routes) + (b * 4 * a.C + c) * L;
  const R* r1 = r0 + a.C * L;
  const R* r2 = r1 + a.C * L;
  const R* r3 = r2 + a.C * L;
  constexpr int kStep = 4 * kThreads;
  // routes 1 and 3 are in column-major order: t1[w][h] = r1[w*H + h], t3[w][h] = r3[L-1-(w*H + h)]
  for (int t0 = 4 * int(threadIdx.x); t0 < L; t0 += kStep * kMergeBatch) {
    float4 v1[kMergeBatch], v3[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {  // past the plane: re-read quad 0, not stored
      const int t = t0 + kStep * e, tc = t < L ? t : 0;
      v1[e] = Elem<R>::load4(r1, tc);
      v3[e] = Elem<R>::load4(r3, L - 4 - tc);  // route-3 steps L-4-t .. L-1-t
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int t = t0 + kStep * e;
      if (t >= L) break;
      const float a1[4] = {v1[e].x, v1[e].y, v1[e].z, v1[e].w};
      const float a3[4] = {v3[e].w, v3[e].z, v3[e].y, v3[e].x};  // pixel order t .. t+3
      int w = t / H, h = t - w * H;  // one division; the quad's steps follow down the column
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t1[w * ld + h] = a1[j];
        t3[w * ld + h] = a3[j];
        if (++h == H) { h = 0; ++w; }
      }
    }
  }
  __syncthreads();
  float dsum = 0.0f;
  if (kSkip) dsum = ((a.Dskip[c] + a.Dskip[a.C + c]) + a.Dskip[2 * a.C + c]) + a.Dskip[3 * a.C + c];
  const T* xg = static_cast<const T*>(a.x) + plane * L;
  const float* xf = static_cast<const float*>(a.x) + plane * L;
  const T* zg = kZ ? static_cast<const T*>(a.z) + plane * L : nullptr;
  T* yg = a.y ? static_cast<T*>(a.y) + plane * L : nullptr;
  float* mg = a.merged_f32 ? a.merged_f32 + plane * L : nullptr;
  for (int p0 = 4 * int(threadIdx.x); p0 < L; p0 += kStep * kMergeBatch) {
    float4 v0[kMergeBatch], v2[kMergeBatch], xv[kMergeBatch], zv[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int p = p0 + kStep * e, pc = p < L ? p : 0;
      v0[e] = Elem<R>::load4(r0, pc);
      v2[e] = Elem<R>::load4(r2, L - 4 - pc);
      if constexpr (kSkip) xv[e] = kXF32 ? Elem<float>::load4(xf, pc) : Elem<T>::load4(xg, pc);
      if constexpr (kZ) zv[e] = Elem<T>::load4(zg, pc);
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int p = p0 + kStep * e;
      if (p >= L) break;
      const float a0[4] = {v0[e].x, v0[e].y, v0[e].z, v0[e].w};
      const float a2[4] = {v2[e].w, v2[e].z, v2[e].y, v2[e].x};
      float v[4];
      int h = p / Wd, w = p - h * Wd;  // one division; the quad's pixels follow along the row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float sum = a0[j] + t1[w * ld + h];
        sum = sum + a2[j];
        v[j] = sum + t3[w * ld + h];
        if (++w == Wd) { w = 0; ++h; }
      }
      if constexpr (kSkip) {
        v[0] = fmaf(dsum, xv[e].x, v[0]); v[1] = fmaf(dsum, xv[e].y, v[1]);
        v[2] = fmaf(dsum, xv[e].z, v[2]); v[3] = fmaf(dsum, xv[e].w, v[3]);
      }
      if (mg) *reinterpret_cast<float4*>(mg + p) = make_float4(v[0], v[1], v[2], v[3]);
      if constexpr (kZ) {
        v[0] *= silu(zv[e].x); v[1] *= silu(zv[e].y); v[2] *= silu(zv[e].z); v[3] *= silu(zv[e].w);
      }
      if (yg) Elem<T>::store4(yg, p, make_float4(v[0], v[1], v[2], v[3]));
    }
  }
}

// The SS2D merge from route outputs in 4-step blocks (MergeArgs: fp32, route k's step s of
// channel c at ((b 4 + k) (L/4) + s/4) C 4 + c 4 + s % 4; H and W multiples of 4).  One thread =
// one channel x one 4 x 4 pixel block: with W % 4 == 0 a block row is one 4-step group of the
// row-major routes, and with H % 4 == 0 a block column is one group of the column-major ones, so
// each route is read as four 16-byte groups and transposed in registers (no LDS).  A wavefront =
// 8 consecutive channels (lane % 8: one 128-byte line per group and route) x 8 consecutive blocks
// of the plane (row-major block order).  Same sum, in the same order, as merge_plane_kernel.
// kVecIO: x, z, y and merged are aligned for 4-element accesses (else element by element).
// 16 bytes read once, or written for a later kernel (whole lines across the wavefront), not kept
// in the caches
typedef float F4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_nt(const float* p) {
  const F4 v = __builtin_nontemporal_load(reinterpret_cast<const F4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store4_nt(float* p, float4 v) {
  __builtin_nontemporal_store(F4{v.x, v.y, v.z, v.w}, reinterpret_cast<F4*>(p));
}

template <typename T, bool kSkip, bool kZ, bool kXF32, bool kVecIO>
__global__ __launch_bounds__(64) void merge_blocked_kernel(MergeArgs a, int cblocks, int jchunks) {
  const int lane = int(threadIdx.x);
  // neighbouring chunks of a plane share the lines of its rows (a chunk's 8 blocks cover part of
  // a line per row and channel): consecutive ids on one XCD merge those partial lines in one L2
  int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int jc = int(bid % jchunks);
  bid /= jchunks;
  const int cb = int(bid % cblocks);
  const int64_t b = bid / cblocks;
  const int64_t C = a.C;
  const int64_t c = int64_t(cb) * 8 + (lane & 7);
  const int H = int(a.H), Wd = int(a.W);
  const int H4 = H / 4, W4 = Wd / 4;
  const int j = jc * 8 + (lane >> 3);
  // no LDS and no barrier in this kernel: threads past the channels or blocks leave at once
  if (c >= C || j >= H4 * W4) return;
  const int bh = j / W4, bw = j - bh * W4;
  const int h0 = 4 * bh, w0 = 4 * bw;
  const int64_t L = int64_t(H) * Wd, L4 = L / 4;
  const float* rt = static_cast<const float*>(a.routes) + (b * 4 * L4 * C + c) * 4;
  const int64_t kst = L4 * C * 4;  // between routes
  float4 r0[4], r1[4], r2[4], r3[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t g0 = int64_t(h0 + i) * W4 + bw;   // row h0 + i of the block, row-major order
    const int64_t g1 = int64_t(w0 + i) * H4 + bh;   // column w0 + i, column-major order
    r0[i] = load4_nt(rt + g0 * C * 4);
    r1[i] = load4_nt(rt + kst + g1 * C * 4);
    r2[i] = load4_nt(rt + 2 * kst + (L4 - 1 - g0) * C * 4);
    r3[i] = load4_nt(rt + 3 * kst + (L4 - 1 - g1) * C * 4);
  }
  const int64_t plane = (b * C + c) * L;
  float4 xv[4], zv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t o = plane + int64_t(h0 + i) * Wd + w0;
    if constexpr (kSkip) {
      if constexpr (kXF32) {
        const float* xf = static_cast<const float*>(a.x);
        xv[i] = kVecIO ? Elem<float>::load4(xf, o) : make_float4(xf[o], xf[o + 1], xf[o + 2], xf[o + 3]);
      } else {
        const T* xg = static_cast<const T*>(a.x);
        xv[i] = kVecIO ? Elem<T>::load4(xg, o)
                       : make_float4(Elem<T>::load(xg, o), Elem<T>::load(xg, o + 1), Elem<T>::load(xg, o + 2),
                                     Elem<T>::load(xg, o + 3));
      }
    }
    if constexpr (kZ) {
      const T* zg = static_cast<const T*>(a.z);
      zv[i] = kVecIO ? Elem<T>::load4(zg, o)
                     : make_float4(Elem<T>::load(zg, o), Elem<T>::load(zg, o + 1), Elem<T>::load(zg, o + 2),
                                   Elem<T>::load(zg, o + 3));
    }
  }
  float dsum = 0.0f;
  if (kSkip) dsum = ((a.Dskip[c] + a.Dskip[C + c]) + a.Dskip[2 * C + c]) + a.Dskip[3 * C + c];
  auto el = [](const float4& v, int e) { return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w)); };
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // block row i: pixels (h0 + i, w0 + q)
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // route 0: group row i, element q; route 1: column q, element i; route 2 runs backwards
      // through the row (element 3 - q), route 3 backwards down the column (element 3 - i)
      float sum = el(r0[i], q) + el(r1[q], i);
      sum = sum + el(r2[i], 3 - q);
      v[q] = sum + el(r3[q], 3 - i);
    }
    if constexpr (kSkip) {
      v[0] = fmaf(dsum, xv[i].x, v[0]); v[1] = fmaf(dsum, xv[i].y, v[1]);
      v[2] = fmaf(dsum, xv[i].z, v[2]); v[3] = fmaf(dsum, xv[i].w, v[3]);
    }
    const int64_t o = plane + int64_t(h0 + i) * Wd + w0;
    if (a.merged_f32) {
      if (kVecIO)
        *reinterpret_cast<float4*>(a.merged_f32 + o) = make_float4(v[0], v[1], v[2], v[3]);
      else
        for (int q = 0; q < 4; ++q) a.merged_f32[o + q] = v[q];
    }
    if constexpr (kZ) {
      v[0] *= silu(zv[i].x); v[1] *= silu(zv[i].y); v[2] *= silu(zv[i].z); v[3] *= silu(zv[i].w);
    }
    if (a.y) {
      T* yg = static_cast<T*>(a.y);
      if (kVecIO)
        Elem<T>::store4(yg, o, make_float4(v[0], v[1], v[2], v[3]));
      else
        for (int q = 0; q < 4; ++q) Elem<T>::store(yg, o + q, v[q]);
    }
  }
}

// The same merge for small planes whose H or W is not a multiple of 4 (L a multiple of 4, at
// most kSmallBlockedL pixels): one workgroup per (image, 8 consecutive channels).  Each route's
// 4-step groups of the 8 channels (one whole line per group) are added into an LDS copy of the 8
// planes at the pixels of their steps, route by route, so each pixel's sum is ((y0 + y1) + y2) + y3
// as in the other merges; then every pixel of the 8 planes gets its skip term and gate and is
// written in grid order.
constexpr int64_t kSmallBlockedL = 2048;  // 8 planes of fp32 in 64 KB of LDS
template <typename T, bool kSkip, bool kZ, bool kXF32>
__global__ __launch_bounds__(256) void merge_blocked_small_kernel(MergeArgs a, int cblocks) {
  extern __shared__ __align__(16) float acc[];  // [8][L]
  const int tid = int(threadIdx.x);
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = int(bid % cblocks);
  const int64_t b = bid / cblocks;
  const int64_t C = a.C;
  const int H = int(a.H), Wd = int(a.W), L = H * Wd, G = L / 4;
  const float* rt = static_cast<const float*>(a.routes) + b * 4 * int64_t(G) * C * 4;
#pragma unroll 1
  for (int k = 0; k < 4; ++k) {
    for (int idx = tid; idx < G * 8; idx += 256) {
      const int g = idx >> 3, c8 = idx & 7;
      const int64_t c = int64_t(cb) * 8 + c8;
      if (c >= C) continue;
      const float4 v = load4_nt(rt + ((int64_t(k) * G + g) * C + c) * 4);
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int st = 4 * g + q;
        if (k >= 2) st = L - 1 - st;                    // routes 2, 3 run backwards
        const int pix = (k & 1) ? (st % H) * Wd + st / H : st;  // column-major step -> pixel
        float* dst = acc + c8 * L + pix;
        *dst = (k == 0) ? e[q] : *dst + e[q];
      }
    }
    __syncthreads();
  }
  const T* xg = static_cast<const T*>(a.x);
  const float* xf = static_cast<const float*>(a.x);
  const T* zg = static_cast<const T*>(a.z);
  T* yg = static_cast<T*>(a.y);
  for (int idx = tid; idx < 8 * L; idx += 256) {
    const int c8 = idx / L, pix = idx - c8 * L;
    const int64_t c = int64_t(cb) * 8 + c8;
    if (c >= C) continue;
    const int64_t o = (b * C + c) * L + pix;
    float v = acc[idx];
    if constexpr (kSkip) {
      const float dsum = ((a.Dskip[c] + a.Dskip[C + c]) + a.Dskip[2 * C + c]) + a.Dskip[3 * C + c];
      v = fmaf(dsum, kXF32 ? xf[o] : Elem<T>::load(xg, o), v);
    }
    if (a.merged_f32) a.merged_f32[o] = v;
    if constexpr (kZ) v *= silu(Elem<T>::load(zg, o));
    if (yg) Elem<T>::store(yg, o, v);
  }
}

// The gate backward fused with its merge (see MergeGateArgs), one plane per workgroup.  LDS:
// routes 1 and 3 transposed to [w][h] (as in the merge), and dM as [h][w] for the dMT write.  As
// in the merge, the skip term and an fp32 x are template parameters and the loads of up to
// kMergeBatch iterations are issued before any is used.
// kThreads: as in the merge (one wavefront for planes of up to 1024 pixels).
// kM: the pre-gate merged map is read from a.merged (a keep_states forward wrote it, with the
// same sum in the same order) instead of being formed from the routes; LDS then holds only dM.
template <typename T, bool kSkip, bool kXF32, int kThreads, bool kM = false>
__global__ __launch_bounds__(kThreads) void merge_gate_bwd_plane_kernel(MergeGateArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = int(a.H), Wd = int(a.W);
  const int L = H * Wd;  // the plane fits the LDS: 32-bit indices
  const int ldc = H + 1, ldr = Wd + 1;
  float* t1 = reinterpret_cast<float*>(smem);
  float* t3 = t1 + Wd * ldc;
  float* tm = kM ? t1 : t3 + Wd * ldc;  // [h][w]
  const int64_t plane = int64_t(blockIdx.x);
  const int64_t b = plane / a.C, c = plane % a.C;
  const float* r0 = a.routes + (b * 4 * a.C + c) * L;
  const float* r1 = r0 + a.C * L;
  const float* r2 = r1 + a.C * L;
  const float* r3 = r2 + a.C * L;
  const float* mg = a.merged + plane * L;
  constexpr int kStep = 4 * kThreads;
  if (!kM)
  for (int t0 = 4 * int(threadIdx.x); t0 < L; t0 += kStep * kMergeBatch) {
    float4 v1[kMergeBatch], v3[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {  // past the plane: re-read quad 0, not stored
      const int t = t0 + kStep * e, tc = t < L ? t : 0;
      v1[e] = *reinterpret_cast<const float4*>(r1 + tc);
      v3[e] = *reinterpret_cast<const float4*>(r3 + (L - 4 - tc));
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int t = t0 + kStep * e;
      if (t >= L) break;
      const float a1[4] = {v1[e].x, v1[e].y, v1[e].z, v1[e].w};
      const float a3[4] = {v3[e].w, v3[e].z, v3[e].y, v3[e].x};
      int w = t / H, h = t - w * H;  // one division; the quad's steps follow down the column
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t1[w * ldc + h] = a1[j];
        t3[w * ldc + h] = a3[j];
        if (++h == H) { h = 0; ++w; }
      }
    }
  }
  __syncthreads();
  float dsum = 0.0f;
  if (kSkip) dsum = ((a.Dskip[c] + a.Dskip[a.C + c]) + a.Dskip[2 * a.C + c]) + a.Dskip[3 * a.C + c];
  const T* xg = static_cast<const T*>(a.x) + plane * L;
  const float* xf = static_cast<const float*>(a.x) + plane * L;
  const T* zg = static_cast<const T*>(a.z) + plane * L;
  const T* gg = static_cast<const T*>(a.dout) + plane * L;
  T* dzg = static_cast<T*>(a.dz) + plane * L;
  float* dmg = a.dM + plane * L;
  for (int p0 = 4 * int(threadIdx.x); p0 < L; p0 += kStep * kMergeBatch) {
    float4 v0[kMergeBatch], v2[kMergeBatch], xv[kMergeBatch], zv[kMergeBatch], gv[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int p = p0 + kStep * e, pc = p < L ? p : 0;
      if constexpr (kM) {
        v0[e] = load4_nt(mg + pc);  // the kept map: read once
        v2[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        v0[e] = *reinterpret_cast<const float4*>(r0 + pc);
        v2[e] = *reinterpret_cast<const float4*>(r2 + (L - 4 - pc));
      }
      if constexpr (kSkip) xv[e] = kXF32 ? Elem<float>::load4(xf, pc) : Elem<T>::load4(xg, pc);
      zv[e] = Elem<T>::load4(zg, pc);
      gv[e] = Elem<T>::load4(gg, pc);
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int p = p0 + kStep * e;
      if (p >= L) break;
      const float a0[4] = {v0[e].x, v0[e].y, v0[e].z, v0[e].w};
      const float a2[4] = {v2[e].w, v2[e].z, v2[e].y, v2[e].x};
      const float xs[4] = {xv[e].x, xv[e].y, xv[e].z, xv[e].w};
      const float zs[4] = {zv[e].x, zv[e].y, zv[e].z, zv[e].w}, gs[4] = {gv[e].x, gv[e].y, gv[e].z, gv[e].w};
      float dz[4], dm[4];
      int h = p / Wd, w = p - h * Wd;  // one division; the quad's pixels follow along the row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float m = a0[j];
        if constexpr (!kM) {
          m = m + t1[w * ldc + h];
          m = m + a2[j];
          m = m + t3[w * ldc + h];
          if (kSkip) m = fmaf(dsum, xs[j], m);
        }
        const float sz = sigmoid(zs[j]);
        dm[j] = gs[j] * zs[j] * sz;
        dz[j] = gs[j] * m * sz * (1.0f + zs[j] * (1.0f - sz));
        tm[h * ldr + w] = dm[j];
        if (++w == Wd) { w = 0; ++h; }
      }
      store4_nt(dmg + p, make_float4(dm[0], dm[1], dm[2], dm[3]));
      Elem<T>::store4(dzg, p, make_float4(dz[0], dz[1], dz[2], dz[3]));
    }
  }
  __syncthreads();
  float* dmt = a.dMT + plane * L;
  for (int t = 4 * int(threadIdx.x); t < L; t += kStep) {
    float v[4];
    int w = t / H, h = t - w * H;  // one division; the quad's steps follow down the column
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = tm[h * ldr + w];
      if (++h == H) { h = 0; ++w; }
    }
    store4_nt(dmt + t, make_float4(v[0], v[1], v[2], v[3]));
  }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Two-direction merge: one thread per element of the (batch, C, L) output; direction 1 is read
// at L-1-l, so consecutive threads read consecutive (descending) addresses of it.
// element i of (batch, C, L) -> row = b C + c and position l: 32-bit divisions when every index
// fits (a 64-bit division costs several times as many instructions)
__device__ __forceinline__ void row_of(const BidirArgs& a, int64_t i, int64_t& row, int64_t& l, int64_t& b,
                                       int64_t& c) {
  if (a.batch * a.C * a.L <= 0xffffffffLL) {
    const uint32_t ii = uint32_t(i), L = uint32_t(a.L), C = uint32_t(a.C);
    const uint32_t r = ii / L, bb = r / C;
    row = r; l = ii - r * L; b = bb; c = r - bb * C;
  } else {
    row = i / a.L; l = i - row * a.L; b = row / a.C; c = row - b * a.C;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bidir_merge_kernel(BidirArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = a.batch * a.C * a.L;
  if (i >= n) return;
  int64_t row, l, b, c;
  row_of(a, i, row, l, b, c);
  const float* y0 = a.ys + (b * 2 * a.C + c) * a.L;
  const float* y1 = y0 + a.C * a.L;
  float v = y0[l] + y1[a.L - 1 - l];
  if (a.z) v *= silu(Elem<T>::load(static_cast<const T*>(a.z), i));
  Elem<T>::store(static_cast<T*>(a.out), i, v);
}

template <typename T>
__global__ __launch_bounds__(256) void bidir_gate_bwd_kernel(BidirArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = a.batch * a.C * a.L;
  if (i >= n) return;
  int64_t row, l, b, c;
  row_of(a, i, row, l, b, c);
  const int64_t r0 = (b * 2 * a.C + c) * a.L, r1 = r0 + a.C * a.L;
  const float g = Elem<T>::load(static_cast<const T*>(a.dout), i);
  float dm = g;
  if (a.z) {
    const float m = a.ys[r0 + l] + a.ys[r1 + a.L - 1 - l];
    const float zv = Elem<T>::load(static_cast<const T*>(a.z), i);
    const float sz = sigmoid(zv);
    dm = g * zv * sz;
    Elem<T>::store(static_cast<T*>(a.dz), i, g * m * sz * (1.0f + zv * (1.0f - sz)));
  }
  a.dy[r0 + l] = dm;
  a.dy[r1 + a.L - 1 - l] = dm;
}

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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

namespace {
template <typename T, typename R, bool kSkip, bool kZ, int kThreads>
void launch_merge_plane_t(const MergeArgs& a, dim3 g, size_t lds, hipStream_t s) {
  const dim3 b{kThreads};
  if (kSkip && a.x_f32)
    merge_plane_kernel<T, R, kSkip, kZ, true, kThreads><<<g, b, lds, s>>>(a);
  else
    merge_plane_kernel<T, R, kSkip, kZ, false, kThreads><<<g, b, lds, s>>>(a);
}
template <typename T, typename R, bool kSkip, bool kZ>
void launch_merge_plane_x(const MergeArgs& a, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  if (b.x == 64)
    launch_merge_plane_t<T, R, kSkip, kZ, 64>(a, g, lds, s);
  else
    launch_merge_plane_t<T, R, kSkip, kZ, kPlaneThreads>(a, g, lds, s);
}
template <typename T, typename R>
void launch_merge_plane(const MergeArgs& a, dim3 g, dim3 b, size_t lds, hipStream_t s) {
  const bool skip = a.Dskip != nullptr && a.x != nullptr, z = a.z != nullptr;
  if (skip)
    z ? launch_merge_plane_x<T, R, true, true>(a, g, b, lds, s) : launch_merge_plane_x<T, R, true, false>(a, g, b, lds, s);
  else
    z ? launch_merge_plane_x<T, R, false, true>(a, g, b, lds, s) : launch_merge_plane_x<T, R, false, false>(a, g, b, lds, s);
}
}  // namespace

namespace {
template <typename T, bool kSkip, bool kZ, bool kXF32>
void launch_merge_blocked_v(const MergeArgs& a, dim3 g, int cblocks, int jchunks, bool vec_io, hipStream_t s) {
  if (vec_io)
    merge_blocked_kernel<T, kSkip, kZ, kXF32, true><<<g, dim3(64), 0, s>>>(a, cblocks, jchunks);
  else
    merge_blocked_kernel<T, kSkip, kZ, kXF32, false><<<g, dim3(64), 0, s>>>(a, cblocks, jchunks);
}
template <typename T>
void launch_merge_blocked_t(const MergeArgs& a, dim3 g, int cblocks, int jchunks, bool vec_io, hipStream_t s) {
  const bool skip = a.Dskip != nullptr && a.x != nullptr, z = a.z != nullptr;
  if (skip && a.x_f32)
    z ? launch_merge_blocked_v<T, true, true, true>(a, g, cblocks, jchunks, vec_io, s)
      : launch_merge_blocked_v<T, true, false, true>(a, g, cblocks, jchunks, vec_io, s);
  else if (skip)
    z ? launch_merge_blocked_v<T, true, true, false>(a, g, cblocks, jchunks, vec_io, s)
      : launch_merge_blocked_v<T, true, false, false>(a, g, cblocks, jchunks, vec_io, s);
  else
    z ? launch_merge_blocked_v<T, false, true, false>(a, g, cblocks, jchunks, vec_io, s)
      : launch_merge_blocked_v<T, false, false, false>(a, g, cblocks, jchunks, vec_io, s);
}

template <typename T, bool kSkip, bool kZ, bool kXF32>
void launch_merge_small_v(const MergeArgs& a, dim3 g, int cblocks, size_t lds, hipStream_t s) {
  merge_blocked_small_kernel<T, kSkip, kZ, kXF32><<<g, dim3(256), lds, s>>>(a, cblocks);
}
template <typename T>
void launch_merge_small_t(const MergeArgs& a, dim3 g, int cblocks, size_t lds, hipStream_t s) {
  const bool skip = a.Dskip != nullptr && a.x != nullptr, z = a.z != nullptr;
  if (skip && a.x_f32)
    z ? launch_merge_small_v<T, true, true, true>(a, g, cblocks, lds, s)
      : launch_merge_small_v<T, true, false, true>(a, g, cblocks, lds, s);
  else if (skip)
    z ? launch_merge_small_v<T, true, true, false>(a, g, cblocks, lds, s)
      : launch_merge_small_v<T, true, false, false>(a, g, cblocks, lds, s);
  else
    z ? launch_merge_small_v<T, false, true, false>(a, g, cblocks, lds, s)
      : launch_merge_small_v<T, false, false, false>(a, g, cblocks, lds, s);
}
}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t L = a.H * a.W;
  if (a.routes_blocked && !(a.H % 4 == 0 && a.W % 4 == 0)) {
    // fp32 routes in 4-step blocks on a small plane whose sides are not multiples of 4
    if (!a.routes_f32 || !ss2d_routes_blocked(a.H, a.W) || L > kSmallBlockedL || !aligned16(a.routes))
      return hipErrorInvalidValue;
    const int64_t cblocks = cdiv(a.C, 8), blocks = a.batch * cblocks;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const size_t lds = size_t(8) * size_t(L) * 4;
    const dim3 g{uint32_t(blocks)};
    if (a.dtype == 0)
      launch_merge_small_t<float>(a, g, int(cblocks), lds, s);
    else
      launch_merge_small_t<bf16>(a, g, int(cblocks), lds, s);
    return hipGetLastError();
  }
  if (a.routes_blocked) {
    // fp32 routes in 4-step blocks (written by the route scans when H and W are multiples of 4)
    if (!a.routes_f32 || !ss2d_routes_blocked(a.H, a.W) || !aligned16(a.routes)) return hipErrorInvalidValue;
    const int64_t cblocks = cdiv(a.C, 8), jchunks = cdiv((a.H / 4) * (a.W / 4), 8);
    const int64_t blocks = a.batch * cblocks * jchunks;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const uintptr_t tio = reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.z) |
                          (a.x_f32 ? 0 : reinterpret_cast<uintptr_t>(a.x));
    const bool vec_io = (tio & (a.dtype == 0 ? 15 : 7)) == 0 && (!a.x_f32 || aligned16(a.x)) &&
                        (!a.merged_f32 || aligned16(a.merged_f32));
    const dim3 g{uint32_t(blocks)};
    if (a.dtype == 0)
      launch_merge_blocked_t<float>(a, g, int(cblocks), int(jchunks), vec_io, s);
    else
      launch_merge_blocked_t<bf16>(a, g, int(cblocks), int(jchunks), vec_io, s);
    return hipGetLastError();
  }
  const size_t plane_lds = size_t(2) * size_t(a.W) * size_t(a.H + 1) * 4;
  const uintptr_t route_align = a.routes_f32 ? 15 : (a.dtype == 0 ? 15 : 7);
  if (plane_lds <= 64 * 1024 && a.batch * a.C > 0 &&
      (reinterpret_cast<uintptr_t>(a.routes) & route_align) == 0 && (!a.merged_f32 || aligned16(a.merged_f32)) &&
      (a.dtype == 0 ? (aligned16(a.y) && aligned16(a.x) && aligned16(a.z))
                    : ((reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.x) |
                        reinterpret_cast<uintptr_t>(a.z)) & 7) == 0) &&
      (!a.x_f32 || aligned16(a.x)) && L % 4 == 0) {
    const dim3 g{uint32_t(a.batch * a.C)}, b{L <= 1024 ? 64u : uint32_t(kPlaneThreads)};
    if (a.dtype == 0)
      launch_merge_plane<float, float>(a, g, b, plane_lds, s);
    else if (a.routes_f32)
      launch_merge_plane<bf16, float>(a, g, b, plane_lds, s);
    else
      launch_merge_plane<bf16, bf16>(a, g, b, plane_lds, s);
    return hipGetLastError();
  }
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

hipError_t launch_bidir_merge(const BidirArgs& a, hipStream_t s) {
  const int64_t n = a.batch * a.C * a.L;
  if (n == 0) return hipSuccess;
  const dim3 g{uint32_t(cdiv(n, 256))}, b{256};
  if (a.dtype == 0)
    bidir_merge_kernel<float><<<g, b, 0, s>>>(a);
  else
    bidir_merge_kernel<bf16><<<g, b, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_bidir_gate_bwd(const BidirArgs& a, hipStream_t s) {
  const int64_t n = a.batch * a.C * a.L;
  if (n == 0) return hipSuccess;
  const dim3 g{uint32_t(cdiv(n, 256))}, b{256};
  if (a.dtype == 0)
    bidir_gate_bwd_kernel<float><<<g, b, 0, s>>>(a);
  else
    bidir_gate_bwd_kernel<bf16><<<g, b, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* x, void* xT, int64_t batch, int64_t C, int64_t H, int64_t W, int elem_bytes,
                            hipStream_t s) {
  const int64_t planes = batch * C;
  if (planes == 0 || H * W == 0) return hipSuccess;
  const size_t lds = size_t(H) * size_t(W + 1) * size_t(elem_bytes);
  const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(xT);
  if ((H * W) % 4 == 0 && lds <= 64 * 1024 && (al % (4 * elem_bytes)) == 0) {
    // planes of under 512 pixels: several per workgroup, about 2048 pixels in all
    int pp = H * W < 512 ? int(2048 / (H * W)) : 1;
    if (pp > 16) pp = 16;
    while (pp > 1 && size_t(pp) * lds > 64 * 1024) --pp;
    const int64_t blocks = (planes + pp - 1) / pp;
    const dim3 g{uint32_t(blocks)}, b{kPlaneThreads};
    const size_t l = size_t(pp) * lds;
    if (elem_bytes == 2) {
      const auto* xi = static_cast<const uint16_t*>(x);
      auto* xo = static_cast<uint16_t*>(xT);
      if (pp > 1)
        transpose_plane_kernel<uint16_t, true><<<g, b, l, s>>>(xi, xo, int(H), int(W), planes, pp);
      else
        transpose_plane_kernel<uint16_t, false><<<g, b, l, s>>>(xi, xo, int(H), int(W), planes, 1);
    } else {
      const auto* xi = static_cast<const uint32_t*>(x);
      auto* xo = static_cast<uint32_t*>(xT);
      if (pp > 1)
        transpose_plane_kernel<uint32_t, true><<<g, b, l, s>>>(xi, xo, int(H), int(W), planes, pp);
      else
        transpose_plane_kernel<uint32_t, false><<<g, b, l, s>>>(xi, xo, int(H), int(W), planes, 1);
    }
    return hipGetLastError();
  }
  ScanOutputs o{};
  o.out[1] = xT;
  o.batch_stride = C * H * W;
  return launch_route_scatter(x, o, batch, C, H, W, elem_bytes, s);
}

template <int kThreads>
static void launch_merge_gate_bwd_t(const MergeGateArgs& a, dim3 g, size_t lds, hipStream_t s) {
  const dim3 b{kThreads};
  const bool skip = a.Dskip != nullptr && a.x != nullptr;
  if (a.merged_in) {
    if (a.dtype == 0)
      merge_gate_bwd_plane_kernel<float, false, false, kThreads, true><<<g, b, lds, s>>>(a);
    else
      merge_gate_bwd_plane_kernel<bf16, false, false, kThreads, true><<<g, b, lds, s>>>(a);
  } else if (a.dtype == 0) {
    if (skip)
      merge_gate_bwd_plane_kernel<float, true, true, kThreads><<<g, b, lds, s>>>(a);
    else
      merge_gate_bwd_plane_kernel<float, false, false, kThreads><<<g, b, lds, s>>>(a);
  } else {
    if (skip && a.x_f32)
      merge_gate_bwd_plane_kernel<bf16, true, true, kThreads><<<g, b, lds, s>>>(a);
    else if (skip)
      merge_gate_bwd_plane_kernel<bf16, true, false, kThreads><<<g, b, lds, s>>>(a);
    else
      merge_gate_bwd_plane_kernel<bf16, false, false, kThreads><<<g, b, lds, s>>>(a);
  }
}

hipError_t launch_merge_gate_bwd(const MergeGateArgs& a, hipStream_t s) {
  if (a.routes_blocked && !a.merged_in) {
    // the plane kernels read routes in the row layout: form the pre-gate map from the blocked
    // routes first (the same sum in the same order), then take the path that reads it
    MergeArgs m{};
    m.routes = a.routes;
    m.routes_f32 = 1;
    m.routes_blocked = 1;
    m.x = a.x;
    m.x_f32 = a.x_f32;
    m.Dskip = a.Dskip;
    m.merged_f32 = a.merged;
    m.batch = a.batch;
    m.C = a.C;
    m.H = a.H;
    m.W = a.W;
    m.dtype = a.dtype;
    const hipError_t e = a.z ? launch_merge(m, s) : hipSuccess;
    if (e != hipSuccess) return e;
    MergeGateArgs k = a;
    k.routes_blocked = 0;
    k.merged_in = 1;
    return launch_merge_gate_bwd(k, s);
  }
  const int64_t L = a.H * a.W;
  const size_t lds = ((a.merged_in ? 0 : size_t(2) * size_t(a.W) * size_t(a.H + 1)) + size_t(a.H) * size_t(a.W + 1)) * 4;
  const uintptr_t io = reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.z) |
                       reinterpret_cast<uintptr_t>(a.dout) | reinterpret_cast<uintptr_t>(a.dz);
  if (a.z && lds <= 64 * 1024 && L % 4 == 0 && a.batch * a.C > 0 && aligned16(a.routes) && aligned16(a.dM) &&
      aligned16(a.dMT) && aligned16(a.merged) && (io & (a.dtype == 0 ? 15 : 7)) == 0 && (!a.x_f32 || aligned16(a.x))) {
    const dim3 g{uint32_t(a.batch * a.C)};
    if (L <= 1024)
      launch_merge_gate_bwd_t<64>(a, g, lds, s);
    else
      launch_merge_gate_bwd_t<kPlaneThreads>(a, g, lds, s);
    return hipGetLastError();
  }
  // two kernels: the pre-gate merge into `merged` (only needed with a gate, and not when the
  // forward left it there), then the gate
  if (a.z && !a.merged_in) {
    MergeArgs m{};
    m.routes = a.routes;
    m.routes_f32 = 1;
    m.x = a.x;
    m.x_f32 = a.x_f32;
    m.Dskip = a.Dskip;
    m.merged_f32 = a.merged;
    m.batch = a.batch;
    m.C = a.C;
    m.H = a.H;
    m.W = a.W;
    m.dtype = a.dtype;
    const hipError_t e = launch_merge(m, s);
    if (e != hipSuccess) return e;
  }
  GateBwdArgs g{};
  g.merged = a.merged;
  g.z = a.z;
  g.dout = a.dout;
  g.dM = a.dM;
  g.dMT = a.dMT;
  g.dz = a.dz;
  g.batch = a.batch;
  g.C = a.C;
  g.H = a.H;
  g.W = a.W;
  g.dtype = a.dtype;
  return launch_gate_bwd(g, s);
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
