// Dense fp32 products of the Δ/B/C producer (the per-route x_proj and dt_proj of the scanned
// sequence, the `Mamba` module's projections on "Vision Mamba structure and principle", section
// 2) and of its gradient, on the matrix cores: v_mfma_f32_32x32x2f32, fp32 operands and
// accumulation (no rounding of any operand).  Lane layout of the instruction (checked on the
// device): lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator v of lane l is
// C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].  The two k-slots of an instruction may stand for any
// two elements of the contraction as long as A and B agree: here step s of a chunk of 2H
// elements takes slot 0 from element s and slot 1 from element H + s, so that each lane reads H
// consecutive elements of its row.
//
// Two kernels, both with every load branch-free (clamped addresses) and the next chunk's loads
// issued before the current chunk's MFMAs.  Values past the end of the contraction are zeroed
// on one operand by a product with a 0/1 mask (exact for the finite values read through a
// clamped address), not by a select: the compiler turns a select of a loaded word into a branch
// around the load and so moves the load behind the MFMAs.  The other operand is then finite
// (a valid element), so the padded terms are exact zeros.
//   proj_kernel   C (M x L) (+)= W (M x K) X (K x L): a small weight times a long sequence (x_proj,
//                 dt_proj, and the transposed products of the gradient).  A tile is 32 MB rows x
//                 128 columns (MB <= 4); wavefront w owns columns [32 w, 32 w + 32) and all MB
//                 row blocks.
//                 The sequence chunk goes through LDS (double buffered); the weight values come
//                 straight from memory (a few KB per route, cache resident).
//   wgrad_kernel  C (M x N) = sum_l A (M x l) B (N x l): the weight gradients, a contraction over
//                 images and steps.  Each wavefront takes 16 steps of every 64-step unit of its
//                 slice and keeps the whole tile; the four wavefronts are summed through LDS.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kPN = 128;  // columns per tile of proj_kernel

__device__ __forceinline__ float4 rev4(float4 v) { return make_float4(v.w, v.z, v.y, v.x); }

// kVec: 4-element sequence loads (L % 4 == 0, aligned views).  kAVec: the weight rows are
// contiguous along the contraction (K % 4 == 0, aligned): 4-element weight loads.  kPair: routes
// k and k + 2 in one tile (rows [0, M/2) route k, rows [M/2, M) route k + 2, written at column
// L - 1 - j, since route k + 2 is route k read backwards): one read of the sequence serves both.
template <int MB, int TK, bool kVec, bool kAVec, bool kPair>
__global__ __launch_bounds__(kThreads) void proj_kernel(const ProjArgs g) {
  constexpr int kHalf = TK / 2;
  constexpr int kXPer = kVec ? TK * kPN / 4 / kThreads : TK * kPN / kThreads;
  typedef typename std::conditional<kVec, float4, float>::type XReg;
  __shared__ float xs[2][TK][kPN + 4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, jl = lane & 31, h = lane >> 5;
  const int64_t z = blockIdx.y, b = z / g.nk;
  const int k = int(z - b * g.nk);
  // x = column tile * row tiles + row tile: the row tiles of one column tile run together and
  // share the sequence chunk in the caches
  const int64_t ct = blockIdx.x / g.m_tiles;
  const int64_t n0 = ct * kPN, m0 = (int64_t(blockIdx.x) - ct * g.m_tiles) * (32 * MB);
  const bool rev = !kPair && g.rev_routes && k >= 2;
  const float* xb = ((k & 1) ? g.x1 : g.x0) + b * g.x_b + k * g.x_k;
  const int64_t mh = g.M / 2;  // rows per route when paired
  const float* wrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t i = m0 + 32 * mb + jl, ic = i < g.M ? i : g.M - 1;  // rows past M feed no output
    if (kPair)
      wrow[mb] = g.w + (ic < mh ? k : k + 2) * g.w_k + (ic < mh ? ic : ic - mh) * g.w_i;
    else
      wrow[mb] = g.w + k * g.w_k + ic * g.w_i;
  }
  // this thread's column of the sequence chunk and its first row
  const int xr0 = kVec ? (t >> 5) : (t >> 7), xstep = kVec ? 8 : 2;
  const int xcol = kVec ? 4 * (t & 31) : (t & 127);
  const int64_t cg = n0 + xcol;
  const bool colok = cg < g.L;  // vector path: L % 4 == 0, so a granule is all in or all out
  const int64_t gcol = colok ? (rev ? g.L - (kVec ? 4 : 1) - cg : cg) : 0;
  const float* xcolp = xb + gcol;
  const int64_t nch = (g.K + TK - 1) / TK;

  // Loads keep the raw words; the column reversal and the zeroing of rows past K happen when the
  // chunk is written to LDS, after the MFMAs (a select right after a load would make the compiler
  // wait for it there).  Weight values past K need no zeroing: they meet zero sequence rows.
  XReg xr[kXPer];
  bool xok[kXPer];
  float acur[MB][kHalf], anxt[MB][kHalf];
  auto load = [&](int64_t k0, float (&a)[MB][kHalf]) {
#pragma unroll
    for (int q = 0; q < kXPer; ++q) {
      const int64_t kk = k0 + xr0 + xstep * q;
      xok[q] = colok && kk < g.K;
      const float* p = xcolp + (kk < g.K ? kk : g.K - 1) * g.x_r;
      if constexpr (kVec)
        xr[q] = *reinterpret_cast<const float4*>(p);
      else
        xr[q] = *p;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (kAVec) {  // K % 4 == 0: a granule is all in or all out
#pragma unroll
        for (int q = 0; q < kHalf / 4; ++q) {
          const int64_t kk = k0 + h * kHalf + 4 * q;
          const float4 v = *reinterpret_cast<const float4*>(wrow[mb] + (kk < g.K ? kk : g.K - 4));
          a[mb][4 * q] = v.x;
          a[mb][4 * q + 1] = v.y;
          a[mb][4 * q + 2] = v.z;
          a[mb][4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int s = 0; s < kHalf; ++s) {
          const int64_t kk = k0 + h * kHalf + s;
          a[mb][s] = wrow[mb][(kk < g.K ? kk : g.K - 1) * g.w_kk];
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kXPer; ++q) {
      const float m = xok[q] ? 1.0f : 0.0f;
      if constexpr (kVec) {
        const float4 v = rev ? rev4(xr[q]) : xr[q];
        *reinterpret_cast<float4*>(&xs[buf][xr0 + xstep * q][xcol]) = make_float4(v.x * m, v.y * m, v.z * m, v.w * m);
      } else {
        xs[buf][xr0 + xstep * q][xcol] = xr[q] * m;
      }
    }
  };

  floatx16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx16{};
  load(0, acur);
  store(0);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    load((c + 1 < nch ? c + 1 : c) * TK, anxt);  // the last chunk reloads itself (unused)
    __builtin_amdgcn_sched_barrier(0);            // issue the loads before the MFMAs
    const int buf = int(c & 1);
#pragma unroll
    for (int s = 0; s < kHalf; ++s) {
      const float bv = xs[buf][h * kHalf + s][32 * wave + jl];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(acur[mb][s], bv, acc[mb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // use the new words only after the MFMAs
    store(buf ^ 1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int s = 0; s < kHalf; ++s) acur[mb][s] = anxt[mb][s];
    __syncthreads();
  }

  // accumulator v of row block mb is row m0 + 32 mb + 4 h + 8 (v / 4) + v % 4, column jc
  const int64_t jc = n0 + 32 * wave + jl;
  const bool jok = jc < g.L;
  float* cb = g.c + b * g.c_b + k * g.c_k + (jok ? jc : 0);
  float* cb2 = kPair ? g.c + b * g.c_b + (k + 2) * g.c_k + (jok ? g.L - 1 - jc : 0) : cb;  // route k + 2
  auto cptr = [&](int64_t i) {  // i < M
    if (kPair) return i < mh ? cb + i * g.c_r : cb2 + (i - mh) * g.c_r;
    return cb + i * g.c_r;
  };
  // two row blocks at a time: the previous values (when accumulating) are all loaded first
#pragma unroll
  for (int m2 = 0; m2 < MB; m2 += 2) {
    constexpr int kPairRows = MB > 1 ? 2 : 1;
    if (g.accumulate) {
      float old[kPairRows][16];
#pragma unroll
      for (int e = 0; e < kPairRows; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = m0 + 32 * (m2 + e) + 4 * h + 8 * (v / 4) + v % 4;
          old[e][v] = (m2 + e < MB) ? *cptr(jok && i < g.M ? i : 0) : 0.0f;
        }
#pragma unroll
      for (int e = 0; e < kPairRows; ++e)
        if (m2 + e < MB)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m2 + e][v] += old[e][v];
    }
#pragma unroll
    for (int e = 0; e < kPairRows; ++e)
      if (m2 + e < MB)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = m0 + 32 * (m2 + e) + 4 * h + 8 * (v / 4) + v % 4;
          if (jok && i < g.M) *cptr(i) = acc[m2 + e][v];
        }
  }
}

// kPair: routes k and k + 2 in one tile (A rows [0, M/2) of route k, rows [M/2, M) of route
// k + 2, which pairs its step l with step K - 1 - l of the same B): one read of B serves both.
template <int MBW, int NBW, bool kVec, bool kPair>
__global__ __launch_bounds__(kThreads) void wgrad_kernel(const WgradArgs g) {
  constexpr int kBlk = MBW * NBW;
  __shared__ float red[kBlk * 16][64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, jl = lane & 31, h = lane >> 5;
  const int64_t tiles_n = (g.N + 32 * NBW - 1) / (32 * NBW);
  const int64_t mt = blockIdx.x / tiles_n, nt = blockIdx.x - mt * tiles_n;
  const int64_t m0 = mt * (32 * MBW), n0 = nt * (32 * NBW);
  const int64_t sl = blockIdx.y / g.nk;
  const int k = int(blockIdx.y - sl * g.nk);
  const int64_t mh = g.M / 2;  // rows per route when paired
  const int64_t upi = (g.K + kWgradUnit - 1) / kWgradUnit, units = g.batch * upi;
  const int64_t per = (units + g.splits - 1) / g.splits;
  const int64_t u0 = sl * per, u1 = u0 + per < units ? u0 + per : units;
  // rows of this lane (clamped: an out-of-range row only feeds an output that is not written)
  const float* arow[MBW];
  const float* brow[NBW];
  bool arev[MBW];  // A row read backwards (per lane when paired)
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int64_t i = m0 + 32 * mb + jl, ic = i < g.M ? i : g.M - 1;
    const int ka = kPair ? (ic < mh ? k : k + 2) : k;
    arow[mb] = g.a + ka * g.a_k + (kPair && ic >= mh ? ic - mh : ic) * g.a_r;
    arev[mb] = g.rev_routes && ka >= 2;
  }
  const float* bk = (k & 1) ? g.b1 : g.b0;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int64_t j = n0 + 32 * nb + jl;
    brow[nb] = bk + k * g.b_k + (j < g.N ? j : g.N - 1) * g.b_r;
  }
  // lane's 8 steps of unit q: [l0, l0 + 8), l0 = 64 (q mod upi) + 16 wave + 8 h.  Loads keep the
  // raw words in memory order; the reversal and the zeroing of steps past K are applied when the
  // next unit's values become the current ones, after the MFMAs.
  typedef typename std::conditional<kVec, float4, float>::type Raw;
  constexpr int kR = kVec ? 2 : 8;
  Raw ra[MBW][kR], rb[NBW][kR];
  bool rok[kR];
  float acur[MBW][8], bcur[NBW][8];
  auto load = [&](int64_t bi, int64_t ui) {  // unit ui of image bi
    const int64_t l0 = ui * kWgradUnit + 16 * wave + 8 * h;
    const int64_t aoff = bi * g.a_b, boff = bi * g.b_b;
#pragma unroll
    for (int e = 0; e < kR; ++e) {
      const int64_t l = l0 + (kVec ? 4 : 1) * e;
      rok[e] = l < g.K;  // vector path: K % 4 == 0, so a granule is all in or all out
      const int64_t lc = l < g.K ? l : 0;
      const int64_t lr = g.K - (kVec ? 4 : 1) - lc;
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
        ra[mb][e] = *reinterpret_cast<const Raw*>(arow[mb] + aoff + (arev[mb] ? lr : lc));
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) rb[nb][e] = *reinterpret_cast<const Raw*>(brow[nb] + boff + lc);
    }
  };
  auto take = [&]() {
#pragma unroll
    for (int e = 0; e < kR; ++e) {
      const float m = rok[e] ? 1.0f : 0.0f;  // zeroing of B alone suffices: A is finite
      if constexpr (kVec) {
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
          const float4 v = arev[mb] ? rev4(ra[mb][e]) : ra[mb][e];
          acur[mb][4 * e] = v.x;
          acur[mb][4 * e + 1] = v.y;
          acur[mb][4 * e + 2] = v.z;
          acur[mb][4 * e + 3] = v.w;
        }
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const float4 v = rb[nb][e];
          bcur[nb][4 * e] = v.x * m;
          bcur[nb][4 * e + 1] = v.y * m;
          bcur[nb][4 * e + 2] = v.z * m;
          bcur[nb][4 * e + 3] = v.w * m;
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acur[mb][e] = ra[mb][e];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) bcur[nb][e] = rb[nb][e] * m;
      }
    }
  };

  floatx16 acc[MBW][NBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = floatx16{};
  const int64_t uf = u0 < units ? u0 : units - 1;
  int64_t bi = uf / upi, ui = uf - bi * upi;  // image and unit of the next load
  load(bi, ui);
  take();
  for (int64_t q = u0; q < u1; ++q) {
    if (q + 1 < u1 && ++ui == upi) {  // the last unit reloads itself (unused)
      ui = 0;
      ++bi;
    }
    load(bi, ui);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the MFMAs
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(acur[mb][s], bcur[nb][s], acc[mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // use the new words only after the MFMAs
    take();
  }

  // the four wavefronts' tiles summed through LDS (wave 3 first, wave 0 writes the result)
#pragma unroll
  for (int r = 3; r >= 1; --r) {
    if (wave == r) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float& e = red[(mb * NBW + nb) * 16 + v][lane];
            e = r == 3 ? acc[mb][nb][v] : e + acc[mb][nb][v];
          }
    }
    __syncthreads();
  }
  if (wave == 0) {
    // partial of route r: c + ((sl * routes + r) * rows + i) * N, routes = 2 nk when paired
    const int64_t rows = kPair ? mh : g.M, routes = kPair ? 2 * g.nk : g.nk;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = m0 + 32 * mb + 8 * (v / 4) + 4 * h + v % 4, j = n0 + 32 * nb + jl;
          const float val = acc[mb][nb][v] + red[(mb * NBW + nb) * 16 + v][lane];
          const int64_t r = kPair && i >= mh ? k + 2 : k, ir = kPair && i >= mh ? i - mh : i;
          if (i < g.M && j < g.N) g.c[((sl * routes + r) * rows + ir) * g.N + j] = val;
        }
  }
}

// out[i] = sum over the partials, in a fixed order: a workgroup takes 64 outputs; its four
// wavefronts sum the partials s = g, g + 4, g + 8, ... (g = wavefront) with eight loads in flight,
// and the four sums are added in the order g = 0, 1, 2, 3.  Partials past the end re-read a valid
// one and are weighted 0 (they are finite).
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* part, float* out, int64_t n, int64_t n_parts) {
  __shared__ float red[4][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t i = int64_t(blockIdx.x) * 64 + c, ic = i < n ? i : n - 1;
  constexpr int kInFlight = 8;
  float acc = 0.0f;
  for (int64_t s0 = g; s0 < n_parts; s0 += 4 * kInFlight) {
    float v[kInFlight];
#pragma unroll
    for (int e = 0; e < kInFlight; ++e) {
      const int64_t sp = s0 + 4 * e;
      v[e] = part[(sp < n_parts ? sp : g) * n + ic];
    }
#pragma unroll
    for (int e = 0; e < kInFlight; ++e) acc += v[e] * (s0 + 4 * e < n_parts ? 1.0f : 0.0f);
  }
  red[g][c] = acc;
  __syncthreads();
  if (g == 0 && i < n) out[i] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// 32 x 32 tile of one plane: fp32 copy in grid order and, through LDS, transposed
template <typename T>
__global__ __launch_bounds__(256) void cast_transpose_kernel(const T* x, float* xf, float* xfT, int64_t C, int H,
                                                             int W) {
  __shared__ float tile[32][33];
  const int tw = (W + 31) / 32, th = (H + 31) / 32;
  int64_t bid = blockIdx.x;
  const int t = int(bid % (int64_t(tw) * th));
  const int64_t plane = bid / (int64_t(tw) * th);
  const int h0 = (t / tw) * 32, w0 = (t % tw) * 32;
  const int64_t base = plane * int64_t(H) * W;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  // the four loads are issued unconditionally (clamped to the tile's first pixel) before any is
  // used: a load behind a branch is waited for at the branch's end
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = h0 + ty + 8 * r, w = w0 + tx;
    const bool in = h < H && w < W;
    v[r] = Elem<T>::load(x, base + (in ? int64_t(h) * W + w : int64_t(h0) * W + w0));
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = h0 + ty + 8 * r, w = w0 + tx;
    tile[ty + 8 * r][tx] = v[r];
    if (h < H && w < W) xf[base + int64_t(h) * W + w] = v[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int w = w0 + ty + 8 * r, h = h0 + tx;
    if (h < H && w < W) xfT[base + int64_t(w) * H + h] = tile[tx][ty + 8 * r];
  }
}

// One plane per workgroup (when the fp32 plane fits the LDS): 4 consecutive pixels per thread,
// four loads issued before any is used, the grid-order copy written as it is read, the
// column-major copy from the LDS tile.
template <typename T>
__global__ __launch_bounds__(256) void cast_transpose_plane_kernel(const T* x, float* xf, float* xfT, int H, int W) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* tile = reinterpret_cast<float*>(smem);  // [h][w], row stride W + 1
  const int L = H * W, ld = W + 1;
  const int64_t base = int64_t(blockIdx.x) * L;
  const T* xp = x + base;
  float* fp = xf + base;
  float* tp = xfT + base;
  constexpr int kStep = 4 * 256, kBatch = 4;
  for (int q0 = 4 * int(threadIdx.x); q0 < L; q0 += kStep * kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {  // past the plane: re-read quad 0, not stored
      const int q = q0 + kStep * e;
      v[e] = Elem<T>::load4(xp, q < L ? q : 0);
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int q = q0 + kStep * e;
      if (q >= L) break;
      *reinterpret_cast<float4*>(fp + q) = v[e];
      const float a4[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
      int h = q / W, w = q - h * W;  // one division; the quad's pixels follow along the row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[h * ld + w] = a4[j];
        if (++w == W) { w = 0; ++h; }
      }
    }
  }
  __syncthreads();
  for (int t = 4 * int(threadIdx.x); t < L; t += kStep) {  // t = w * H + h
    float a4[4];
    int w = t / H, h = t - w * H;  // one division; the quad's steps follow down the column
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a4[j] = tile[h * ld + w];
      if (++h == H) { h = 0; ++w; }
    }
    *reinterpret_cast<float4*>(tp + t) = make_float4(a4[0], a4[1], a4[2], a4[3]);
  }
}

}  // namespace

namespace {
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int MB, int TK, bool kVec>
void run_proj_v(const ProjArgs& g, dim3 grid, bool avec, hipStream_t s) {
  if (g.pair_routes)  // the launcher pairs only weights with 4-element loads
    proj_kernel<MB, TK, kVec, true, true><<<grid, dim3(kThreads), 0, s>>>(g);
  else if (avec)
    proj_kernel<MB, TK, kVec, true, false><<<grid, dim3(kThreads), 0, s>>>(g);
  else
    proj_kernel<MB, TK, kVec, false, false><<<grid, dim3(kThreads), 0, s>>>(g);
}
template <int MB>
hipError_t run_proj(const ProjArgs& g, dim3 grid, bool vec, bool avec, int tk, hipStream_t s) {
  if (tk == 8)
    vec ? run_proj_v<MB, 8, true>(g, grid, avec, s) : run_proj_v<MB, 8, false>(g, grid, avec, s);
  else
    vec ? run_proj_v<MB, 16, true>(g, grid, avec, s) : run_proj_v<MB, 16, false>(g, grid, avec, s);
  return hipGetLastError();
}
template <int MBW, int NBW>
hipError_t run_wgrad(const WgradArgs& g, dim3 grid, bool vec, hipStream_t s) {
  if (g.pair_routes)
    vec ? wgrad_kernel<MBW, NBW, true, true><<<grid, dim3(kThreads), 0, s>>>(g)
        : wgrad_kernel<MBW, NBW, false, true><<<grid, dim3(kThreads), 0, s>>>(g);
  else
    vec ? wgrad_kernel<MBW, NBW, true, false><<<grid, dim3(kThreads), 0, s>>>(g)
        : wgrad_kernel<MBW, NBW, false, false><<<grid, dim3(kThreads), 0, s>>>(g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_proj(const ProjArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.L <= 0 || g.batch <= 0) return hipSuccess;
  if (g.K <= 0 || g.nk <= 0) return hipErrorInvalidValue;
  // row blocks of 32 spread evenly over tiles of at most 4 blocks
  const int64_t blocks = (g.M + 31) / 32, tiles = (blocks + 3) / 4;
  const int mb = int((blocks + tiles - 1) / tiles);
  // chunk of 8 when it pads the contraction less than a chunk of 16
  const int tk = (g.K <= 8 || (g.K + 7) / 8 * 8 < (g.K + 15) / 16 * 16) ? 8 : 16;
  ProjArgs a = g;
  a.m_tiles = (g.M + 32 * mb - 1) / (32 * mb);
  const int64_t gx = (g.L + kPN - 1) / kPN * a.m_tiles;
  if (gx > int64_t(INT32_MAX)) return hipErrorInvalidValue;
  const bool vec = g.L % 4 == 0 && g.x_b % 4 == 0 && g.x_k % 4 == 0 && g.x_r % 4 == 0 && al16(g.x0) && al16(g.x1);
  const bool avec = g.w_kk == 1 && g.K % 4 == 0 && g.w_i % 4 == 0 && g.w_k % 4 == 0 && al16(g.w);
  if (g.pair_routes && (!avec || g.nk != 2 || g.M % 2 != 0 || g.x_k != 0)) return hipErrorInvalidValue;
  // grid y = (image, route) pairs, at most 65535 per launch: images in slices
  const int64_t per = 65535 / g.nk;
  for (int64_t b0 = 0; b0 < g.batch; b0 += per) {
    a.batch = g.batch - b0 < per ? g.batch - b0 : per;
    a.x0 = g.x0 + b0 * g.x_b;
    a.x1 = g.x1 + b0 * g.x_b;
    a.c = g.c + b0 * g.c_b;
    const dim3 grid{uint32_t(gx), uint32_t(a.batch * g.nk), 1u};
    hipError_t e;
    switch (mb) {
      case 1: e = run_proj<1>(a, grid, vec, avec, tk, s); break;
      case 2: e = run_proj<2>(a, grid, vec, avec, tk, s); break;
      case 3: e = run_proj<3>(a, grid, vec, avec, tk, s); break;
      default: e = run_proj<4>(a, grid, vec, avec, tk, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_wgrad(const WgradArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0 || g.batch <= 0 || g.nk <= 0 || g.splits <= 0) return hipErrorInvalidValue;
  if (g.pair_routes && (g.nk != 2 || g.M % 2 != 0 || g.b_k != 0)) return hipErrorInvalidValue;
  const int64_t mbn = (g.M + 31) / 32, nbn = (g.N + 31) / 32;
  const int mbw = mbn < 3 ? int(mbn) : 3;
  const int nmax = 6 / mbw;
  const int nbw = nbn < nmax ? int(nbn) : nmax;
  const int64_t tiles = ((g.M + 32 * mbw - 1) / (32 * mbw)) * ((g.N + 32 * nbw - 1) / (32 * nbw));
  const int64_t gy = g.splits * g.nk;
  if (tiles > int64_t(INT32_MAX) || gy > 65535) return hipErrorInvalidValue;
  const bool vec = g.K % 4 == 0 && g.a_b % 4 == 0 && g.a_k % 4 == 0 && g.a_r % 4 == 0 && g.b_b % 4 == 0 &&
                   g.b_k % 4 == 0 && g.b_r % 4 == 0 && al16(g.a) && al16(g.b0) && al16(g.b1);
  const dim3 grid{uint32_t(tiles), uint32_t(gy), 1u};
  switch (mbw * 8 + nbw) {
    case 8 + 1: return run_wgrad<1, 1>(g, grid, vec, s);
    case 8 + 2: return run_wgrad<1, 2>(g, grid, vec, s);
    case 8 + 3: return run_wgrad<1, 3>(g, grid, vec, s);
    case 8 + 4: return run_wgrad<1, 4>(g, grid, vec, s);
    case 8 + 5: return run_wgrad<1, 5>(g, grid, vec, s);
    case 8 + 6: return run_wgrad<1, 6>(g, grid, vec, s);
    case 16 + 1: return run_wgrad<2, 1>(g, grid, vec, s);
    case 16 + 2: return run_wgrad<2, 2>(g, grid, vec, s);
    case 16 + 3: return run_wgrad<2, 3>(g, grid, vec, s);
    case 24 + 1: return run_wgrad<3, 1>(g, grid, vec, s);
    default: return run_wgrad<3, 2>(g, grid, vec, s);
  }
}

hipError_t launch_sum_parts(const float* part, float* out, int64_t n, int64_t n_parts, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n_parts <= 0 || (n + 63) / 64 > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  sum_parts_kernel<<<dim3(uint32_t((n + 63) / 64)), dim3(256), 0, s>>>(part, out, n, n_parts);
  return hipGetLastError();
}

hipError_t launch_cast_transpose(const void* x, float* xf, float* xfT, int64_t batch, int64_t C, int64_t H,
                                 int64_t W, int dtype, hipStream_t s) {
  const size_t lds = size_t(H) * size_t(W + 1) * 4;
  const int64_t planes = batch * C;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  if (planes > 0 && (H * W) % 4 == 0 && lds <= 64 * 1024 && planes <= int64_t(UINT32_MAX) && al16(xf) && al16(xfT) &&
      (xa & (dtype == 0 ? 15 : 7)) == 0) {
    if (dtype == 0)
      cast_transpose_plane_kernel<float><<<dim3(uint32_t(planes)), dim3(256), lds, s>>>(
          static_cast<const float*>(x), xf, xfT, int(H), int(W));
    else
      cast_transpose_plane_kernel<bf16><<<dim3(uint32_t(planes)), dim3(256), lds, s>>>(
          static_cast<const bf16*>(x), xf, xfT, int(H), int(W));
    return hipGetLastError();
  }
  const int64_t blocks = batch * C * ((H + 31) / 32) * ((W + 31) / 32);
  if (blocks == 0) return hipSuccess;
  if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  if (dtype == 0)
    cast_transpose_kernel<float><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(static_cast<const float*>(x), xf, xfT,
                                                                             C, int(H), int(W));
  else
    cast_transpose_kernel<bf16><<<dim3(uint32_t(blocks)), dim3(256), 0, s>>>(static_cast<const bf16*>(x), xf, xfT, C,
                                                                            int(H), int(W));
  return hipGetLastError();
}

}  // namespace ss2d
