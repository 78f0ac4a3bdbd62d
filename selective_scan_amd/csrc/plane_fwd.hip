// SS2D forward in one kernel for small state sizes (N = 1, 2, 4): cross-scan, the four route
// scans and the cross-merge with its skip term and gate, one workgroup per (image, channel)
// plane.  Semantics as the three-stage path: routes after the SS2D section of the VMamba paper
// (Fig. 2; k = 0 row-major, 1 column-major, 2 / 3 the same from the last pixel back), the scan
// as `selective_scan_ref` on the "Vision Mamba structure and principle" page (section 2), the
// merge as the fp32 sum ((y0 + y1) + y2) + y3, plus (sum_k D[k]) x, times silu(z), rounded once.
//
// Why a second path: with one or a few states the recurrence costs little and the staged path
// is bound by moving the fp32 route outputs through HBM (16 bytes written and read per element,
// against 2-4 bytes of delta).  Here the plane stays in LDS: x is read once, each route's delta
// and B/C rows once, and only the gated result is written.
//
// Within a plane a route's L steps cannot go to one lane each (that would leave the GPU idle
// with one sequential row per workgroup), so each route is scanned in parallel over the 256
// threads: thread j owns kT consecutive steps of a segment of 256 kT steps.
//   pass 1: the thread's local end state h_loc (zero start) and S = sum of Lam over its steps;
//   combine: the pair (S, h_loc) is the affine map h -> 2^(A S) h + h_loc of its steps; the
//            maps compose as (S1, h1) then (S2, h2) = (S1 + S2, 2^(A S2) h1 + h2), an
//            associative operator, scanned over the lanes with shuffles and over the four
//            wavefronts through LDS, and applied to the state carried in from the last segment
//            (with one state the pair holds P = 2^(A S) instead of S: (P1 P2, P2 h1 + h2));
//   pass 2: the thread reruns its steps from its true start state and writes y.
// The per-step decays and inputs of pass 1 stay in registers for pass 2.  Arithmetic is in base
// 2 as in the route scans (Lam = log2(1 + 2^(v log2 e)), decay 2^(Lam A)); the state is carried
// as h / ln 2 (input Lam u B), so the route outputs and their sum are y / ln 2, scaled once per
// pixel before the skip term.
//
// LDS (four arrays of L): the column-major routes' outputs and the route sum in row-major order
// (fp32), and x in row-major and in column-major order (in the I/O type: bf16 words are exact,
// and 12 instead of 16 bytes per pixel let four planes share a CU), all in "chunk" layout (quad Q of each
// 16-quad group stored at Q ^ ((Q >> 4) & 3), so that a wavefront reading or writing 16-step
// chunks as 16-byte pieces hits distinct banks).  Routes 0 and 2 write their outputs into the
// sum directly (their steps are pixels, forwards or backwards); routes 1 and 3 write theirs in
// column-major order, which is then folded into the sum pixel by pixel (one add per pixel, in
// 4 x 4 blocks when H and W are multiples of 4).  Route order keeps the sum ((y0 + y1) + y2) + y3.
#include <type_traits>

#include "device_common.h"
#include "plane_fwd.h"

namespace ss2d {
namespace {

constexpr int kPT = 256;  // threads per plane
constexpr int kPWaves = kPT / kWave;
constexpr size_t kPlaneLdsMax = 63 * 1024;  // dynamic part; the wave totals are static

__device__ __forceinline__ int swz(int i) {
  const int q = i >> 2;
  return ((q ^ ((q >> 4) & 3)) << 2) | (i & 3);
}
// the layout permutes within groups of 64 words, so a step of 256 words maps to itself:
// swz(i + 256) == swz(i) + 256

// n (4 or 8) consecutive elements from a 16-byte aligned (8-byte for 4 bf16) position
template <typename T>
struct Ld;
template <>
struct Ld<float> {
  template <int n>
  __device__ __forceinline__ static void get(const float* p, int64_t i, float* v) {
#pragma unroll
    for (int q = 0; q < n / 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(p + i + 4 * q);
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  }
};
template <>
struct Ld<bf16> {
  template <int n>
  __device__ __forceinline__ static void get(const bf16* p, int64_t i, float* v) {
    if constexpr (n == 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(p + i);
      v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
      v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p + i);
      v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
    }
  }
};

// x in LDS in its own type: bf16 maps keep their 16-bit words (exact), fp32 maps fp32.  A quad is
// four consecutive elements of the chunk layout (16 or 8 bytes).
template <typename T>
struct XQ;
template <>
struct XQ<float> {
  using E = float;
  using Q = float4;
  __device__ __forceinline__ static float4 get(const E* p) { return *reinterpret_cast<const float4*>(p); }
  // the 4 x 4 block of rows r[0..3] transposed: column j of the block as a quad
  __device__ __forceinline__ static void transpose(const Q* r, Q* c) {
    c[0] = make_float4(r[0].x, r[1].x, r[2].x, r[3].x);
    c[1] = make_float4(r[0].y, r[1].y, r[2].y, r[3].y);
    c[2] = make_float4(r[0].z, r[1].z, r[2].z, r[3].z);
    c[3] = make_float4(r[0].w, r[1].w, r[2].w, r[3].w);
  }
};
template <>
struct XQ<bf16> {
  using E = uint16_t;
  using Q = uint2;
  __device__ __forceinline__ static float4 get(const E* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
  }
  // words (e0 | e1 << 16, e2 | e3 << 16) per row; column j takes the same half of two rows' words
  // (byte permute: selector 0x05040100 joins the low halves of its second and first operand,
  // 0x07060302 the high halves)
  __device__ __forceinline__ static void transpose(const Q* r, Q* c) {
    constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
    c[0] = make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, kLo), __builtin_amdgcn_perm(r[3].x, r[2].x, kLo));
    c[1] = make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, kHi), __builtin_amdgcn_perm(r[3].x, r[2].x, kHi));
    c[2] = make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, kLo), __builtin_amdgcn_perm(r[3].y, r[2].y, kLo));
    c[3] = make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, kHi), __builtin_amdgcn_perm(r[3].y, r[2].y, kHi));
  }
};

// (q, r) = divmod(i, n) along i = i0, i0 + s, i0 + 2s, ... (i0, s >= 0)
struct DivWalk {
  int q, r, dq, dr, n;
  __device__ DivWalk(int i0, int s, int n_) : n(n_) {
    q = i0 / n;
    r = i0 - q * n;
    dq = s / n;
    dr = s - dq * n;
  }
  __device__ void next() {
    q += dq;
    r += dr;
    if (r >= n) { r -= n; ++q; }
  }
};

template <typename T, int NS, bool kSoftplus>
__global__ __launch_bounds__(kPT) void plane_fwd_kernel(const PlaneFwdArgs a) {
  constexpr int kT = 16 / NS;          // steps per thread and segment
  constexpr int kG = kT < 8 ? kT : 8;  // elements per global load
  constexpr int kSeg = kPT * kT;
  extern __shared__ __align__(16) float smem[];
  using XE = typename XQ<T>::E;
  using XQd = typename XQ<T>::Q;
  const int H = int(a.H), Wd = int(a.W), L = H * Wd;
  const int Ls = (L + 15) & ~15;
  float* syb = smem;                            // route 1 / 3 outputs, column-major, chunk layout
  float* sacc = syb + Ls;                       // the route sum, row-major, chunk layout
  XE* sxR = reinterpret_cast<XE*>(sacc + Ls);  // x, row-major (routes 0, 2), chunk layout
  XE* sxT = sxR + Ls;                          // x, column-major (routes 1, 3), chunk layout
  __shared__ float wtot[2][kPWaves][NS + 1];

  const int tid = int(threadIdx.x), lane = tid % kWave, wv = tid / kWave;
  const int64_t plane = xcd_remap(blockIdx.x, gridDim.x);  // b * dim + d
  const int64_t b = plane / a.dim, d = plane - b * a.dim;

  {  // x -> sxR (quads copied as they are)
    const XE* xg = reinterpret_cast<const XE*>(static_cast<const T*>(a.x) + plane * L);
    for (int p = 4 * tid; p < L; p += 4 * kPT)
      *reinterpret_cast<XQd*>(sxR + swz(p)) = *reinterpret_cast<const XQd*>(xg + p);
  }
  __syncthreads();
  // With H and W multiples of 4 the plane is cut into 4 x 4 blocks: a block's four row quads
  // (row-major, 16 bytes each) are its four column quads transposed (column-major index
  // w H + h, also 16 bytes each), so a thread moves a block with eight 16-byte LDS accesses.
  // Other shapes go element by element.
  const bool blocks4 = (H & 3) == 0 && (Wd & 3) == 0;
  const int Wq = Wd >> 2, nblk = (H >> 2) * Wq;
  if (blocks4) {  // block (bh, bw): rows 4 bh .. 4 bh + 3, columns 4 bw .. 4 bw + 3
    for (int blk = tid; blk < nblk; blk += kPT) {
      const int bh = blk / Wq, h = 4 * bh, w = 4 * (blk - bh * Wq);
      XQd r[4], cq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = *reinterpret_cast<const XQd*>(sxR + swz((h + i) * Wd + w));
      XQ<T>::transpose(r, cq);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<XQd*>(sxT + swz((w + j) * H + h)) = cq[j];
    }
  } else {  // column-major index t is pixel (h, w) = (t % H, t / H)
    DivWalk dw(tid, kPT, H);
    for (int t = tid, st = swz(tid); t < L; t += kPT, st += kPT, dw.next()) sxT[st] = sxR[swz(dw.r * Wd + dw.q)];
  }
  // (route 0's segment barrier orders these writes before route 1 reads them)

  int it = 0;  // segments so far: selects the wave-total buffer
  auto route = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr bool kCol = (k & 1) != 0, kRev = k >= 2;
    const XE* su = kCol ? sxT : sxR;
    const T* dr = static_cast<const T*>(a.delta) + ((b * 4 + k) * a.dim + d) * L;
    const T* Br = static_cast<const T*>(a.Bm) + (b * 4 + k) * NS * int64_t(L);
    const T* Cr = static_cast<const T*>(a.Cm) + (b * 4 + k) * NS * int64_t(L);
    float Ak[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) Ak[n] = a.A[(k * a.dim + d) * NS + n];
    const float bias_l2 = a.delta_bias ? a.delta_bias[k * a.dim + d] * kLog2e : 0.0f;
    float carry[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) carry[n] = 0.0f;

    for (int s0 = 0; s0 < L; s0 += kSeg) {
      const int t0 = s0 + tid * kT;
      // per step: Lam, the decays 2^(Lam A), the inputs Lam u B, and C (kept for pass 2)
      float lam[kT], aa[kT][NS], bu[kT][NS], cc[kT][NS];
      {
        float dv[kT], bv[NS][kT], uv[kT];
#pragma unroll
        for (int g = 0; g < kT / kG; ++g) {  // a group is wholly inside or past the row (L % 8 == 0)
          const int t = t0 + g * kG, tc = t < L ? t : 0;
          Ld<T>::template get<kG>(dr, tc, dv + g * kG);
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            Ld<T>::template get<kG>(Br + n * int64_t(L), tc, bv[n] + g * kG);
            float cv[kG];
            Ld<T>::template get<kG>(Cr + n * int64_t(L), tc, cv);
#pragma unroll
            for (int e = 0; e < kG; ++e) cc[g * kG + e][n] = cv[e];
          }
        }
#pragma unroll
        for (int q = 0; q < kT / 4; ++q) {  // u: x at the pixels of steps t .. t+3
          const int t = t0 + 4 * q;
          const int ti = t < L ? (kRev ? L - 4 - t : t) : 0;
          const float4 f = XQ<T>::get(su + swz(ti));
          if (kRev) {
            uv[4 * q] = f.w; uv[4 * q + 1] = f.z; uv[4 * q + 2] = f.y; uv[4 * q + 3] = f.x;
          } else {
            uv[4 * q] = f.x; uv[4 * q + 1] = f.y; uv[4 * q + 2] = f.z; uv[4 * q + 3] = f.w;
          }
        }
#pragma unroll
        for (int i = 0; i < kT; ++i) {
          // steps past the row (clamped loads of real data) feed only lanes after the row's
          // end, whose results are never stored nor carried into another segment
          const float w = fmaf(dv[i], kLog2e, bias_l2);
          const float l = kSoftplus ? softplus_log2<sizeof(T) == 4>(w) : w;
          lam[i] = l;
          const float du = l * uv[i];
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            aa[i][n] = fast_exp2(l * Ak[n]);
            bu[i][n] = du * bv[n][i];
          }
        }
      }
      // pass 1: this thread's map (S, h_loc).  With one state the map carries its decay
      // P = 2^(A S) itself, the product of its steps' decays: two maps then compose with a
      // multiply and an FMA, no exp.  With more states S is shared by all of them.
      constexpr bool kProd = NS == 1;
      auto decay = [&](int n, float s) { return kProd ? s : fast_exp2(Ak[n] * s); };
      float S = kProd ? 1.0f : 0.0f, hl[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) hl[n] = 0.0f;
#pragma unroll
      for (int i = 0; i < kT; ++i) {
        S = kProd ? S * aa[i][0] : S + lam[i];
#pragma unroll
        for (int n = 0; n < NS; ++n) hl[n] = fmaf(aa[i][n], hl[n], bu[i][n]);
      }
      // inclusive scan of the maps over the wavefront's lanes
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float So = __shfl_up(S, off);
        float ho[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) ho[n] = __shfl_up(hl[n], off);
        if (lane >= off) {
#pragma unroll
          for (int n = 0; n < NS; ++n) hl[n] = fmaf(decay(n, S), ho[n], hl[n]);
          S = kProd ? S * So : S + So;
        }
      }
      float Se = __shfl_up(S, 1), he[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) he[n] = __shfl_up(hl[n], 1);
      if (lane == 0) {
        Se = kProd ? 1.0f : 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) he[n] = 0.0f;
      }
      float* wt = &wtot[it & 1][0][0];
      if (lane == kWave - 1) {
        wt[wv * (NS + 1)] = S;
#pragma unroll
        for (int n = 0; n < NS; ++n) wt[wv * (NS + 1) + 1 + n] = hl[n];
      }
      __syncthreads();
      ++it;
      // the carried state through the earlier wavefronts, then the earlier lanes of this one;
      // the state through all four is the next segment's carry
      float st[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) st[n] = carry[n];
#pragma unroll
      for (int w2 = 0; w2 < kPWaves; ++w2) {
        const float Sw = wt[w2 * (NS + 1)];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          carry[n] = fmaf(decay(n, Sw), carry[n], wt[w2 * (NS + 1) + 1 + n]);
          if (w2 + 1 == wv) st[n] = carry[n];
        }
      }
      float h[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) h[n] = fmaf(decay(n, Se), st[n], he[n]);
      // pass 2: outputs from the true start state
      float y[kT];
#pragma unroll
      for (int i = 0; i < kT; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          h[n] = fmaf(aa[i][n], h[n], bu[i][n]);
          acc = fmaf(cc[i][n], h[n], acc);
        }
        y[i] = acc;
      }
      // steps t .. t+3 are pixels (routes 0, 2) / column-major indices (1, 3) idx .. idx+3,
      // forwards, or idx+3 .. idx backwards (routes 2, 3)
#pragma unroll
      for (int q = 0; q < kT / 4; ++q) {
        const int t = t0 + 4 * q;
        if (t < L) {
          const float4 v = kRev ? make_float4(y[4 * q + 3], y[4 * q + 2], y[4 * q + 1], y[4 * q])
                                : make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
          float4* dst = reinterpret_cast<float4*>((kCol ? syb : sacc) + swz(kRev ? L - 4 - t : t));
          if (k == 2) {  // the sum holds y0 + y1 here
            const float4 o = *dst;
            *dst = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
          } else {
            *dst = v;
          }
        }
      }
    }
    if constexpr (kCol) {  // fold into the sum, pixel p = (h, w) <- column-major index w H + h
      __syncthreads();
      if (blocks4) {  // one add per pixel, as below: the column quads of a block, transposed
        for (int blk = tid; blk < nblk; blk += kPT) {
          const int bh = blk / Wq, h = 4 * bh, w = 4 * (blk - bh * Wq);
          float4 c[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const float4*>(syb + swz((w + j) * H + h));
          const float cr[4][4] = {{c[0].x, c[1].x, c[2].x, c[3].x},
                                  {c[0].y, c[1].y, c[2].y, c[3].y},
                                  {c[0].z, c[1].z, c[2].z, c[3].z},
                                  {c[0].w, c[1].w, c[2].w, c[3].w}};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float4* dst = reinterpret_cast<float4*>(sacc + swz((h + i) * Wd + w));
            const float4 o = *dst;
            *dst = make_float4(o.x + cr[i][0], o.y + cr[i][1], o.z + cr[i][2], o.w + cr[i][3]);
          }
        }
      } else {
        DivWalk dw(tid, kPT, Wd);
        for (int p = tid, sp = swz(tid); p < L; p += kPT, sp += kPT, dw.next()) sacc[sp] += syb[swz(dw.r * H + dw.q)];
      }
      // (the next route's segment barrier orders this fold before the sum or syb is rewritten)
    }
  };
  route(std::integral_constant<int, 0>{});
  route(std::integral_constant<int, 1>{});
  route(std::integral_constant<int, 2>{});
  route(std::integral_constant<int, 3>{});
  __syncthreads();

  // skip term, gate, one rounding
  float dsum = 0.0f;
  if (a.Dskip) dsum = ((a.Dskip[d] + a.Dskip[a.dim + d]) + a.Dskip[2 * a.dim + d]) + a.Dskip[3 * a.dim + d];
  const T* zg = a.z ? static_cast<const T*>(a.z) + plane * L : nullptr;
  T* og = static_cast<T*>(a.out) + plane * L;
  for (int p = 4 * tid; p < L; p += 4 * kPT) {
    float zv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (zg) Ld<T>::template get<4>(zg, p, zv);
    const float4 xq = XQ<T>::get(sxR + swz(p));
    const float4 sq = *reinterpret_cast<const float4*>(sacc + swz(p));
    const float xv[4] = {xq.x, xq.y, xq.z, xq.w};
    float v[4] = {sq.x * kLn2, sq.y * kLn2, sq.z * kLn2, sq.w * kLn2};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (a.Dskip) v[e] = fmaf(dsum, xv[e], v[e]);
      if (zg) v[e] *= silu(zv[e]);
    }
    Elem<T>::store4(og, p, make_float4(v[0], v[1], v[2], v[3]));
  }
}

// LDS a plane may take: the rule that admits a plane to the single kernel (16 bytes per pixel)
size_t plane_lds_bytes(int64_t H, int64_t W) {
  const int64_t Ls = (H * W + 15) / 16 * 16;
  return size_t(4 * Ls) * sizeof(float);
}
// what a launch allocates: two fp32 arrays, and the two copies of x in the I/O type
template <typename T>
size_t plane_lds_alloc(int64_t H, int64_t W) {
  const int64_t Ls = (H * W + 15) / 16 * 16;
  return size_t(2 * Ls) * (sizeof(float) + sizeof(typename XQ<T>::E));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename T, int NS>
void launch_t(const PlaneFwdArgs& a, hipStream_t s) {
  const dim3 grid{uint32_t(a.batch * a.dim)}, block{kPT};
  const size_t lds = plane_lds_alloc<T>(a.H, a.W);
  if (a.softplus)
    plane_fwd_kernel<T, NS, true><<<grid, block, lds, s>>>(a);
  else
    plane_fwd_kernel<T, NS, false><<<grid, block, lds, s>>>(a);
}

template <typename T>
void launch_n(const PlaneFwdArgs& a, hipStream_t s) {
  if (a.N == 1)
    launch_t<T, 1>(a, s);
  else if (a.N == 2)
    launch_t<T, 2>(a, s);
  else
    launch_t<T, 4>(a, s);
}

}  // namespace

bool plane_fwd_supported(const PlaneFwdArgs& a) {
  if (a.N != 1 && a.N != 2 && a.N != 4) return false;
  if (a.dtype != 0 && a.dtype != 1) return false;
  if (a.H < 1 || a.W < 1 || a.H > 4096 || a.W > 4096) return false;
  const int64_t L = a.H * a.W;
  if (L % 8 != 0 || plane_lds_bytes(a.H, a.W) > kPlaneLdsMax) return false;
  if (a.batch < 1 || a.dim < 1 || a.batch * a.dim > 0x7fffffffLL) return false;
  for (const void* p : {a.x, a.delta, a.Bm, a.Cm, a.z, static_cast<const void*>(a.out)})
    if (!aligned16(p)) return false;
  return a.x && a.delta && a.Bm && a.Cm && a.A && a.out;
}

hipError_t launch_plane_fwd(const PlaneFwdArgs& a, hipStream_t s) {
  if (!plane_fwd_supported(a)) return hipErrorInvalidValue;
  if (a.dtype == 0)
    launch_n<float>(a, s);
  else
    launch_n<bf16>(a, s);
  return hipGetLastError();
}

}  // namespace ss2d
