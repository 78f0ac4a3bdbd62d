// Selective scan S6, backward kernel (included by the scan_bwd_inst_*.hip instantiations).
//
// Gradient of the forward of `selective_scan_ref` ("Vision Mamba structure and principle"
// page, section 2), with the outputs of `SelectiveScanFn.backward` on the same page.  Per row,
// with a_t = exp(delta_t A), dy_t = dL/dy_t (dout * silu(z_t) when gated):
//   lambda_t = C_t dy_t + a_{t+1} lambda_{t+1}                   (adjoint of h_t, lambda_L = 0)
//   du_t     = delta_t <lambda_t, B_t> + D dy_t
//   ddelta_t = <lambda_t, A a_t h_{t-1} + B_t u_t>   (then * sigmoid(v_t) through the softplus)
//   dA      += lambda_t a_t h_{t-1} delta_t,  dB_t += lambda_t delta_t u_t,  dC_t += dy_t h_t,
//   dD      += dy_t u_t,                      dz_t  = dout_t (y_t + D u_t) silu'(z_t)
// (dB, dC summed over the channels of a group; dA, dD, ddelta_bias over batch and time).
//
// Mapping: as in the forward, one wavefront = channels of one (batch, group): one lane per channel
// for N <= 8, two adjacent lanes per channel (half of the states each) from N = 16 up.
// A row is walked backwards in 32-step tiles; a tile is cut into sub-intervals of kSub steps
// whose start states were checkpointed by the forward.  For each sub-interval the states are
// recomputed forwards into registers (kSub x NS floats), then the adjoint recurrence runs
// backwards over them.  The per-(step, state) terms of dB and dC are summed over the 64 lanes
// with a transpose-reduce (halving exchanges across lanes), so every lane ends up owning a
// slice of the (step, state) sums, which it writes once per 64-channel block; a small kernel
// adds the blocks.  When rows are few, the sequence is split into chunks: pass 1 runs the
// adjoint recurrence of each chunk from zero, a combine kernel chains the chunks, and pass 0
// starts every chunk from the true carried adjoint.
#pragma once
#include <type_traits>

#include "scan_common.h"

namespace ss2d {
namespace bwd_detail {
using namespace scan_detail;

// Cross-lane exchanges of the transpose-reduce below.
//
// v_permlane32_swap_b32 x, y exchanges lanes 32..63 of x with lanes 0..31 of y, and
// v_permlane16_swap_b32 x, y the odd 16-lane rows of x with the even rows of y.  Either way,
// afterwards the lane whose mask bit is clear holds (its own x, its partner's x) and the lane
// whose bit is set (its partner's y, its own y): x + y is the pair sum of the half the lane
// keeps, with no per-lane select.  The instructions are written as inline asm (the compiler
// builtin returns only one of the two registers here); a VALU result read by a swap needs two
// wait states, hence the s_nop ahead of each group of swaps.
template <int kMask>
__device__ __forceinline__ void swap_pairs4(float& x0, float& y0, float& x1, float& y1, float& x2, float& y2,
                                            float& x3, float& y3) {
  if (kMask == 32)
    asm volatile(
        "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
        "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7"
        : "+v"(x0), "+v"(y0), "+v"(x1), "+v"(y1), "+v"(x2), "+v"(y2), "+v"(x3), "+v"(y3));
  else
    asm volatile(
        "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
        "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7"
        : "+v"(x0), "+v"(y0), "+v"(x1), "+v"(y1), "+v"(x2), "+v"(y2), "+v"(x3), "+v"(y3));
}
template <int kMask>
__device__ __forceinline__ void swap_pair(float& x, float& y) {
  if (kMask == 32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}

// the value of lane (lane ^ m) within a 16-lane row, read by DPP; for m = 4 there is no xor
// pattern, so lanes with bit 2 clear read row_shl:4 (lane + 4) and the others row_shr:4
template <int kCtrl>
__device__ __forceinline__ float dpp_read(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
template <int m, bool kUpper>
__device__ __forceinline__ float row_partner(float x) {
  if (m == 8) return dpp_read<0x128>(x);            // row_ror:8
  if (m == 4) return dpp_read<kUpper ? 0x114 : 0x104>(x);  // row_shr:4 / row_shl:4
  if (m == 2) return dpp_read<0x4E>(x);             // quad_perm [2,3,0,1]
  return dpp_read<0xB1>(x);                         // quad_perm [1,0,3,2]
}

// One halving level at mask m over cnt values (cnt even): lane bit m set keeps the upper half.
template <int V, int m>
__device__ __forceinline__ void halve_level(float* v, int cnt, int lane) {
  const int half = cnt / 2;
  if (m >= 16) {
    int k = 0;
#pragma unroll
    for (int k4 = 0; k4 < V / 8; ++k4)
      if (4 * k4 + 3 < half) {
        swap_pairs4<m>(v[4 * k4], v[4 * k4 + half], v[4 * k4 + 1], v[4 * k4 + 1 + half], v[4 * k4 + 2],
                       v[4 * k4 + 2 + half], v[4 * k4 + 3], v[4 * k4 + 3 + half]);
        k = 4 * k4 + 4;
      }
#pragma unroll
    for (int j = 0; j < V / 2; ++j)
      if (j >= k && j < half) swap_pair<m>(v[j], v[j + half]);
#pragma unroll
    for (int j = 0; j < V / 2; ++j)
      if (j < half) v[j] = v[j] + v[j + half];
  } else {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      if (j < half) {
        const float lo = v[j] + row_partner<m, false>(v[j]);
        const float hi = v[j + half] + row_partner<m, true>(v[j + half]);
        v[j] = upper ? hi : lo;
      }
    }
  }
}

// Butterfly on one value at mask m: every lane gets the sum with lane (lane ^ m).
template <int m>
__device__ __forceinline__ void butterfly(float* v, int lane) {
  if (m >= 16) {
    float x = v[0], y = v[0];
    swap_pair<m>(x, y);
    v[0] = x + y;
  } else if (m == 4) {
    const float lo = row_partner<4, false>(v[0]), hi = row_partner<4, true>(v[0]);
    v[0] += (lane & 4) ? hi : lo;
  } else {
    v[0] += row_partner<m, false>(v[0]);
  }
}

// Sum V values per lane over the lanes that differ in the bits of the masks 32, 16, ..., kMinMask
// (kMinMask = 1: all 64 lanes; kMinMask = 2: the 32 lanes of the same parity).  Halving exchanges
// from the highest mask down while more than one value is left (lane bit m set: keep the upper
// half), then butterflies.  On return v[0 .. reduce_left) of lane l holds the totals of the
// original indices reduce_index<V, kMinMask>(l, r).
template <int V, int kMinMask, int m = 32>
__device__ __forceinline__ void lane_transpose_reduce_from(float* v, int lane, int cnt) {
  if (cnt > 1) {
    halve_level<V, m>(v, cnt, lane);
    cnt /= 2;
  } else {
    butterfly<m>(v, lane);
  }
  if constexpr (m / 2 >= kMinMask) lane_transpose_reduce_from<V, kMinMask, m / 2>(v, lane, cnt);
}
template <int V, int kMinMask>
__device__ __forceinline__ void lane_transpose_reduce(float* v, int lane) {
  lane_transpose_reduce_from<V, kMinMask, 32>(v, lane, V);
}

// values left per lane after lane_transpose_reduce, and the original index of v[r]
template <int V, int kMinMask>
constexpr int reduce_left() {
  int cnt = V;
  for (int m = 32; m >= kMinMask; m >>= 1)
    if (cnt > 1) cnt /= 2;
  return cnt;
}
template <int V, int kMinMask>
__device__ __forceinline__ int reduce_index(int lane, int r) {
  int cnt = V, idx = 0;
#pragma unroll
  for (int m = 32; m >= kMinMask; m >>= 1) {
    if (cnt > 1) {
      cnt /= 2;
      if (lane & m) idx += cnt;
    }
  }
  return idx + r;
}
// true for the one lane (per index and parity) that writes a total: no butterfly-mask bit set
template <int V, int kMinMask>
__device__ __forceinline__ bool reduce_writer(int lane) {
  int cnt = V, bits = 0;
#pragma unroll
  for (int m = 32; m >= kMinMask; m >>= 1) {
    if (cnt > 1)
      cnt /= 2;
    else
      bits |= m;
  }
  return (lane & bits) == 0;
}

// kSplit: lanes per channel (1 or 2); NSL = NS / kSplit states per lane.
// kMode: 0 = generic rows, dout in the I/O type; 1 = SS2D routes (u from the map and its
// transpose, fp32 dout planes); 2 = generic rows with an fp32 dout.
// TU: element type of u (T, or fp32 for an SS2D input computed in fp32 by the input front).
// kDtR: 0, or the padded rank (8, 16) of the dt_proj product that forms the raw delta in the
//       kernel (fp32 SS2D rows; dt rows staged per tile in LDS beside B and C).
template <typename T, int NS, int kSplit, int kMode, bool kVec, int kPass, typename TU, int kDtR = 0>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kPass == 0 && NS >= 16 ? 2 : 1)))
void scan_bwd_kernel(const ScanBwdParams p) {
  constexpr bool kSS2D = kMode == 1;
  using DT = typename std::conditional<kMode == 0, T, float>::type;  // type of dout rows
  constexpr int NSL = NS / kSplit;
  constexpr int kRows = kWave / kSplit;
  constexpr int S = (NS < 4) ? 4 : NS + 4;
  constexpr int kSub = ckpt_steps(NS);
  constexpr int kMinMask = kSplit;                                  // lanes of a channel differ in bit 0
  constexpr int kRW = 2 * NSL;  // per-step dB/dC values of a lane (its states' dB terms, then dC terms)
  constexpr int kLeft = reduce_left<kRW, kMinMask>();
  constexpr int kInner = (64 / NSL < kSub) ? 64 / NSL : kSub;       // steps whose states are held at once
  // Deferred outputs (two lanes per channel, 16 states, vector rows, fp32 or SS2D dout): a
  // sub-interval's du / ddelta stay in registers and its dB / dC sums in LDS until the next
  // sub-interval has consumed its loads; only then are they stored, as 16-byte pieces.  A load
  // that is waited for while stores are outstanding waits for the stores too (the wait counter
  // covers both, and they complete out of order), so stores issued at the end of a sub-interval
  // would be drained at the start of the next; issued after its loads, they drain while it
  // computes.
  constexpr bool kStage = kSplit == 2 && kVec && kPass == 0 && NS == 16 && kMode != 0 && kSub == 8 &&
                          kInner == kSub;
  constexpr int kRedStride = 2 * NS + 4;  // [step][dB states, dC states] (+4: no bank conflicts)
  __shared__ __align__(16) float sB[kTile * S];
  __shared__ __align__(16) float sC[kTile * S];
  __shared__ __align__(16) float sDt[kDtR > 0 ? kTile * kDtR : 4];
  __shared__ __align__(16) float sRed[kStage ? kSub * kRedStride : 4];

  const int lane = threadIdx.x;
  const int part = lane % kSplit;
  const int n0 = part * NSL;
  int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t dblk = bid % p.dblocks;
  bid /= p.dblocks;
  const int c = int(bid % p.n_chunks);
  bid /= p.n_chunks;
  const int64_t g = bid % p.G;
  const int64_t b = bid / p.G;
  const int64_t dg = dblk * kRows + lane / kSplit;
  const bool active = dg < p.per_group;
  const int64_t dl = active ? dg : 0;
  const int64_t d = g * p.per_group + dl;
  const int64_t row = b * p.dim + d;
  const int64_t L = p.L;
  const int N = p.N;
  const int nvalid = (N - n0 < 0) ? 0 : ((N - n0 > NSL) ? NSL : N - n0);

  const T* delta_row = kDtR > 0 ? nullptr : static_cast<const T*>(p.delta) + row * L;
  const TU* u_row;
  const DT* dout_row;
  bool rev = false;
  if (kSS2D) {
    const int64_t plane = (b * p.per_group + dl) * L;
    u_row = ((g & 1) ? static_cast<const TU*>(p.uT) : static_cast<const TU*>(p.u)) + plane;
    dout_row = ((g & 1) ? static_cast<const DT*>(p.doutT) : static_cast<const DT*>(p.dout)) + plane;
    rev = g >= 2;
  } else {
    u_row = static_cast<const TU*>(p.u) + row * L;
    dout_row = static_cast<const DT*>(p.dout) + row * L;
  }
  const bool has_z = !kSS2D && p.z != nullptr;
  const T* z_row = has_z ? static_cast<const T*>(p.z) + row * L : nullptr;
  const int64_t bcs = p.bc_stride ? p.bc_stride : N * L;
  const T* Bg = static_cast<const T*>(p.Bm) + (b * p.G + g) * bcs;
  const T* Cg = static_cast<const T*>(p.Cm) + (b * p.G + g) * bcs;
  const float* dtg = kDtR > 0 ? p.dt + (b * p.G + g) * bcs : nullptr;
  float wdt[kDtR > 0 ? kDtR : 1];
  if constexpr (kDtR > 0) load_dt_w<kDtR>(wdt, p.dt_w + d * p.dt_rank, p.dt_rank);

  float Acoef[NSL];
#pragma unroll
  for (int n = 0; n < NSL; ++n) Acoef[n] = (n < nvalid) ? p.A[d * N + n0 + n] : 0.0f;
  const float bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  const float Dd = p.Dskip ? p.Dskip[d] : 0.0f;

  const int64_t t_begin = int64_t(c) * p.chunk_len;
  const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;

  // Output offsets.  du of step t: du_base + (t - t % 4) * du_step + t % 4 (row layout: du_step 1;
  // blocked route layout: the 4-step group of the wavefront's consecutive channels is contiguous).
  // dB / dC partial sum of (state n, step t): bc_base + bc_off(n, t), rows of L steps or 4-step
  // blocks of all N states.
  const bool du_blk = kSS2D && p.du_blocked;
  const int64_t du_base = du_blk ? ((b * p.G + g) * (L / 4) * p.per_group + dl) * 4 : row * L;
  const int64_t du_step = du_blk ? p.per_group : 1;
  const bool bc_blk = p.bc_blocked != 0;
  const int64_t bc_base = ((dblk * p.batch + b) * p.G + g) * N * L;
  auto bc_off = [&](int n, int64_t t) { return bc_blk ? (t - (t & 3)) * N + 4 * n + (t & 3) : n * L + t; };

  // mu = a_{t+1} lambda_{t+1}: the adjoint flowing into step t from later steps
  float mu[NSL];
#pragma unroll
  for (int n = 0; n < NSL; ++n) mu[n] = 0.0f;
  if (kPass == 0 && p.n_chunks > 1) {
    const float* src = p.lam_carry + (row * p.n_chunks + c) * N + n0;
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      if (n < nvalid) mu[n] = src[n];
  }
  float dA_acc[NSL];
#pragma unroll
  for (int n = 0; n < NSL; ++n) dA_acc[n] = 0.0f;
  float dD_acc = 0.0f, dbias_acc = 0.0f, lam_sum = 0.0f;

  // deferred outputs of the last sub-interval (kStage): this lane's half of its channel's steps
  float pd_du[4], pd_dd[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pd_du[k] = pd_dd[k] = 0.0f;
  int64_t pd_s0 = -1;
  auto flush = [&]() {
    if constexpr (kStage) {
      if (pd_s0 < 0) return;
      const int64_t th = pd_s0 + 4 * part;  // this lane stores steps th .. th + 3 of its channel
      if (active && th < t_end) {
        Elem<T>::store4(static_cast<T*>(p.ddelta), row * L + th, make_float4(pd_dd[0], pd_dd[1], pd_dd[2], pd_dd[3]));
        const float4 v = make_float4(pd_du[0], pd_du[1], pd_du[2], pd_du[3]);
        if (kSS2D)
          if (du_blk)  // whole lines per store instruction: written past the caches
            store4_nt(static_cast<float*>(p.du) + du_base + th * du_step, v);
          else
            Elem<float>::store4(static_cast<float*>(p.du) + du_base, th * du_step, v);
        else
          Elem<T>::store4(static_cast<T*>(p.du), row * L + th, v);
      }
      // dB / dC block sums: lane pair (2 r, 2 r + 1) stores the two halves of row r (dB state r
      // for r < NS, else dC state r - NS)
      const int r = lane >> 1, h = lane & 1, n = r % NS;
      const int64_t t = pd_s0 + 4 * h;
      if (n < N && t < t_end) {
        float4 v;
        v.x = sRed[(4 * h) * kRedStride + r];
        v.y = sRed[(4 * h + 1) * kRedStride + r];
        v.z = sRed[(4 * h + 2) * kRedStride + r];
        v.w = sRed[(4 * h + 3) * kRedStride + r];
        float* dst = (r < NS) ? p.dB_part : p.dC_part;
        if (bc_blk)
          store4_nt(dst + bc_base + bc_off(n, t), v);
        else
          *reinterpret_cast<float4*>(dst + bc_base + bc_off(n, t)) = v;
      }
      pd_s0 = -1;
    }
  };

  auto pair_sum = [&](float x) {
    if (kSplit == 2)
      x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    return x;
  };

  // The range is walked backwards one sub-interval (kSub steps) at a time.  seg_body handles
  // the sub-interval starting at s0 (index q within the tile staged in LDS): dv, uv, gv, zv are
  // its delta, u, dout and z values and h0_of(n) the state before s0.
  auto seg_body = [&](int64_t s0, int q, const float* dv, const float* uv, const float* gv, const float* zv,
                      auto h0_of) {
      const int ns = int((t_end - s0 < kSub) ? (t_end - s0) : kSub);
      // per-step quantities (steps past the range and inactive lanes contribute nothing):
      // Lam = delta / ln 2 and sg = d delta / d raw (the sigmoid through the softplus, else 1)
      float lam[kSub], sg[kSub], dup[kSub], dy[kSub];
      auto lam_sg = [&](float v, float& l, float& g) {
        if (p.softplus) {
          softplus_sigmoid_log2<sizeof(T) == 4>(v * kLog2e, l, g);
        } else {
          l = v * kLog2e;
          g = 1.0f;
        }
      };
      if (kSplit == 2) {
        // the two lanes of a channel evaluate alternate steps and share the results by DPP
        // (quad_perm [0,0,2,2] from the even lane, [1,1,3,3] from the odd one)
#pragma unroll
        for (int i = 0; i < kSub; i += 2) {
          float l, g;
          lam_sg((part ? dv[i + 1] : dv[i]) + bias, l, g);
          lam[i] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, l), 0xA0, 0xF, 0xF, false));
          lam[i + 1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, l), 0xF5, 0xF, 0xF, false));
          sg[i] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, g), 0xA0, 0xF, 0xF, false));
          sg[i + 1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, g), 0xF5, 0xF, 0xF, false));
        }
      } else {
#pragma unroll
        for (int i = 0; i < kSub; ++i) lam_sg(dv[i] + bias, lam[i], sg[i]);
      }
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const float l = (i < ns) ? lam[i] : 0.0f;
        lam[i] = l;
        dup[i] = active ? l * uv[i] : 0.0f;
        float gy = gv[i];
        if (has_z) gy *= silu(zv[i]);
        dy[i] = (active && i < ns) ? gy : 0.0f;
      }
      if (kPass == 0) {
        // Start state of this sub-interval (its checkpoint).  The sub-interval is handled in
        // pieces of kInner steps, last piece first; for each piece the states are recomputed
        // forwards from the checkpoint and only the piece's own kInner x NSL states are kept.
        float h0[NSL];
#pragma unroll
        for (int n = 0; n < NSL; ++n) h0[n] = h0_of(n);
        if constexpr (kStage) {
          // the previous sub-interval's outputs, now that this one's loads are in: the empty asm
          // reads the loaded start state (so the loads are waited for here) and clobbers memory
          // (so the stores below are not moved above it, into the wait)
          asm volatile("" ::"v"(h0[0]), "v"(h0[NSL - 1]), "v"(lam[0]), "v"(dy[kSub - 1]) : "memory");
          flush();
        }
#pragma unroll
        for (int pc = kSub / kInner - 1; pc >= 0; --pc) {
          float hstart[NSL];
#pragma unroll
          for (int n = 0; n < NSL; ++n) hstart[n] = h0[n];
#pragma unroll
          for (int i = 0; i < pc * kInner; ++i) {
            const float* bt = sB + (q * kSub + i) * S + n0;
#pragma unroll
            for (int n = 0; n < NSL; ++n) hstart[n] = fmaf(fast_exp2(lam[i] * Acoef[n]), hstart[n], dup[i] * bt[n]);
          }
          float hs[kInner][NSL];
#pragma unroll
          for (int j = 0; j < kInner; ++j) {
            const int i = pc * kInner + j;
            const float* bt = sB + (q * kSub + i) * S + n0;
#pragma unroll
            for (int n = 0; n < NSL; ++n) {
              const float hp = (j == 0) ? hstart[n] : hs[j - 1][n];
              hs[j][n] = fmaf(fast_exp2(lam[i] * Acoef[n]), hp, dup[i] * bt[n]);
            }
          }
          float o_du[kInner], o_dd[kInner], o_dz[kInner];
          // adjoint recurrence backwards over the piece
#pragma unroll
          for (int j = kInner - 1; j >= 0; --j) {
            const int i = pc * kInner + j;
            const int idx = q * kSub + i;
            const float* bt = sB + idx * S + n0;
            const float* ct = sC + idx * S + n0;
            // recompute the decays here instead of keeping the forward's values alive
            float lr = lam[i];
            asm volatile("" : "+v"(lr));
            float sbl = 0.0f, ddt = 0.0f, yv = 0.0f;
            float red[kRW];
#pragma unroll
            for (int n = 0; n < NSL; ++n) {
              const float a = fast_exp2(lr * Acoef[n]);
              const float l = fmaf(ct[n], dy[i], mu[n]);
              const float hp = (j == 0) ? hstart[n] : hs[j - 1][n];
              const float gg = l * a * hp;
              dA_acc[n] = fmaf(gg, lam[i], dA_acc[n]);
              ddt = fmaf(gg, Acoef[n], ddt);
              sbl = fmaf(l, bt[n], sbl);
              red[n] = l * dup[i];              // dB term (times ln 2, applied when the blocks are summed)
              red[NSL + n] = dy[i] * hs[j][n];  // dC term
              if (has_z) yv = fmaf(ct[n], hs[j][n], yv);
              mu[n] = a * l;
            }
            // the two lanes of a channel hold complementary halves of the state sums
            sbl = pair_sum(sbl);
            ddt = pair_sum(ddt);
            if (has_z) yv = pair_sum(yv);
            o_du[j] = fmaf(lam[i], sbl, Dd * dy[i]);
            float dd = fmaf(uv[i] * kLog2e, sbl, ddt);  // ddelta (B was staged times ln 2)
            dd *= sg[i];
            dd = (i < ns && active) ? dd : 0.0f;
            o_dd[j] = dd;
            dbias_acc += dd;
            dD_acc = fmaf(dy[i], uv[i], dD_acc);
            if (has_z) {
              const float sz = sigmoid(zv[i]);
              o_dz[j] = gv[i] * fmaf(Dd, uv[i], yv) * sz * (1.0f + zv[i] * (1.0f - sz));
            }
            // dB / dC for (this step, this lane's states): sum over the channels of the block
            lane_transpose_reduce<kRW, kMinMask>(red, lane);
            if constexpr (kStage) {
              static_assert(kLeft == 1, "one block total per writer lane");
              if (i < ns && reduce_writer<kRW, kMinMask>(lane)) {
                const int e = reduce_index<kRW, kMinMask>(lane, 0);  // e < NSL: dB, else dC (state n0 + e % NSL)
                sRed[i * kRedStride + (e < NSL ? n0 + e : NS + n0 + e - NSL)] = red[0];
              }
            } else if (i < ns && reduce_writer<kRW, kMinMask>(lane)) {
              const int64_t t = s0 + i;
#pragma unroll
              for (int r = 0; r < kLeft; ++r) {
                const int e = reduce_index<kRW, kMinMask>(lane, r);  // e < NSL: dB, else dC (state n0 + e % NSL)
                const int n = e < NSL ? e : e - NSL;
                if (n < nvalid) {
                  float* dst = (e < NSL) ? p.dB_part : p.dC_part;
                  dst[bc_base + bc_off(n0 + n, t)] = red[r];
                }
              }
            }
          }
          if constexpr (kStage) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              pd_du[k] = part ? o_du[4 + k] : o_du[k];
              pd_dd[k] = part ? o_dd[4 + k] : o_dd[k];
            }
            pd_s0 = s0;
            if (has_z && active && part == 0)
              store_seg<T, kVec, kInner>(static_cast<T*>(p.dz) + row * L, o_dz, s0 + pc * kInner, t_end);
          } else if (active && part == 0) {
            const int64_t sp = s0 + pc * kInner;
            store_seg<T, kVec, kInner>(static_cast<T*>(p.ddelta) + row * L, o_dd, sp, t_end);
            if (kSS2D && du_blk) {
#pragma unroll
              for (int k = 0; k < kInner; ++k) {
                const int64_t t = sp + k;
                if (t < t_end) static_cast<float*>(p.du)[du_base + (t - (t & 3)) * du_step + (t & 3)] = o_du[k];
              }
            } else if (kSS2D)
              store_seg<float, kVec, kInner>(static_cast<float*>(p.du) + row * L, o_du, sp, t_end);
            else
              store_seg<T, kVec, kInner>(static_cast<T*>(p.du) + row * L, o_du, sp, t_end);
            if (has_z) store_seg<T, kVec, kInner>(static_cast<T*>(p.dz) + row * L, o_dz, sp, t_end);
          }
        }
      } else {
        // pass 1: adjoint recurrence of the chunk from zero (no states needed)
#pragma unroll
        for (int i = kSub - 1; i >= 0; --i) {
          const float* ct = sC + (q * kSub + i) * S + n0;
#pragma unroll
          for (int n = 0; n < NSL; ++n) {
            const float a = fast_exp2(lam[i] * Acoef[n]);
            mu[n] = a * fmaf(ct[n], dy[i], mu[n]);
          }
          lam_sum += lam[i];
        }
      }
  };

  auto stage_tile = [&](int64_t t0) {
    BCStage<T, NS, kVec> bc;
    bc.load(Bg, Cg, N, L, t0, t_end, lane);
    DtStage<(kDtR > 0 ? kDtR : 8), kVec> dts;
    if constexpr (kDtR > 0) dts.load(dtg, p.dt_rank, L, t0, t_end, lane);
    __syncthreads();  // the previous tile's LDS reads are complete
    bc.template store<S>(sB, sC, lane);
    if constexpr (kDtR > 0) dts.store(sDt, lane);
    __syncthreads();
  };
  // raw delta of the kSub steps of sub-interval q of the staged tile, formed from the dt rows;
  // with two lanes per channel a lane needs only the steps of its parity (both slots of a pair
  // get that value)
  auto fused_delta = [&](float* dv, int q) {
    if constexpr (kDtR > 0) {
      if (kSplit == 2) {
#pragma unroll
        for (int i = 0; i < kSub; i += 2) dv[i] = dv[i + 1] = dt_dot<kDtR>(sDt, wdt, q * kSub + i + part);
      } else {
#pragma unroll
        for (int i = 0; i < kSub; ++i) dv[i] = dt_dot<kDtR>(sDt, wdt, q * kSub + i);
      }
    }
  };
  constexpr int kSegsPerTile = kTile / kSub;
  if constexpr (kSplit == 1) {
    // One lane per channel (used when rows are few and the kernel is latency-bound): the row
    // segments and start state of the next sub-interval are loaded while this one computes.
    const int64_t n_segs = (t_end - t_begin + kSub - 1) / kSub;
    RowTile<T, kSub> nd, nz;
    RowTile<TU, kSub> nu;
    RowTile<DT, kSub> ng;
    float nh0[NSL];
    auto prefetch_seg = [&](int64_t s0) {
      if constexpr (kDtR == 0) load_row<T, kVec, kSub>(nd, delta_row, s0, t_end, L, false);
      // reversed rows stay in memory order here (reversed when used), and no load sits behind a
      // branch: either would make this prefetch wait for its own loads
      load_row<TU, kVec, kSub, true>(nu, u_row, s0, t_end, L, rev);
      load_row<DT, kVec, kSub, true>(ng, dout_row, s0, t_end, L, rev);
      if (has_z) load_row<T, kVec, kSub>(nz, z_row, s0, t_end, L, false);
      if (kPass == 0) {
        const float* ck = p.ckpt + ((s0 / kSub) * p.batch * p.dim + row) * N + n0;
#pragma unroll
        for (int n = 0; n < NSL; ++n) {
          const float v = ck[n < nvalid ? n : 0];
          nh0[n] = (n < nvalid) ? v : 0.0f;
        }
      }
    };
    if (n_segs > 0) prefetch_seg(t_begin + (n_segs - 1) * kSub);
#pragma unroll 1
    for (int64_t si = n_segs - 1; si >= 0; --si) {
      const int64_t s0 = t_begin + si * kSub;
      const int q = int(((s0 - t_begin) % kTile) / kSub);
      if (si == n_segs - 1 || q == kSegsPerTile - 1) stage_tile(s0 - int64_t(q) * kSub);
      const RowTile<T, kSub> cd = nd, cz = nz;
      RowTile<TU, kSub> cu = nu;
      RowTile<DT, kSub> cg = ng;
      if (kVec && rev) {  // vector loads leave a reversed row in memory order
        cu.reverse();
        cg.reverse();
      }
      float h0[NSL];
#pragma unroll
      for (int n = 0; n < NSL; ++n) h0[n] = nh0[n];
      if (si > 0) prefetch_seg(s0 - kSub);
      float dv[kSub], uv[kSub], gv[kSub], zv[kSub];
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        dv[i] = kDtR > 0 ? 0.0f : cd.get(i);
        uv[i] = cu.get(i);
        gv[i] = cg.get(i);
        zv[i] = has_z ? cz.get(i) : 0.0f;
      }
      fused_delta(dv, q);
      seg_body(s0, q, dv, uv, gv, zv, [&](int n) { return h0[n]; });
    }
  } else {
    // Two lanes per channel (full occupancy): each sub-interval loads its own values; the
    // other resident wavefronts cover the latency.  SS2D rows with vector loads (the register
    // budget allows it there) load the B/C words of the next tile (backwards) while this one
    // computes.
    constexpr bool kBCAhead = kSS2D && kVec && kDtR == 0 && kStage;
    // this lane's start states at checkpoint index s: ck_base + s * ck_step, 16-byte pieces
    // ck_stride apart (lane-major blocks when the forward stored them so: whole wavefronts of
    // rows, every state real; else row-major)
    const bool ck_lanes = ckpt_lane_major<NSL, kSplit>(N, p.per_group);
    const float* const ck_base = p.ckpt + ckpt_slot<NSL, kSplit>(ck_lanes, 0, 0, row, N, lane);
    const int64_t ck_step = p.batch * p.dim * N;
    const int ck_stride = ckpt_piece_stride(ck_lanes);
    const int64_t n_tiles = (t_end - t_begin + kTile - 1) / kTile;
    BCStage<T, NS, kVec> nbc;
    if (kBCAhead && n_tiles > 0) nbc.load(Bg, Cg, N, L, t_begin + (n_tiles - 1) * kTile, t_end, lane);
    for (int64_t jt = n_tiles - 1; jt >= 0; --jt) {
      const int64_t t0 = t_begin + jt * kTile;
      if constexpr (!kBCAhead) {
        stage_tile(t0);
      } else {
        __syncthreads();  // the previous tile's LDS reads are complete
        nbc.template store<S>(sB, sC, lane);
        __syncthreads();
        if (jt > 0) nbc.load(Bg, Cg, N, L, t0 - kTile, t_end, lane);
      }
#pragma unroll 1
      for (int q = kSegsPerTile - 1; q >= 0; --q) {
        const int64_t s0 = t0 + int64_t(q) * kSub;
        if (s0 >= t_end) continue;
        float dv[kSub], uv[kSub], gv[kSub], zv[kSub];
        if constexpr (kDtR > 0)
          fused_delta(dv, q);
        else
          load_seg<T, kVec, kSub>(dv, delta_row, s0, t_end, L, false);
        load_seg<TU, kVec, kSub>(uv, u_row, s0, t_end, L, rev);
        load_seg<DT, kVec, kSub>(gv, dout_row, s0, t_end, L, rev);
        if (has_z) load_seg<T, kVec, kSub>(zv, z_row, s0, t_end, L, false);
        const float* ck = ck_base + (s0 / kSub) * ck_step;
        // issued with the row loads so that one wait covers both: 16-byte loads when every state
        // is real (N == NS, the state rows are then 16-byte aligned pieces), else one load per
        // state (a state past N re-reads state n0, zeroed by a select)
        float ckv[NSL];
        if (NSL % 4 == 0 && N == NS) {
#pragma unroll
          for (int j = 0; j < NSL / 4; ++j) {
            const F4 c4 = __builtin_nontemporal_load(reinterpret_cast<const F4*>(ck + j * ck_stride));
            ckv[4 * j] = c4.x; ckv[4 * j + 1] = c4.y; ckv[4 * j + 2] = c4.z; ckv[4 * j + 3] = c4.w;
          }
        } else {
          // (volatile: kept apart from the vector loads, which the compiler would otherwise merge
          // with these into one set of per-state loads for both cases)
          const volatile float* ckq = ck;
#pragma unroll
          for (int n = 0; n < NSL; ++n) ckv[n] = ckq[n < nvalid ? n : 0];
        }
        seg_body(s0, q, dv, uv, gv, zv, [&](int n) { return (n < nvalid) ? ckv[n] : 0.0f; });
      }
    }
    flush();  // the last sub-interval's outputs
  }

  if (!active) return;
  if (kPass == 1) {
    float* dst = p.lam_carry + (row * p.n_chunks + c) * N + n0;  // local adjoint at the chunk start
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      if (n < nvalid) dst[n] = mu[n];
    if (part == 0) p.chunk_sum[row * p.n_chunks + c] = lam_sum;
  } else {
    float* dA = p.dA_part + (int64_t(c) * p.batch * p.dim + row) * N + n0;
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      if (n < nvalid) dA[n] = dA_acc[n];
    if (part == 0) {
      p.dD_part[int64_t(c) * p.batch * p.dim + row] = dD_acc;
      p.dbias_part[int64_t(c) * p.batch * p.dim + row] = dbias_acc;
    }
  }
}

template <typename T, int NS, int kSplit, int kMode, bool kVec, typename TU, int kDtR>
void launch_dt(const ScanBwdParams& p, dim3 grid, hipStream_t s) {
  if (p.pass == 1)
    scan_bwd_kernel<T, NS, kSplit, kMode, kVec, 1, TU, kDtR><<<grid, dim3(kWave), 0, s>>>(p);
  else
    scan_bwd_kernel<T, NS, kSplit, kMode, kVec, 0, TU, kDtR><<<grid, dim3(kWave), 0, s>>>(p);
}

template <typename T, int NS, int kSplit, int kMode, bool kVec, typename TU>
hipError_t launch_t(ScanBwdParams p, hipStream_t s) {
  p.dblocks = (p.per_group + kWave / kSplit - 1) / (kWave / kSplit);
  const int64_t blocks = p.batch * p.G * p.dblocks * p.n_chunks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if constexpr (kMode == 1 && std::is_same_v<T, float> && std::is_same_v<TU, float>) {
    if (p.dt_w) {
      if (p.dt_rank < 1 || p.dt_rank > 16 || p.dt == nullptr) return hipErrorInvalidValue;
      const dim3 grid{uint32_t(blocks)};
      if (p.dt_rank <= 8)
        launch_dt<T, NS, kSplit, kMode, kVec, TU, 8>(p, grid, s);
      else
        launch_dt<T, NS, kSplit, kMode, kVec, TU, 16>(p, grid, s);
      return hipGetLastError();
    }
  }
  if (p.dt_w) return hipErrorInvalidValue;
  if (p.pass == 1)
    scan_bwd_kernel<T, NS, kSplit, kMode, kVec, 1, TU><<<dim3(uint32_t(blocks)), dim3(kWave), 0, s>>>(p);
  else
    scan_bwd_kernel<T, NS, kSplit, kMode, kVec, 0, TU><<<dim3(uint32_t(blocks)), dim3(kWave), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bwd_detail

// Two lanes per channel from 16 states up (as in the forward).  TU != T (fp32 u with bf16 I/O)
// exists for the SS2D routes only.
template <typename T, int NS, typename TU>
hipError_t scan_bwd_launch(const ScanBwdParams& p, hipStream_t s) {
  using namespace bwd_detail;
  constexpr int kSplit = NS >= 16 ? 2 : 1;
  if (p.ss2d) return p.vec ? launch_t<T, NS, kSplit, 1, true, TU>(p, s) : launch_t<T, NS, kSplit, 1, false, TU>(p, s);
  if constexpr (!std::is_same_v<T, TU>) {
    return hipErrorInvalidValue;
  } else {
    if constexpr (sizeof(T) != 4) {  // for fp32 I/O an fp32 dout is the ordinary case
      if (p.dout_f32)
        return p.vec ? launch_t<T, NS, kSplit, 2, true, TU>(p, s) : launch_t<T, NS, kSplit, 2, false, TU>(p, s);
    }
    return p.vec ? launch_t<T, NS, kSplit, 0, true, TU>(p, s) : launch_t<T, NS, kSplit, 0, false, TU>(p, s);
  }
}

}  // namespace ss2d
