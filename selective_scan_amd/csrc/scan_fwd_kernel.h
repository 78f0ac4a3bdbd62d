// Selective scan S6, forward kernel (included by the scan_fwd_inst_*.hip instantiations).  Semantics: `selective_scan_ref` on the "Vision Mamba structure
// and principle" page (section 2):
//   delta_t = softplus(delta_raw_t + bias[d]);  h_t = exp(delta_t A[d,:]) h_{t-1} + delta_t B_t u_t
//   y_t = <C_t, h_t> + D[d] u_t ;  out_t = y_t * silu(z_t)
//
// Mapping on CDNA4: one wavefront = consecutive channels d of one (batch, group) pair, so that
// B_t / C_t (shared by the channels of a group) are wave-uniform: they are staged per 32-step
// tile in LDS as fp32 and read back as broadcasts.  Each channel's recurrence runs sequentially
// with its state in VGPRs: for N <= 8 one lane per channel (64 channels per wavefront); for
// N >= 16 two adjacent lanes per channel, each holding half of the states (32 channels per
// wavefront, twice the wavefronts), the two halves of y_t added with one DPP lane swap.  The
// loads of a channel's own row (delta, u, z) are 4-element vectors, prefetched one tile ahead.
//
// Arithmetic is carried in base 2: with Lam = log2(1 + 2^(v log2 e)) (so delta = ln2 * Lam),
//   exp(delta * A) = exp2(Lam * A)    and    delta * u * B = Lam * u * (ln2 * B),
// which costs one multiply and one v_exp_f32 per (step, state) for the decay; ln2 is folded
// into B while it is staged.
//
// When there are too few rows to fill the GPU, the sequence is split into chunks processed by
// different wavefronts: pass 1 runs each chunk from a zero state and keeps its end state and
// sum(Lam); a combine kernel chains the chunks (h_start(c+1) = exp2(A sum Lam_c) h_start(c)
// + h_end_local(c)); pass 0 reruns every chunk from its true start state and writes outputs.
#pragma once
#include <type_traits>

#include "scan_common.h"

namespace ss2d {
namespace fwd_detail {
using namespace scan_detail;

// kPass: 0 = outputs from the chunk-start state, 1 = chunk-local end state (chunked only),
//        2 = as 0 and also the state before every kSub-th step (checkpoints for the backward).
// kSplit: lanes per channel (1 or 2); NSL = NS / kSplit states per lane.
// kSoftplus: delta passes through softplus (else it is used as given).
// TU: element type of u (T, or fp32 for an SS2D input computed in fp32 by the input front).
// kDtR: 0, or the padded rank (8, 16) of the dt_proj product that forms the raw delta in the
//       kernel (fp32 SS2D rows): the group's dt rows are staged per tile in LDS beside B and C.
template <typename T, int NS, int kSplit, bool kSS2D, bool kVec, int kPassArg, bool kSoftplus, typename TU,
          int kDtR = 0>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(
    (kSS2D && kVec && sizeof(T) == 2 && sizeof(TU) == 2) ? fwd_waves_per_simd(NS, true) : 1)))
void scan_fwd_kernel(const ScanFwdParams p) {
  constexpr int kPass = kPassArg == 2 ? 0 : kPassArg;
  constexpr bool kStore = kPassArg == 2;
  constexpr int NSL = NS / kSplit;
  constexpr int kRows = kWave / kSplit;      // channels per wavefront
  constexpr int S = (NS < 4) ? 4 : NS + 4;  // LDS row stride (floats), keeps float4 alignment
  constexpr int kSub = ckpt_steps(NS);       // the state is checkpointed before every kSub-th step
  __shared__ __align__(16) float sB[kTile * S];
  __shared__ __align__(16) float sC[kTile * S];
  __shared__ __align__(16) float sDt[kDtR > 0 ? kTile * kDtR : 4];

  const int lane = threadIdx.x;
  const int part = lane % kSplit;            // which half of the states this lane holds
  const int n0 = part * NSL;                 // first state of this lane
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

  const T* delta_row = kDtR > 0 ? nullptr : static_cast<const T*>(p.delta) + row * L;
  const TU* u_row;
  bool rev = false;
  if (kSS2D) {
    const TU* src = (g & 1) ? static_cast<const TU*>(p.uT) : static_cast<const TU*>(p.u);
    u_row = src + (b * p.per_group + dl) * L;
    rev = g >= 2;
  } else {
    u_row = static_cast<const TU*>(p.u) + row * L;
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
  for (int n = 0; n < NSL; ++n) Acoef[n] = (n0 + n < N) ? p.A[d * N + n0 + n] : 0.0f;
  const int nvalid = (N - n0 < 0) ? 0 : ((N - n0 > NSL) ? NSL : N - n0);  // real states of this lane
  const float bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  const float bias_l2 = bias * kLog2e;
  const float Dd = (!kSS2D && p.Dskip) ? p.Dskip[d] : 0.0f;

  const int64_t t_begin = int64_t(c) * p.chunk_len;
  const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;
  // SS2D route outputs: the 4-step group starting at step tg (tg % 4 == 0) goes to
  // out + o_base + tg * o_step, in the row layout (row * L + tg) or in 4-step blocks
  // (((b G + g) (L / 4) + tg / 4) per_group + dl) * 4, where the wavefront's 32 or 64 consecutive
  // channels store one contiguous piece of whole lines per group
  const bool blocked = kSS2D && p.out_blocked;
  // checkpoint slots of the states kept for the backward: lane-major blocks when the wavefront's
  // rows are whole and every state is real (whole-line stores), else row-major
  // (this lane's slot at checkpoint index s: ck_base + s * ck_step, 16-byte pieces ck_stride apart)
  const bool ck_lanes = kStore && ckpt_lane_major<NSL, kSplit>(N, p.per_group);
  float* const ck_base = kStore ? p.ckpt + ckpt_slot<NSL, kSplit>(ck_lanes, 0, 0, row, N, lane) : nullptr;
  const int64_t ck_step = p.batch * p.dim * N;
  const int ck_stride = ckpt_piece_stride(ck_lanes);
  const int64_t o_base = blocked ? ((b * p.G + g) * (L / 4) * p.per_group + dl) * 4 : row * L;
  const int64_t o_step = blocked ? p.per_group : 1;

  float h[NSL];
#pragma unroll
  for (int n = 0; n < NSL; ++n) h[n] = 0.0f;
  if (kPass == 0 && p.n_chunks > 1 && c > 0) {
    const float* src = p.ckpt + ((t_begin / kSub) * p.batch * p.dim + row) * N + n0;
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      if (n < nvalid) h[n] = src[n];
  }
  float lam_sum = 0.0f;

  // Steps past the end of the range must leave the state unchanged: Lam = 0 (decay exp2(0) = 1,
  // zero input; B/C are zero-filled there).  With softplus, delta is padded with -inf there, whose
  // softplus is exactly 0; without it Lam is masked per step.
  const uint32_t dpad = kSoftplus ? (sizeof(T) == 2 ? 0xFF80u : 0xFF800000u) : 0u;
  // Row tiles in two register sets: tile k computes from set k % 2 while tile k + 1 is loaded
  // into the other (the loop body is instantiated once per set, so no copies between them).
  RowTile<T> rd[2], rz[2];
  RowTile<TU> ru[2];
  BCStage<T, NS, kVec> nbc;
  DtStage<(kDtR > 0 ? kDtR : 8), kVec> ndt;
  auto prefetch = [&](auto set, int64_t t) {
    constexpr int k = decltype(set)::value;
    if constexpr (kDtR > 0)
      ndt.load(dtg, p.dt_rank, L, t, t_end, lane);
    else
      load_row<T, kVec>(rd[k], delta_row, t, t_end, L, false, dpad);
    load_row<TU, kVec, kTile, true>(ru[k], u_row, t, t_end, L, rev);  // reversed when used
    if (has_z) load_row<T, kVec>(rz[k], z_row, t, t_end, L, false);
    nbc.load(Bg, Cg, N, L, t, t_end, lane);
  };
  if (t_begin < t_end) prefetch(std::integral_constant<int, 0>{}, t_begin);

  auto tile = [&](auto set, int64_t t0) {
    constexpr int k_set = decltype(set)::value;
    const RowTile<T>& cd = rd[k_set];
    RowTile<TU>& cu = ru[k_set];
    const RowTile<T>& cz = rz[k_set];
    __syncthreads();  // the previous tile's LDS reads are complete
    nbc.template store<S>(sB, sC, lane);
    if constexpr (kDtR > 0) ndt.store(sDt, lane);
    __syncthreads();
    const int64_t t1 = t0 + kTile;
    if (t1 < t_end) prefetch(std::integral_constant<int, 1 - k_set>{}, t1);
    // vector loads leave a reversed row in memory order (the scalar path indexes steps directly);
    // flipped here, after the next tile's loads are issued, so the wait covers only this tile's
    if (kVec && rev) cu.reverse();

    const int nt = int((t_end - t0 < kTile) ? (t_end - t0) : kTile);
    // One step's B (times ln 2) and C from LDS into one of two register buffers: the reads for
    // step i+1 go to buffer (i+1)&1 while step i computes from buffer i&1 (software pipelining
    // of the LDS latency; the buffer choice is resolved at compile time in the unrolled loop).
    float bufb[2][NSL], bufc[2][NSL];
    auto read_bc = [&](int i, float* nb, float* nc) {
      if (NSL >= 4) {
        const float4* bt = reinterpret_cast<const float4*>(sB + i * S + n0);
        const float4* ct = reinterpret_cast<const float4*>(sC + i * S + n0);
#pragma unroll
        for (int n4 = 0; n4 < NSL / 4; ++n4) {
          const float4 bb = bt[n4];
          nb[4 * n4] = bb.x; nb[4 * n4 + 1] = bb.y; nb[4 * n4 + 2] = bb.z; nb[4 * n4 + 3] = bb.w;
          if (kPass == 0) {
            const float4 cc = ct[n4];
            nc[4 * n4] = cc.x; nc[4 * n4 + 1] = cc.y; nc[4 * n4 + 2] = cc.z; nc[4 * n4 + 3] = cc.w;
          }
        }
      } else {
#pragma unroll
        for (int n = 0; n < NSL; ++n) {
          nb[n] = sB[i * S + n0 + n];
          if (kPass == 0) nc[n] = sC[i * S + n0 + n];
        }
      }
    };
    read_bc(0, bufb[0], bufc[0]);
    // The tile is processed in groups of 4 steps: per-step quantities, recurrence, epilogue and
    // a 4-element store per group, so that only a group's worth of temporaries is live.  Groups
    // wholly past the end of the range are skipped (a padded step leaves the state as it is).
#pragma unroll
    for (int g4 = 0; g4 < kTile / 4; ++g4) {
      if (4 * g4 >= nt) break;
      float lam[4], du[4], y[4];
      // raw delta of step i of the tile: loaded, or formed from the staged dt rows (-inf past
      // the end of the range, as the padded loads give)
      auto raw_delta = [&](const RowTile<T>& rt, int i, int lane_part) {
        if constexpr (kDtR > 0) {
          const int st = i + lane_part;
          return st < nt ? dt_dot<kDtR>(sDt, wdt, st) : -__builtin_huge_valf();
        } else {
          return kSplit == 2 ? rt.get_pair(i, lane_part) : rt.get(i);
        }
      };
      // Lam of step i (0 past the end of the range)
      auto step_lam = [&](float d, int i) {
        const float w = fmaf(d, kLog2e, bias_l2);
        if (kSoftplus) return softplus_log2<sizeof(T) == 4>(w);
        return (i < nt) ? w : 0.0f;
      };
      if (kSplit == 2) {
        // The two lanes of a channel share the softplus work: lane part p evaluates the steps of
        // parity p, and each result is broadcast to both lanes of the pair by DPP
        // (quad_perm [0,0,2,2] from the even lane, [1,1,3,3] from the odd one).
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int i = 4 * g4 + 2 * j;
          const float x = step_lam(raw_delta(cd, i, part), i + part);
          lam[2 * j] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xA0, 0xF, 0xF, false));
          lam[2 * j + 1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xF5, 0xF, 0xF, false));
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) lam[k] = step_lam(raw_delta(cd, 4 * g4 + k, 0), 4 * g4 + k);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) du[k] = lam[k] * cu.get(4 * g4 + k);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 4 * g4 + k;
        // compiler barrier: LDS reads are not hoisted by more than one step (that would keep
        // several steps' values live at once and exceed the register file)
        asm volatile("" ::: "memory");
        if (kStore && (i % kSub) == 0) {
          if (i < nt && active) {
            float* dst = ck_base + ((t0 + i) / kSub) * ck_step;
            if (NSL % 4 == 0 && nvalid == NSL)
              store_state_pieces<NSL>(dst, h, ck_stride);
            else
              store_state<NSL>(dst, h, nvalid);
          }
        }
        const float* cb = bufb[i & 1];
        const float* cc = bufc[i & 1];
        if (i + 1 < kTile) read_bc(i + 1, bufb[(i + 1) & 1], bufc[(i + 1) & 1]);
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NSL; ++n) {
          const float a = fast_exp2(lam[k] * Acoef[n]);
          h[n] = fmaf(a, h[n], du[k] * cb[n]);
          if (kPass == 0) acc = fmaf(cc[n], h[n], acc);
        }
        // the two lanes of a channel hold complementary halves of sum_n C h: add the partner's
        // (DPP quad_perm [1,0,3,2] swaps adjacent lanes)
        if (kPass == 0 && kSplit == 2)
          acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0xB1, 0xF,
                                                                       0xF, false));
        // pin the output here: otherwise the C*h sums are sunk into the (lane-conditional) store
        // block at the end of the group, which keeps every step's states live until then
        if (kPass == 0) asm volatile("" : "+v"(acc));
        y[k] = acc;
        if (kPass == 1) lam_sum += lam[k];
      }
      if (kPass == 0 && p.out != nullptr && active && part == 0) {
        const int64_t tg = t0 + 4 * g4;
        if (!kSS2D) {
          if (p.Dskip) {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = fmaf(Dd, cu.get(4 * g4 + k), y[k]);
          }
          if (has_z) {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] *= silu(cz.get(4 * g4 + k));
          }
          if (p.out_f32)
            store_seg<float, kVec, 4>(static_cast<float*>(p.out) + row * L, y, tg, t_end);
          else
            store_seg<T, kVec, 4>(static_cast<T*>(p.out) + row * L, y, tg, t_end);
        } else if constexpr (kVec) {
          // route outputs stay fp32 until the merge has added them: the result is rounded once.
          // The group is in range (groups at or past the end of the range exit the tile loop
          // above, and vector rows have L and the chunk ends a multiple of 4), so no bounds test.
          // (in 4-step blocks the wavefront's stores are whole lines: written past the caches)
          if (blocked)
            store4_nt(static_cast<float*>(p.out) + o_base + tg * o_step, make_float4(y[0], y[1], y[2], y[3]));
          else
            Elem<float>::store4(static_cast<float*>(p.out) + o_base, tg * o_step, make_float4(y[0], y[1], y[2], y[3]));
        } else {
          // element tg + k of the group at o_base + tg * o_step + k
          store_seg<float, kVec, 4>(static_cast<float*>(p.out) + o_base + tg * (o_step - 1), y, tg, t_end);
        }
      }
    }
    // the state is complete here: keeps the next tile's arithmetic from being interleaved with
    // this one's (which would hold both tiles' temporaries at once).  A scheduling barrier, not an
    // inline-asm pin of h: the compiler waits for every outstanding global store (vmcnt(0)) before
    // an inline-asm statement that redefines registers.
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kTile) {
    tile(std::integral_constant<int, 0>{}, t0);
    if (t0 + kTile < t_end) tile(std::integral_constant<int, 1>{}, t0 + kTile);
  }

  if (!active) return;
  if (kPass == 1) {
    if (t_end < L) store_state<NSL>(p.ckpt + ((t_end / kSub) * p.batch * p.dim + row) * N + n0, h, nvalid);
    if (part == 0) p.chunk_sum[row * p.n_chunks + c] = lam_sum;
  } else if (p.last_state && t_end == L) {
    store_state<NSL>(p.last_state + row * N + n0, h, nvalid);
  }
}

template <typename T, int NS, int kSplit, bool kSS2D, bool kVec, typename TU, int kDtR>
void launch_dt(const ScanFwdParams& p, dim3 grid, dim3 block, hipStream_t s) {
  if (p.softplus) {
    if (p.pass == 1)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 1, true, TU, kDtR><<<grid, block, 0, s>>>(p);
    else if (p.store_states)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 2, true, TU, kDtR><<<grid, block, 0, s>>>(p);
    else
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 0, true, TU, kDtR><<<grid, block, 0, s>>>(p);
  } else {
    if (p.pass == 1)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 1, false, TU, kDtR><<<grid, block, 0, s>>>(p);
    else if (p.store_states)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 2, false, TU, kDtR><<<grid, block, 0, s>>>(p);
    else
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 0, false, TU, kDtR><<<grid, block, 0, s>>>(p);
  }
}

template <typename T, int NS, int kSplit, bool kSS2D, bool kVec, typename TU>
hipError_t launch_t(ScanFwdParams p, hipStream_t s) {
  p.dblocks = (p.per_group + kWave / kSplit - 1) / (kWave / kSplit);
  const int64_t blocks = p.batch * p.G * p.dblocks * p.n_chunks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid{uint32_t(blocks)}, block{kWave};
  if constexpr (kSS2D && std::is_same_v<T, float> && std::is_same_v<TU, float>) {
    if (p.dt_w) {
      if (p.dt_rank < 1 || p.dt_rank > 16 || p.dt == nullptr) return hipErrorInvalidValue;
      if (p.dt_rank <= 8)
        launch_dt<T, NS, kSplit, kSS2D, kVec, TU, 8>(p, grid, block, s);
      else
        launch_dt<T, NS, kSplit, kSS2D, kVec, TU, 16>(p, grid, block, s);
      return hipGetLastError();
    }
  }
  if (p.dt_w) return hipErrorInvalidValue;
  if (p.softplus) {
    if (p.pass == 1)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 1, true, TU><<<grid, block, 0, s>>>(p);
    else if (p.store_states)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 2, true, TU><<<grid, block, 0, s>>>(p);
    else
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 0, true, TU><<<grid, block, 0, s>>>(p);
  } else {
    if (p.pass == 1)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 1, false, TU><<<grid, block, 0, s>>>(p);
    else if (p.store_states)
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 2, false, TU><<<grid, block, 0, s>>>(p);
    else
      scan_fwd_kernel<T, NS, kSplit, kSS2D, kVec, 0, false, TU><<<grid, block, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace fwd_detail

// Two lanes per channel from 16 states up (halves the per-lane state and doubles the
// wavefronts, which balances the stage-1 workload over the 1024 SIMDs).
// TU != T (fp32 u with bf16 I/O) exists for the SS2D routes only.
template <typename T, int NS, typename TU>
hipError_t scan_fwd_launch(const ScanFwdParams& p, hipStream_t s) {
  using namespace fwd_detail;
  constexpr int kSplit = NS >= 16 ? 2 : 1;
  if (p.ss2d) return p.vec ? launch_t<T, NS, kSplit, true, true, TU>(p, s) : launch_t<T, NS, kSplit, true, false, TU>(p, s);
  if constexpr (!std::is_same_v<T, TU>) {
    return hipErrorInvalidValue;
  } else {
    return p.vec ? launch_t<T, NS, kSplit, false, true, TU>(p, s) : launch_t<T, NS, kSplit, false, false, TU>(p, s);
  }
}

}  // namespace ss2d
