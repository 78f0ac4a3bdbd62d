// Helpers shared by the selective-scan forward and backward kernels: per-lane row tiles,
// B/C staging into LDS, output and state stores.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ss2d {
namespace scan_detail {

// Per-lane copy of kLen consecutive elements of one row (a tile by default), kept in the storage
// format until used.
template <typename T, int kLen = kTile>
struct RowTile;
template <int kLen>
struct RowTile<float, kLen> {
  float4 v[(kLen + 3) / 4];
  __device__ __forceinline__ float get(int i) const {
    const float4 q = v[i / 4];
    return (i % 4 == 0) ? q.x : (i % 4 == 1) ? q.y : (i % 4 == 2) ? q.z : q.w;
  }
  // element i + sel of an even i, sel in {0, 1} chosen per lane
  __device__ __forceinline__ float get_pair(int i, int sel) const { return sel ? get(i + 1) : get(i); }
  // every element set to the value with bit pattern `bits`
  __device__ __forceinline__ void fill(uint32_t bits) {
    const float f = __uint_as_float(bits);
#pragma unroll
    for (int j = 0; j < (kLen + 3) / 4; ++j) v[j] = make_float4(f, f, f, f);
  }
  __device__ __forceinline__ void load_vec(const float* p, int j) { v[j] = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void set(int i, float x) {
    float4& q = v[i / 4];
    if (i % 4 == 0) q.x = x; else if (i % 4 == 1) q.y = x; else if (i % 4 == 2) q.z = x; else q.w = x;
  }
  __device__ __forceinline__ void reverse() {
    float4 r[(kLen + 3) / 4];
#pragma unroll
    for (int j = 0; j < kLen / 4; ++j) {
      const float4 q = v[kLen / 4 - 1 - j];
      r[j] = make_float4(q.w, q.z, q.y, q.x);
    }
#pragma unroll
    for (int j = 0; j < kLen / 4; ++j) v[j] = r[j];
  }
};
template <int kLen>
struct RowTile<bf16, kLen> {
  uint2 v[(kLen + 3) / 4];
  __device__ __forceinline__ float get(int i) const {
    const uint2 q = v[i / 4];
    const uint32_t w = ((i % 4) < 2) ? q.x : q.y;
    return (i % 2 == 0) ? bf16lo(w) : bf16hi(w);
  }
  // element i + sel of an even i, sel in {0, 1} chosen per lane: both halves of one dword, the
  // wanted one moved to the top and the other cleared by one byte permute with a per-lane
  // selector (bytes 1, 0 or 3, 2 of the dword into bytes 3, 2; selector byte 0x0c gives zero)
  __device__ __forceinline__ float get_pair(int i, int sel) const {
    const uint2 q = v[i / 4];
    const uint32_t w = ((i % 4) < 2) ? q.x : q.y;
    return __uint_as_float(__builtin_amdgcn_perm(w, w, sel ? 0x03020c0cu : 0x01000c0cu));
  }
  // every element set to the bf16 value with bit pattern `bits` (low 16 bits)
  __device__ __forceinline__ void fill(uint32_t bits) {
    const uint32_t w = (bits & 0xffffu) * 0x10001u;
#pragma unroll
    for (int j = 0; j < (kLen + 3) / 4; ++j) v[j] = make_uint2(w, w);
  }
  __device__ __forceinline__ void load_vec(const bf16* p, int j) { v[j] = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void set(int i, uint16_t bits) {
    uint2& q = v[i / 4];
    uint32_t& w = ((i % 4) < 2) ? q.x : q.y;
    w = (i % 2 == 0) ? ((w & 0xffff0000u) | bits) : ((w & 0xffffu) | (uint32_t(bits) << 16));
  }
  __device__ __forceinline__ void reverse() {
    uint2 r[(kLen + 3) / 4];
#pragma unroll
    for (int j = 0; j < kLen / 4; ++j) {
      const uint2 q = v[kLen / 4 - 1 - j];
      r[j] = make_uint2(__builtin_amdgcn_alignbit(q.y, q.y, 16), __builtin_amdgcn_alignbit(q.x, q.x, 16));
    }
#pragma unroll
    for (int j = 0; j < kLen / 4; ++j) v[j] = r[j];
  }
};

template <typename T, int kLen>
__device__ __forceinline__ void set_elem(RowTile<T, kLen>& t, int i, const T* p) {
  if constexpr (sizeof(T) == 4)
    t.set(i, *p);
  else
    t.set(i, p->bits);
}

// Load steps [t0, t0 + kLen) of a row.  Forward rows read elements t0.., reversed rows read
// pixels L-1-t for the same steps (then the tile is flipped so that index i is step t0 + i).
// Steps at or past t_end read as the value with bit pattern pad_bits (zero by default).  Vector
// loads need L % 4 == 0, t0 % 4 == 0 and kLen % 4 == 0 (shorter pieces are read element by
// element).
// kDeferRev: with vector loads a reversed row is left in memory order and the caller reverses the
// tile just before using it -- reversing here would make the prefetch wait for its own loads.
// (The element-by-element path places reversed rows in step order either way.)
template <typename T, bool kVecArg, int kLen = kTile, bool kDeferRev = false>
__device__ __forceinline__ void load_row(RowTile<T, kLen>& tile, const T* row, int64_t t0, int64_t t_end, int64_t L,
                                         bool rev, uint32_t pad_bits = 0) {
  constexpr bool kVec = kVecArg && kLen % 4 == 0;
  if (kVec && t0 + kLen <= t_end) {
    // whole tile in range: unconditional vector loads, nothing to zero
    const int64_t base = rev ? (L - t0 - kLen) : t0;
#pragma unroll
    for (int j = 0; j < kLen / 4; ++j) tile.load_vec(row + base + 4 * j, j);
    if (!kDeferRev && rev) tile.reverse();
    return;
  }
  if constexpr (!kVec && sizeof(T) == 2 && kLen % 4 == 0) {
    if (!rev && t0 + kLen <= t_end) {
      // a whole bf16 tile at any 2-byte offset: the dwords from the 4-byte boundary at or below
      // its first element, each output word shifted into place (v_alignbit by 0 or 16 bits);
      // when the tile starts mid-dword its last element is fetched on its own, so that no load
      // reaches past the tile
      const uintptr_t addr = reinterpret_cast<uintptr_t>(row + t0);
      const uint32_t odd = uint32_t(addr >> 1) & 1u;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(addr - 2 * odd);
      uint32_t d[kLen / 2 + 1];
#pragma unroll
      for (int j = 0; j < kLen / 2; ++j) d[j] = w[j];
      d[kLen / 2] = odd ? uint32_t(row[t0 + kLen - 1].bits) : 0u;
#pragma unroll
      for (int j = 0; j < kLen / 4; ++j) {
        const uint32_t lo = __builtin_amdgcn_alignbit(d[2 * j + 1], d[2 * j], 16u * odd);
        const uint32_t hi = __builtin_amdgcn_alignbit(d[2 * j + 2], d[2 * j + 1], 16u * odd);
        tile.v[j] = make_uint2(lo, hi);
      }
      return;
    }
  }
  tile.fill(pad_bits);
  if (kVec) {
    if (!rev) {
#pragma unroll
      for (int j = 0; j < kLen / 4; ++j)
        if (t0 + 4 * j < t_end) tile.load_vec(row + t0 + 4 * j, j);
    } else {
      const int64_t base = L - t0 - kLen;  // pixel of tile element kLen-1
#pragma unroll
      for (int j = 0; j < kLen / 4; ++j)
        if (base + 4 * j >= 0 && L - 1 - (base + 4 * j + 3) < t_end) tile.load_vec(row + base + 4 * j, j);
      if (!kDeferRev) tile.reverse();
    }
  } else {
#pragma unroll
    for (int i = 0; i < kLen; ++i) {
      const int64_t t = t0 + i;
      if (t < t_end) set_elem<T, kLen>(tile, i, row + (rev ? (L - 1 - t) : t));
    }
  }
}

// B/C staging: per lane, the raw values it copies into LDS for one tile.  The vector path keeps
// the loaded words as they are (bf16 pairs, or fp32) and converts them only in store(), at the
// next tile: converting at load time would make the prefetch wait for its own loads.
// Work item j (a 4-step vector, or one element) covers state n = j % NS: consecutive lanes take
// consecutive states, so that the LDS stores of a half-wavefront, at [step][state] with a row
// stride of NS + 4 floats, fall on distinct banks from 16 states up (stepping through the steps
// first put a half-wavefront's stores on 8 banks, four to a bank).
template <typename T, int NS, bool kVec>
struct BCStage {
  using Raw = typename std::conditional<sizeof(T) == 2, uint2, float4>::type;  // 4 steps of one state
  static constexpr int kVecs = (NS * kTile / 4 + kWave - 1) / kWave;  // 4-step vectors per lane
  static constexpr int kElems = (NS * kTile + kWave - 1) / kWave;     // scalars per lane
  Raw rb[kVec ? kVecs : 1], rc[kVec ? kVecs : 1];
  float b[kVec ? 1 : kElems], c[kVec ? 1 : kElems];

  __device__ __forceinline__ static Raw raw_zero() {
    if constexpr (sizeof(T) == 2)
      return make_uint2(0u, 0u);
    else
      return make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ static float4 to_f32(const Raw& r) {
    if constexpr (sizeof(T) == 2)
      return make_float4(bf16lo(r.x), bf16hi(r.x), bf16lo(r.y), bf16hi(r.y));
    else
      return r;
  }

  __device__ __forceinline__ void load(const T* Bg, const T* Cg, int N, int64_t L, int64_t t0, int64_t t_end,
                                       int lane) {
    if (kVec && t0 + kTile <= t_end && NS * kTile / 4 >= kWave * kVecs) {
      // whole tile in range and every lane has whole vectors: no branch around the loads (a load
      // in a conditional block is waited for at the join); states past N read state N-1 and are
      // zeroed by a select
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const int j = lane + k * kWave;
        const int n = j % NS, q = j / NS;
        const int64_t off = int64_t(n < N ? n : N - 1) * L + t0 + 4 * q;
        Raw vb = *reinterpret_cast<const Raw*>(Bg + off), vc = *reinterpret_cast<const Raw*>(Cg + off);
        if (n >= N) vb = vc = raw_zero();
        rb[k] = vb;
        rc[k] = vc;
      }
      return;
    }
    if (kVec) {
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const int j = lane + k * kWave;            // vector id: n = j % NS, q = j / NS
        const int n = j % NS, q = j / NS;
        Raw vb = raw_zero(), vc = raw_zero();
        if (n < N && j < NS * kTile / 4 && t0 + 4 * q < t_end) {
          vb = *reinterpret_cast<const Raw*>(Bg + int64_t(n) * L + t0 + 4 * q);
          vc = *reinterpret_cast<const Raw*>(Cg + int64_t(n) * L + t0 + 4 * q);
        }
        rb[k] = vb;
        rc[k] = vc;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kElems; ++k) {
        const int e = lane + k * kWave;            // element id: n = e % NS, i = e / NS
        const int n = e % NS, i = e / NS;
        float vb = 0.f, vc = 0.f;
        if (n < N && e < NS * kTile && t0 + i < t_end) {
          vb = Elem<T>::load(Bg, int64_t(n) * L + t0 + i);
          vc = Elem<T>::load(Cg, int64_t(n) * L + t0 + i);
        }
        b[k] = vb;
        c[k] = vc;
      }
    }
  }

  // LDS layout: [step][state] with row stride S floats; B is pre-multiplied by ln 2.
  template <int S>
  __device__ __forceinline__ void store(float* sB, float* sC, int lane) const {
    if (kVec) {
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const int j = lane + k * kWave;
        if (j < NS * kTile / 4) {
          const int n = j % NS, q = j / NS;
          const float4 vb = to_f32(rb[k]), vc = to_f32(rc[k]);
          const float bb[4] = {vb.x, vb.y, vb.z, vb.w}, cc[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sB[(4 * q + i) * S + n] = bb[i] * kLn2;
            sC[(4 * q + i) * S + n] = cc[i];
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kElems; ++k) {
        const int e = lane + k * kWave;
        if (e < NS * kTile) {
          const int n = e % NS, i = e / NS;
          sB[i * S + n] = b[k] * kLn2;
          sC[i * S + n] = c[k];
        }
      }
    }
  }
};

// The low-rank projection rows dt (R <= kR rows, fp32, shared by the channels of a group) of one
// 32-step tile, staged in LDS as [step][kR] (rows past R are zero) so that a channel forms its
// raw delta for a step as the dot product of its kR dt_proj weights with the step's kR values.
// As in BCStage, the loads are unconditional (clamped addresses) and keep the raw words; values
// outside the rows or the range are zeroed when stored (a product with a 0/1 mask: a select of
// a loaded word would be turned into a branch around the load).
template <int kR, bool kVec>
struct DtStage {
  static constexpr int kVecs = kR * kTile / 4 / kWave;  // 4-step vectors per lane (kR = 8 or 16)
  static constexpr int kElems = kR * kTile / kWave;     // scalars per lane
  float4 rv[kVec ? kVecs : 1];
  float re[kVec ? 1 : kElems];
  bool ok[kVec ? kVecs : kElems];

  // dt: the group's rows, row r at dt + r * L; steps [t0, t0 + kTile) clipped at t_end
  __device__ __forceinline__ void load(const float* dt, int R, int64_t L, int64_t t0, int64_t t_end, int lane) {
    if (kVec) {  // L % 4 == 0 and t0, t_end are multiples of 4
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const int j = lane + k * kWave, r = j / (kTile / 4), q = j % (kTile / 4);
        const int64_t t = t0 + 4 * q;
        ok[k] = r < R && t < t_end;
        rv[k] = *reinterpret_cast<const float4*>(dt + int64_t(r < R ? r : R - 1) * L + (t < t_end ? t : t0));
      }
    } else {
#pragma unroll
      for (int k = 0; k < kElems; ++k) {
        const int e = lane + k * kWave, r = e / kTile, i = e % kTile;
        const int64_t t = t0 + i;
        ok[k] = r < R && t < t_end;
        re[k] = dt[int64_t(r < R ? r : R - 1) * L + (t < t_end ? t : t0)];
      }
    }
  }
  __device__ __forceinline__ void store(float* sDt, int lane) const {
    if (kVec) {
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const int j = lane + k * kWave, r = j / (kTile / 4), q = j % (kTile / 4);
        const float m = ok[k] ? 1.0f : 0.0f;
        sDt[(4 * q) * kR + r] = rv[k].x * m;
        sDt[(4 * q + 1) * kR + r] = rv[k].y * m;
        sDt[(4 * q + 2) * kR + r] = rv[k].z * m;
        sDt[(4 * q + 3) * kR + r] = rv[k].w * m;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kElems; ++k) {
        const int e = lane + k * kWave, r = e / kTile, i = e % kTile;
        sDt[i * kR + r] = re[k] * (ok[k] ? 1.0f : 0.0f);
      }
    }
  }
};

// raw delta of one step: <w, dt(step)> over the kR staged rows (w past R is zero)
template <int kR>
__device__ __forceinline__ float dt_dot(const float* sDt, const float* w, int step) {
  const float4* v = reinterpret_cast<const float4*>(sDt + step * kR);
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < kR / 4; ++m) {
    const float4 x = v[m];
    acc = fmaf(w[4 * m], x.x, acc);
    acc = fmaf(w[4 * m + 1], x.y, acc);
    acc = fmaf(w[4 * m + 2], x.z, acc);
    acc = fmaf(w[4 * m + 3], x.w, acc);
  }
  return acc;
}

// a channel's dt_proj row (kR weights, zero past R)
template <int kR>
__device__ __forceinline__ void load_dt_w(float* w, const float* row, int R) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const float v = row[r < R ? r : 0];
    w[r] = r < R ? v : 0.0f;
  }
}

template <typename O, bool kVec>
__device__ __forceinline__ void store_out(O* row, const float* y, int64_t t0, int64_t t_end) {
  if (kVec) {
#pragma unroll
    for (int j = 0; j < kTile / 4; ++j)
      if (t0 + 4 * j < t_end)
        Elem<O>::store4(row, t0 + 4 * j, make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]));
  } else {
#pragma unroll
    for (int i = 0; i < kTile; ++i)
      if (t0 + i < t_end) Elem<O>::store(row, t0 + i, y[i]);
  }
}

// Checkpoint slots in lane-major blocks.  When every state is real (N == NS), the per-lane state
// count is a multiple of 4 and a wavefront's rows are whole (per_group a multiple of the rows per
// wavefront), the wavefront's slot at one checkpoint is a contiguous block of kWave x NSL floats
// (its rows, N states each).  Row-major, lane l's states fill bytes [16 NSL l, 16 NSL (l + 1))
// of it, so each 16-byte store instruction writes every other piece of a line.  Lane-major, the
// 16-byte piece j of lane l sits at floats (j kWave + l) 4 of the block: one store instruction
// writes 1 KB of whole lines.  Only the states' order inside the wavefront's own block differs.
template <int NSL, int kSplit>
__device__ __forceinline__ bool ckpt_lane_major(int N, int64_t per_group) {
  return kSplit == 2 && NSL % 4 == 0 && N == NSL * kSplit && per_group % (kWave / kSplit) == 0;
}
// First float of this lane's slot at checkpoint index s for row `row` (lane-major or row-major);
// its 16-byte piece j follows at + j * ckpt_piece_stride.
template <int NSL, int kSplit>
__device__ __forceinline__ int64_t ckpt_slot(bool lane_major, int64_t s, int64_t rows, int64_t row, int N, int lane) {
  const int n0 = (lane % kSplit) * NSL;
  if (lane_major) return (s * rows + row - lane / kSplit) * N + 4 * lane;
  return (s * rows + row) * N + n0;
}
__device__ __forceinline__ int ckpt_piece_stride(bool lane_major) { return lane_major ? 4 * kWave : 4; }

// four floats as a native vector (what the nontemporal builtins accept)
typedef float F4 __attribute__((ext_vector_type(4)));

// a 16-byte store that does not keep its line in the caches (for data written once and read
// back by a later kernel, when the store instructions of a wavefront cover whole lines)
__device__ __forceinline__ void store4_nt(float* p, float4 v) {
  __builtin_nontemporal_store(F4{v.x, v.y, v.z, v.w}, reinterpret_cast<F4*>(p));
}

// Store NS state values (all real, NS % 4 == 0) as 16-byte pieces `stride` floats apart.
template <int NS>
__device__ __forceinline__ void store_state_pieces(float* dst, const float* h, int stride) {
#pragma unroll
  for (int j = 0; j < NS / 4; ++j)
    __builtin_nontemporal_store(F4{h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]},
                                reinterpret_cast<F4*>(dst + j * stride));
}

// Store the first `count` (<= NS) of NS state values; 16-byte stores when NS and count allow.
template <int NS>
__device__ __forceinline__ void store_state(float* dst, const float* h, int count) {
  if (NS % 4 == 0 && count == NS) {  // every state real (the common case): 16-byte stores
#pragma unroll
    for (int n = 0; n < NS; n += 4) *reinterpret_cast<float4*>(dst + n) = make_float4(h[n], h[n + 1], h[n + 2], h[n + 3]);
  } else if (NS % 4 == 0 && (count % 4) == 0) {
#pragma unroll
    for (int n = 0; n < NS; n += 4)
      if (n < count) *reinterpret_cast<float4*>(dst + n) = make_float4(h[n], h[n + 1], h[n + 2], h[n + 3]);
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n)
      if (n < count) dst[n] = h[n];
  }
}

// kSeg consecutive steps [t, t + kSeg) of a row as floats (reversed rows read pixel L-1-step).
// Steps at or past t_end read as 0.  Vector loads need L % 4 == 0, t % 4 == 0 and kSeg % 4 == 0.
template <typename T, bool kVec, int kSeg>
__device__ __forceinline__ void load_seg(float* out, const T* row, int64_t t, int64_t t_end, int64_t L, bool rev) {
  if constexpr (!kVec && sizeof(T) == 2 && kSeg % 4 == 0) {
    if (!rev && t + kSeg <= t_end) {  // whole bf16 segment at any 2-byte offset (as in load_row)
      RowTile<T, kSeg> tile;
      load_row<T, false, kSeg>(tile, row, t, t_end, L, false);
#pragma unroll
      for (int i = 0; i < kSeg; ++i) out[i] = tile.get(i);
      return;
    }
  }
  // Loads are unconditional (steps past t_end re-read step t, which is in range, and are zeroed
  // by a select): a load behind a branch is waited for at the join, one round trip per load.
  if (kVec && kSeg % 4 == 0) {
#pragma unroll
    for (int j = 0; j < kSeg / 4; ++j) {
      const int64_t s = t + 4 * j;
      const bool in = s < t_end;
      const int64_t sc = in ? s : t;
      float4 v = Elem<T>::load4(row, rev ? (L - 4 - sc) : sc);
      if (!in) v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!rev) {
        out[4 * j] = v.x; out[4 * j + 1] = v.y; out[4 * j + 2] = v.z; out[4 * j + 3] = v.w;
      } else {
        out[4 * j] = v.w; out[4 * j + 1] = v.z; out[4 * j + 2] = v.y; out[4 * j + 3] = v.x;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const int64_t s = t + i;
      const bool in = s < t_end;
      const int64_t sc = in ? s : t;
      const float v = Elem<T>::load(row, rev ? (L - 1 - sc) : sc);
      out[i] = in ? v : 0.0f;
    }
  }
}

template <typename O, bool kVec, int kSeg>
__device__ __forceinline__ void store_seg(O* row, const float* v, int64_t t, int64_t t_end) {
  if (kVec && kSeg % 4 == 0) {
#pragma unroll
    for (int j = 0; j < kSeg / 4; ++j)
      if (t + 4 * j < t_end) Elem<O>::store4(row, t + 4 * j, make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]));
  } else {
#pragma unroll
    for (int i = 0; i < kSeg; ++i)
      if (t + i < t_end) Elem<O>::store(row, t + i, v[i]);
  }
}

}  // namespace scan_detail
}  // namespace ss2d
