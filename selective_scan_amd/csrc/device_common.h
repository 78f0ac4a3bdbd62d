// Device helpers shared by the SS2D kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss2d {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 is carried as its raw 16-bit pattern.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (the default rounding mode), NaN stays NaN:
// gfx950's v_cvt_pk_bf16_f32, which converts two values in one instruction.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// Element access for the two I/O types.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
  // four consecutive elements starting at i (i % 4 == 0, 16-byte aligned)
  __device__ __forceinline__ static float4 load4(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  __device__ __forceinline__ static void store4(float* p, int64_t i, float4 v) {
    *reinterpret_cast<float4*>(p + i) = v;
  }
};
template <>
struct Elem<bf16> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ __forceinline__ static void store(bf16* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
  __device__ __forceinline__ static float4 load4(const bf16* p, int64_t i) {
    uint2 w = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
  }
  __device__ __forceinline__ static void store4(bf16* p, int64_t i, float4 v) {
    uint2 w = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    *reinterpret_cast<uint2*>(p + i) = w;
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log2(1 + 2^w) for any w (softplus(v) = ln 2 * log2(1 + 2^(v log2 e))), evaluated as
// max(w, 0) + log2(1 + e) with e = 2^-|w| in (0, 1]: no overflow; -inf gives exactly 0 (the
// padded steps).  Forming s = fl(1 + e) drops the digits of e below half an ulp of 1, an
// absolute error of up to 2^-24 log2(e) < 9e-8 in the result: relative 6e-5 at delta = 1e-3.
// kExact adds that rounding error back to first order, log2(1 + e) = log2(s) + (e - (s - 1)) /
// (s ln 2) with (e - (s - 1)) exact, the 1/s factor dropped (< 1e-7 absolute for every e): three
// more VALU operations, used for fp32 inputs.  bf16 inputs carry a relative error of 2^-9 in
// delta already, so their kernels use the plain form.
template <bool kExact = true>
__device__ __forceinline__ float softplus_log2(float w) {
  const float m = fmaxf(w, 0.0f);
  const float e = fast_exp2(-fabsf(w));
  const float s = 1.0f + e;
  if constexpr (!kExact) return m + fast_log2(s);
  const float corr = e - (s - 1.0f);
  return m + fast_log2(s) + corr * kLog2e;
}

// softplus_log2<kExact>(w) and, from the same e = 2^-|w| and s = 1 + e, the sigmoid of the
// softplus argument v = w ln 2 (its derivative): 1 / (1 + e^-v) = (w >= 0 ? 1 : e) / s.
template <bool kExact = true>
__device__ __forceinline__ void softplus_sigmoid_log2(float w, float& lam, float& sg) {
  const float m = fmaxf(w, 0.0f);
  const float e = fast_exp2(-fabsf(w));
  const float s = 1.0f + e;
  if constexpr (kExact) {
    const float corr = e - (s - 1.0f);
    lam = m + fast_log2(s) + corr * kLog2e;
  } else {
    lam = m + fast_log2(s);
  }
  sg = (w >= 0.0f ? 1.0f : e) * fast_rcp(s);
}

// silu(z) = z / (1 + e^-z)
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }
__device__ __forceinline__ float sigmoid(float z) { return fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).  Remap so that
// consecutive logical ids land on the same XCD (and share its L2).  Bijective for any n.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
  const int64_t q = n / 8, r = n % 8;
  const int64_t x = i % 8, j = i / 8;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

}  // namespace ss2d
