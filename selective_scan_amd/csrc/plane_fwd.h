// The single-kernel SS2D forward for small state sizes (one workgroup per (image, channel) plane).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ss2d {

struct PlaneFwdArgs {
  const void* x;            // (batch, dim, H, W), I/O dtype
  const void* delta;        // (batch, 4, dim, L) raw delta, each route in its own step order
  const void* Bm;           // (batch, 4, N, L)
  const void* Cm;           // (batch, 4, N, L)
  const float* A;           // (4, dim, N)
  const float* Dskip;       // (4, dim) or null
  const float* delta_bias;  // (4, dim) or null
  const void* z;            // (batch, dim, H, W) or null
  void* out;                // (batch, dim, H, W)
  int64_t batch, dim;
  int64_t H, W;
  int N;
  int dtype;     // 0 = fp32, 1 = bf16
  int softplus;  // delta = softplus(delta_raw + bias), else delta_raw + bias
};

// Whether launch_plane_fwd handles these arguments (state size 1, 2 or 4; L a multiple of 8;
// the plane's four LDS arrays of L floats within 63 KB; every tensor 16-byte aligned).
bool plane_fwd_supported(const PlaneFwdArgs& a);
hipError_t launch_plane_fwd(const PlaneFwdArgs& a, hipStream_t s);

}  // namespace ss2d
