// Instantiation of the selective-scan forward kernels for bf16 I/O with an fp32 u (the SS2D input front's output), up to 64 states.
#include "scan_fwd_kernel.h"

namespace ss2d {
template hipError_t scan_fwd_launch<bf16, 64, float>(const ScanFwdParams&, hipStream_t);
}  // namespace ss2d
