// Instantiation of the selective-scan backward kernels for bf16 I/O with an fp32 u (the SS2D input front's output), up to 1 states.
#include "scan_bwd_kernel.h"

namespace ss2d {
template hipError_t scan_bwd_launch<bf16, 1, float>(const ScanBwdParams&, hipStream_t);
}  // namespace ss2d
