// Instantiation of the selective-scan backward kernels for f32 I/O, up to 16 states.
#include "scan_bwd_kernel.h"

namespace ss2d {
template hipError_t scan_bwd_launch<float, 16, float>(const ScanBwdParams&, hipStream_t);
}  // namespace ss2d
