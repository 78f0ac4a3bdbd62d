// Instantiation of the selective-scan forward kernels for f32 I/O, up to 16 states.
#include "scan_fwd_kernel.h"

namespace ss2d {
template hipError_t scan_fwd_launch<float, 16, float>(const ScanFwdParams&, hipStream_t);
}  // namespace ss2d
