// Instantiation of the selective-scan forward kernels for f32 I/O, up to 1 states.
#include "scan_fwd_kernel.h"

namespace ss2d {
template hipError_t scan_fwd_launch<float, 1, float>(const ScanFwdParams&, hipStream_t);
}  // namespace ss2d
