// Instantiation of the selective-scan backward kernels for bf16 I/O, up to 8 states.
#include "scan_bwd_kernel.h"

namespace ss2d {
template hipError_t scan_bwd_launch<bf16, 8, bf16>(const ScanBwdParams&, hipStream_t);
}  // namespace ss2d
