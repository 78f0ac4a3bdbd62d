// Instantiation of the selective-scan forward kernels for bf16 I/O, up to 32 states.
#include "scan_fwd_kernel.h"

namespace ss2d {
template hipError_t scan_fwd_launch<bf16, 32, bf16>(const ScanFwdParams&, hipStream_t);
}  // namespace ss2d
