// scan_bwd_zoh.hip -- launches of the backward pass (and its checkpoint pass) of the
// selective scan with the zero-order-hold discretisation, B_bar = (exp(dt A) - 1) / A * B.
// A translation unit of its own so that the two discretisations compile in parallel.
#include "scan_bwd_kernel.h"

namespace ssm {

hipError_t launch_ckpt_zoh(const ScanParams& p, bool bf16, hipStream_t s) { return go_ckpt_all<true>(p, bf16, s); }

hipError_t launch_bwd_zoh(const BwdParams& p, bool bf16, hipStream_t s) { return go_bwd_all<true>(p, bf16, s); }

}  // namespace ssm
