// scan_bf16_sum.hip -- instantiations of the scan kernel for bf16 streams, segment summary pass.
#include "ssm_device.h"

namespace ssm {

template <int NL, bool ZOH, bool REV, bool VEC>
static void go(const ScanParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((scan_kernel<bf16_t, NL, 1, ZOH, REV, VEC>), dim3(grid), dim3(256), 0, s, p);
}

template <int NL>
static void go_flags(const ScanParams& p, int grid, hipStream_t s) {
  const int k = (p.zoh ? 4 : 0) + (p.reverse ? 2 : 0) + (p.vec ? 1 : 0);
  switch (k) {
    case 0: go<NL, false, false, false>(p, grid, s); break;
    case 1: go<NL, false, false, true>(p, grid, s); break;
    case 2: go<NL, false, true, false>(p, grid, s); break;
    case 3: go<NL, false, true, true>(p, grid, s); break;
    case 4: go<NL, true, false, false>(p, grid, s); break;
    case 5: go<NL, true, false, true>(p, grid, s); break;
    case 6: go<NL, true, true, false>(p, grid, s); break;
    default: go<NL, true, true, true>(p, grid, s); break;
  }
}

hipError_t launch_scan_bf16_sum(const ScanParams& p, int grid, hipStream_t s) {
  if (p.N <= 16) go_flags<1>(p, grid, s);
  else if (p.N <= 32) go_flags<2>(p, grid, s);
  else go_flags<4>(p, grid, s);
  return hipGetLastError();
}

}  // namespace ssm
