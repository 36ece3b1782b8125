// scan_f32_sum.hip -- instantiations of the scan kernel for fp32 streams, segment summary pass.
#include "ssm_device.h"

namespace ssm {

template <int NL, bool FULLN, bool ZOH, bool REV>
static void go(const ScanParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((scan_kernel<float, NL, FULLN, 1, ZOH, REV>), dim3(grid), dim3(256), 0, s, p);
}

template <int NL, bool FULLN>
static void go_flags(const ScanParams& p, int grid, hipStream_t s) {
  if (p.zoh) {
    if (p.reverse) go<NL, FULLN, true, true>(p, grid, s); else go<NL, FULLN, true, false>(p, grid, s);
  } else {
    if (p.reverse) go<NL, FULLN, false, true>(p, grid, s); else go<NL, FULLN, false, false>(p, grid, s);
  }
}

hipError_t launch_scan_f32_sum(const ScanParams& p, int grid, hipStream_t s) {
  const bool full = (p.N % 16) == 0;
  if (p.N <= 16) { if (full) go_flags<1, true>(p, grid, s); else go_flags<1, false>(p, grid, s); }
  else if (p.N <= 32) { if (full) go_flags<2, true>(p, grid, s); else go_flags<2, false>(p, grid, s); }
  else { if (p.N == 64) go_flags<4, true>(p, grid, s); else go_flags<4, false>(p, grid, s); }
  return hipGetLastError();
}

}  // namespace ssm
