// Scan sweep instantiations for mode 7: softplus step and exact ZOH, decays from A[d, 0].
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<7>(const ScanLaunch& p) {
  return launch_scan_for_mode<7>(p);
}
}  // namespace ssm
