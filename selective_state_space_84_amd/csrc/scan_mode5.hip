// Scan sweep instantiations for mode 5: softplus step, decays from A[d, 0].
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<5>(const ScanLaunch& p) {
  return launch_scan_for_mode<5>(p);
}
}  // namespace ssm
