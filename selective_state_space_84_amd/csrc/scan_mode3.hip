// Scan sweep instantiations for mode 3: softplus step and exact zero-order-hold input term.
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<3>(const ScanLaunch& p) {
  return launch_scan_for_mode<3>(p);
}
}  // namespace ssm
