// Scan sweep instantiations for mode 2: exact zero-order-hold input term.
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<2>(const ScanLaunch& p) {
  return launch_scan_for_mode<2>(p);
}
}  // namespace ssm
