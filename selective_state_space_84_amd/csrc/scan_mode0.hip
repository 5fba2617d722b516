// Scan sweep instantiations for mode 0: plain step and input term.
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<0>(const ScanLaunch& p) {
  return launch_scan_for_mode<0>(p);
}
}  // namespace ssm
