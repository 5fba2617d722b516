// Scan sweep instantiations for mode 4: decays from A[d, 0] (A[d, n] = (n+1) A[d, 0]).
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<4>(const ScanLaunch& p) {
  return launch_scan_for_mode<4>(p);
}
}  // namespace ssm
