// Scan sweep instantiations for mode 1: softplus(delta + dt_bias) step.
// (One translation unit per mode so the instantiations build in parallel.)
#include "scan_sweep.h"

namespace ssm {
template <>
hipError_t launch_scan_mode<1>(const ScanLaunch& p) {
  return launch_scan_for_mode<1>(p);
}
}  // namespace ssm
