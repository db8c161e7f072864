// Rank-r covariance summaries (gfx950) -- not yet built: the launcher reports
// hipErrorNotSupported so the C ABI returns COBS_ERR_HIP for rank-r builds.
#include "cobs_device.h"
#include "cobs_launch.h"

namespace cobs {

hipError_t launch_build_lowrank(const BuildArgs& a) {
  (void)a;
  return hipErrorNotSupported;
}

}  // namespace cobs
