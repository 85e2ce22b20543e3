// qdr_head_int_step.hip -- whole-head kernel over every integer kind, MODE_STEP
// (one translation unit per mode, so the modes compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_step(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_STEP>(cfg, a, n, st);
}

}  // namespace qdr
