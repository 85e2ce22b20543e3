// qdr_head_int_reset.hip -- whole-head kernel over every integer kind, MODE_RESET
// (one translation unit per mode, so the modes compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_reset(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_RESET>(cfg, a, n, st);
}

}  // namespace qdr
