// qdr_head_int_unpack.hip -- whole-head kernel over every integer kind, MODE_UNPACK
// (one translation unit per mode, so the modes compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_unpack(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_UNPACK>(cfg, a, n, st);
}

}  // namespace qdr
