// qdr_head_int_readout.hip -- whole-head kernel over every integer kind,
// MODE_READOUT (the readout-first half of the two-stream step).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_readout(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_READOUT>(cfg, a, n, st);
}

}  // namespace qdr
