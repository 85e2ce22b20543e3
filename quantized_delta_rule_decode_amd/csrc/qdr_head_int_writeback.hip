// qdr_head_int_writeback.hip -- whole-head kernel over every integer kind,
// MODE_WRITEBACK (the write-back half of the two-stream step).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_writeback(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_WRITEBACK>(cfg, a, n, st);
}

}  // namespace qdr
