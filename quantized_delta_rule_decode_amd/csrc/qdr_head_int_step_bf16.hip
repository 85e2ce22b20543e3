// qdr_head_int_step_bf16.hip -- whole-head kernel over every integer kind,
// MODE_STEP_BF16 (the step with bfloat16 q, k, v and o).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_int_step_bf16(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  return launch_head_int_mode<MODE_STEP_BF16>(cfg, a, n, st);
}

}  // namespace qdr
