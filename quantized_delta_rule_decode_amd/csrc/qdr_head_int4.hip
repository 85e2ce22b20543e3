// qdr_head_int4.hip -- whole-head kernels for heads stored as INT4
// (one translation unit per storage kind, so the kinds compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_b4(const PoolConfig &cfg, const LaunchArgs &a, int n, int mode, hipStream_t st) {
  return launch_head_modes<4>(cfg, a, n, mode, st);
}

}  // namespace qdr
