// qdr_head_int2.hip -- whole-head kernels for heads stored as INT2
// (one translation unit per storage kind, so the kinds compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_b2(const PoolConfig &cfg, const LaunchArgs &a, int n, int mode, hipStream_t st) {
  return launch_head_modes<2>(cfg, a, n, mode, st);
}

}  // namespace qdr
