// qdr_head_int8.hip -- whole-head kernels for heads stored as INT8
// (one translation unit per storage kind, so the kinds compile in parallel).
#include "qdr_device.h"

namespace qdr {

hipError_t launch_head_b8(const PoolConfig &cfg, const LaunchArgs &a, int n, int mode, hipStream_t st) {
  return launch_head_modes<8>(cfg, a, n, mode, st);
}

}  // namespace qdr
