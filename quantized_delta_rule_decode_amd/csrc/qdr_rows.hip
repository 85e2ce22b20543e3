// qdr_rows.hip -- row-unit kernels (per-key-row storage kinds) and their launch.
#include <algorithm>

#include "qdr_device.h"

namespace qdr {

namespace {

template <int MODE>
hipError_t launch_rows(const PoolConfig &cfg, LaunchArgs a, int n, const ListEntry *list, int count,
                       hipStream_t st) {
  a.head_list = list;
  a.n_list = count;
  // Each wave's LDS region (rows of 128 words): the staged words of its half
  // plus one row (the second word of a funnel shift), reused after the
  // restore as the row reduction's scratch (64 x 20 floats = 10 rows) and for
  // the stored bits of the half's pivot rows (one row each).
  a.region_rows = std::max({cfg.max_words + 1, cfg.max_pivots, 10});
  const size_t lds = (size_t)2 * a.region_rows * kDim * sizeof(uint32_t);
  const dim3 grid((unsigned)((int64_t)n * count)), block(128);
  if (grid.x == 0) return hipSuccess;
  hipError_t err = hipSuccess;
  with_variant(cfg, [&](auto G, auto S, auto Fi) {
    const void *fn = (const void *)k_rows<MODE, decltype(G)::value, decltype(S)::value, decltype(Fi)::value>;
    if (lds > 65536) {   // pools with FP32 rows: allow the larger dynamic LDS
      err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return;
    }
    hipLaunchKernelGGL((k_rows<MODE, decltype(G)::value, decltype(S)::value, decltype(Fi)::value>), grid, block,
                       lds, st, a);
  });
  if (err != hipSuccess) return err;
  return hipGetLastError();
}


}  // namespace

hipError_t launch_rows_mode(const PoolConfig &cfg, const LaunchArgs &a, int n, const ListEntry *list, int count,
                            int mode, hipStream_t st) {
  switch (mode) {
    case MODE_STEP: return launch_rows<MODE_STEP>(cfg, a, n, list, count, st);
    case MODE_READOUT: return launch_rows<MODE_READOUT>(cfg, a, n, list, count, st);
    case MODE_STEP_BF16: return launch_rows<MODE_STEP_BF16>(cfg, a, n, list, count, st);
    case MODE_WRITEBACK: return launch_rows<MODE_WRITEBACK>(cfg, a, n, list, count, st);
    case MODE_PACK: return launch_rows<MODE_PACK>(cfg, a, n, list, count, st);
    case MODE_UNPACK: return launch_rows<MODE_UNPACK>(cfg, a, n, list, count, st);
    default: return launch_rows<MODE_RESET>(cfg, a, n, list, count, st);
  }
}

}  // namespace qdr
