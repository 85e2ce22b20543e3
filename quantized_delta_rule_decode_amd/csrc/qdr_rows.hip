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
  const bool dual = cfg.scale_mode == 0, fit = cfg.fit_iters > 0, diag = cfg.gate == 1;
  if (lds > 65536) {   // pools with FP32 rows: allow the larger dynamic LDS
    const void *fns[6] = {(const void *)k_rows<MODE, 1, 1, 0>, (const void *)k_rows<MODE, 0, 1, 0>,
                          (const void *)k_rows<MODE, 1, 0, 1>, (const void *)k_rows<MODE, 0, 0, 1>,
                          (const void *)k_rows<MODE, 1, 0, 0>, (const void *)k_rows<MODE, 0, 0, 0>};
    for (const void *f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
  }
  if (!dual) {
    if (diag) hipLaunchKernelGGL((k_rows<MODE, 1, 1, 0>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((k_rows<MODE, 0, 1, 0>), grid, block, lds, st, a);
  } else if (fit) {
    if (diag) hipLaunchKernelGGL((k_rows<MODE, 1, 0, 1>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((k_rows<MODE, 0, 0, 1>), grid, block, lds, st, a);
  } else {
    if (diag) hipLaunchKernelGGL((k_rows<MODE, 1, 0, 0>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((k_rows<MODE, 0, 0, 0>), grid, block, lds, st, a);
  }
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
