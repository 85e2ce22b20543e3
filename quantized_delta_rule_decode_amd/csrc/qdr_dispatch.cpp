// qdr_dispatch.cpp -- picks the kernels of one mode: the row-unit kernel, or
// one whole-head launch per storage kind present, back to back on the stream.
#include "qdr_internal.h"

namespace qdr {

hipError_t launch_all(const PoolConfig &cfg, LaunchArgs args, int n, const ListEntry *const *kind_lists,
                      const int32_t *kind_counts, int mode, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (cfg.unit != 0) return launch_rows_mode(cfg, args, n, kind_lists[0], kind_counts[0], mode, stream);
  typedef hipError_t (*head_fn)(const PoolConfig &, const LaunchArgs &, int, int, hipStream_t);
  static const head_fn fns[6] = {launch_head_b2, launch_head_b4, launch_head_b6,
                                 launch_head_b8, launch_head_b16, launch_head_b32};
  hipError_t e = hipSuccess;
  for (int kidx = 0; kidx < 6 && e == hipSuccess; ++kidx) {
    if (kind_counts[kidx] == 0) continue;
    args.head_list = kind_lists[kidx];
    args.n_list = kind_counts[kidx];
    e = fns[kidx](cfg, args, n, mode, stream);
  }
  return e;
}

}  // namespace qdr
