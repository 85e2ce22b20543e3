// qdr_dispatch.cpp -- picks the kernels of one mode: the row-unit kernel, or
// for whole-head pools one launch over every integer head (kinds mixed) and
// one launch per float kind present.
#include "qdr_internal.h"

namespace qdr {

hipError_t launch_all(const PoolConfig &cfg, LaunchArgs args, int n, const ListEntry *const *kind_lists,
                      const int32_t *kind_counts, int mode, hipStream_t stream, hipStream_t float_stream) {
  if (n <= 0) return hipSuccess;
  if (cfg.unit != 0) return launch_rows_mode(cfg, args, n, kind_lists[0], kind_counts[0], mode, stream);
  hipError_t e = hipSuccess;
  if (kind_counts[kListIntMix] > 0) {
    args.head_list = kind_lists[kListIntMix];
    args.n_list = kind_counts[kListIntMix];
    switch (mode) {
      case MODE_STEP: e = launch_head_int_step(cfg, args, n, stream); break;
      case MODE_READOUT: e = launch_head_int_readout(cfg, args, n, stream); break;
      case MODE_STEP_BF16: e = launch_head_int_step_bf16(cfg, args, n, stream); break;
      case MODE_WRITEBACK: e = launch_head_int_writeback(cfg, args, n, stream); break;
      case MODE_PACK: e = launch_head_int_pack(cfg, args, n, stream); break;
      case MODE_UNPACK: e = launch_head_int_unpack(cfg, args, n, stream); break;
      default: e = launch_head_int_reset(cfg, args, n, stream); break;
    }
  }
  if (e == hipSuccess && kind_counts[4] > 0) {
    args.head_list = kind_lists[4];
    args.n_list = kind_counts[4];
    e = launch_head_b16(cfg, args, n, mode, float_stream);
  }
  if (e == hipSuccess && kind_counts[5] > 0) {
    args.head_list = kind_lists[5];
    args.n_list = kind_counts[5];
    e = launch_head_b32(cfg, args, n, mode, float_stream);
  }
  return e;
}

}  // namespace qdr
