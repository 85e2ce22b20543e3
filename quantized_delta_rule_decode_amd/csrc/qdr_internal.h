// qdr_internal.h -- structures shared by the host runtime and the HIP kernels
// of libqdr (never installed; the public ABI is include/qdr.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace qdr {

constexpr int kDim = 128;

enum Mode : int { MODE_STEP = 0, MODE_PACK = 1, MODE_UNPACK = 2, MODE_RESET = 3, MODE_READOUT = 4, MODE_STEP_BF16 = 5,
                  MODE_WRITEBACK = 6 };

// Per-head metadata on the device (16 bytes).
struct HeadInfo {
  uint64_t off;         // block offset inside a slot
  uint32_t code_bytes;  // bytes of the code region
  uint8_t words0;       // row units: 32-bit words per column for rows 0..63
  uint8_t words1;       // row units: 32-bit words per column for rows 64..127
  uint8_t kind;         // whole-head units: the head's kind; row units: 0
  uint8_t has_scales;   // 1 when the block stores r (and c)
};

// One entry of a launch's head list (32 bytes, read with one scalar load):
// the head's table row and its index.
struct ListEntry {
  HeadInfo info;
  int32_t h;
  int32_t pad[3];
};
static_assert(sizeof(HeadInfo) == 16 && sizeof(ListEntry) == 32, "device table layout");

// Row units: a table with one entry per (head, row) describing the row's
// field in its half of the column streams, as operands the kernel uses with
// at most two scalar instructions each.  With x = byte offset of the field's first
// 32-bit word in the half's [word][column] image (word index * 512, so its
// low 9 bits are zero), y = bit offset of the field in that word and
// z = the field's width (the row's kind).  One word serves the restore and
// the repack:
//   xs = x | (z / 2) << 5 | y | c << 30   (z / 2 in 1..8 for the 2..16-bit
//   kinds, 0 for FP32; c = 1 when a 2..16-bit field reaches the end of its
//   first word, y + z >= 32)
// The restore's funnel shift by y and the repack's completing shift by
// (32 - y) & 31 = (-xs) & 31 read only the low 5 bits of their operand;
// (xs >> 4) & 30 is the width of a 2..16-bit field; the LDS address is x
// (bits 9..29) with the low 9 bits replaced by the lane's byte.
constexpr uint32_t kRowCompletes = 1u << 30;   // c above
struct RowProg {
  uint32_t xs;   // x | width code | shift | completes
  uint32_t z;    // width
};

// Everything a launch needs, passed by value as the kernel argument.
struct LaunchArgs {
  uint8_t *pool;
  uint64_t slot_stride;
  int32_t num_slots;
  int32_t H;
  const ListEntry *head_list;   // heads handled by this launch
  int32_t n_list;
  const RowProg *row_prog;    // [H*128] (row units)
  int32_t region_rows;        // row units: LDS rows of 128 words in each wave's region
  const float *omega;         // [H*128]
  uint32_t *err;              // device error word
  const int32_t *slots;       // [n] slot of each request / dense entry
  const float *q, *k, *v, *beta, *gate;   // q, k, v: uint16 bfloat16 data in MODE_STEP_BF16
  float *o;                               // uint16 bfloat16 data in MODE_STEP_BF16
  const float *S_in;          // pack: [n][H][128][128]
  float *S_out;               // unpack
};

struct PoolConfig {
  int unit, gate, scale_mode, fit_iters;
  int scale_bits;             // 32: fp32 factors; 16: bfloat16
  int max_words;              // row units: largest words-per-column of any half
  int max_pivots;             // row units: most FP16/FP32 rows in any half
};

// Whole-head launches.  Integer kinds share one launch per mode
// (qdr_head_int_<mode>.hip) over the interleaved list of integer heads;
// FP16 and FP32 heads get one launch each (qdr_head_fp16.hip,
// qdr_head_fp32.hip).  args.head_list / n_list name the heads.
hipError_t launch_head_int_step(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_pack(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_unpack(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_reset(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_readout(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_step_bf16(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_int_writeback(const PoolConfig &, const LaunchArgs &, int n, hipStream_t);
hipError_t launch_head_b16(const PoolConfig &, const LaunchArgs &, int n, int mode, hipStream_t);
hipError_t launch_head_b32(const PoolConfig &, const LaunchArgs &, int n, int mode, hipStream_t);
// Row-unit launch (qdr_rows.hip) over the heads in list[0..count).
hipError_t launch_rows_mode(const PoolConfig &, const LaunchArgs &, int n, const ListEntry *list, int count,
                            int mode, hipStream_t);

// Number of head lists a pool keeps: per kind (INT2, INT4, INT6, INT8, FP16,
// FP32) and, last, every integer head interleaved by kind (whole-head units;
// row-unit pools keep all heads in list 0).
constexpr int kNumLists = 7;
constexpr int kListIntMix = 6;

// Launch the kernels of one mode over `n` requests / dense entries: the
// row-unit kernel, or for whole-head pools the integer launch on `stream`
// and the float-kind launches on `float_stream` (the caller orders the two
// streams).  Returns hipSuccess or the first launch error.
hipError_t launch_all(const PoolConfig &cfg, LaunchArgs args, int n,
                      const ListEntry *const *kind_lists, const int32_t *kind_counts,
                      int mode, hipStream_t stream, hipStream_t float_stream);

}  // namespace qdr
