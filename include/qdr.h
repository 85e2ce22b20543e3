/*
 * qdr.h -- C ABI of the MI355X quantized gated delta-rule decode library.
 *
 * The library keeps a pool of packed recurrent states (one 128 x 128 state per
 * (slot, head)) in device memory and runs the fused decode step of STEPQuant
 * on it: restore the mixed-precision packed state, apply the gate and the
 * gated delta rule, read out o = S^T q, refit the dual-axis row/column
 * scales with fixed row-impact weights, requantise and write back in place.
 *
 * Page references (titles of the pages describing the method):
 *   Tutorial  -- "STEPQuant：取代 KV cache 的状态，6-bit 量化精度不掉" (bloombook.cn)
 *   Review-AT -- "STEPQuant: When and Where Errors Matter in Delta-Rule
 *                Recurrent State Quantization" (ai-trend.me)
 *   Review-SL -- "STEPQuant：誤差の寿命と位置から設計するDelta則の再帰状態量子化"
 *                (singularity-lens.com)
 *   Discussion-ZC -- discussion reply on the zhichai.net STEPQuant post
 *
 * Conventions for every entry point:
 *   - Tensor pointers (q, k, v, beta, gate, o, S, slots) are DEVICE pointers
 *     to contiguous arrays, 4-byte aligned, owned by the caller; the library
 *     never frees them, and they must stay valid (and the inputs unchanged)
 *     until the work the call enqueues on `stream` has completed.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *     enqueued asynchronously and the call returns without synchronising,
 *     except where stated (read_raw, write_raw, poll_device_error, and the
 *     host-side slot check enabled by QDR_DEBUG=1).  A whole-head pool that
 *     holds FP16 or FP32 heads next to integer heads also launches on a
 *     stream of its own (default priority, created with the pool): that work
 *     is forked from `stream` by an event recorded there and joined back by
 *     an event `stream` waits on, so work enqueued on `stream` after the call
 *     sees all of its results.  Fork and join are event operations, so a
 *     call on a capturing stream is captured whole into a HIP graph.  Calls
 *     on one pool from several host threads at once race.
 *   - Every call returns a qdr_status.  Argument errors are found on the host
 *     before anything is enqueued, so a failed call has no side effects.
 *     qdr_last_error() gives a message for the calling thread.  No C++
 *     exception or abort crosses the ABI.
 *   - Slot tables are int32 arrays on the device.  Slot -1 marks a padding
 *     row (skipped; its o rows are written as 0).  A slot outside
 *     [-1, num_slots) sets QDR_DEVERR_SLOT in the pool's device error word
 *     and its o rows are written as 0.  Slots must be distinct within one
 *     call (two rows on one slot race); QDR_DEBUG=1 checks this on the host.
 *   - d_k = d_v = 128 (QDR_DIM).
 */
#ifndef QDR_H
#define QDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDR_DIM 128

typedef struct qdr_pool qdr_pool;   /* opaque; owned by the library */

typedef enum {
  QDR_OK = 0,
  QDR_E_INVAL = -1,        /* bad argument (null pointer, size, enum, table) */
  QDR_E_NOMEM = -2,        /* device allocation failed or buffer too small  */
  QDR_E_DEVICE = -3,       /* a HIP runtime call failed                     */
  QDR_E_SLOT = -4,         /* bad slot (host-checked calls)                 */
  QDR_E_UNSUPPORTED = -5   /* combination not supported                     */
} qdr_status;

/* Gate D_t (Tutorial §二): a head-shared scalar alpha (Gated DeltaNet) or a
 * per-key-channel diagonal (Kimi Delta Attention). */
enum { QDR_GATE_SCALAR = 0, QDR_GATE_DIAG = 1 };
/* Unit of the static precision allocation (Review-AT, Method): whole heads
 * (GDN) or key rows (KDA). */
enum { QDR_UNIT_HEAD = 0, QDR_UNIT_ROW = 1 };
/* Scale rule: STEPQuant's dual-axis key-row x value-column factors
 * (Tutorial §四), or the uniform baseline's per-key-row absmax scale
 * (Review-SL, uniform-baseline paragraph). */
enum { QDR_SCALE_DUAL = 0, QDR_SCALE_ROW_ABSMAX = 1 };
/* Storage kinds; the value is the bit width of one element.  INTb rows are
 * symmetric integer codes in [-(2^(b-1)-1), 2^(b-1)-1]; FP16 rows are the
 * pivots kept in half precision (Tutorial §四); FP32 is the uncompressed
 * state. */
enum {
  QDR_K_INT2 = 2, QDR_K_INT4 = 4, QDR_K_INT6 = 6, QDR_K_INT8 = 8,
  QDR_K_FP16 = 16, QDR_K_FP32 = 32
};

/* Bits of the device error word (qdr_poll_device_error). */
#define QDR_DEVERR_SLOT 1u

typedef struct {
  int32_t num_slots;      /* slots in the pool, e.g. 5*B+1 (Discussion-ZC)   */
  int32_t num_heads;      /* heads per slot                                  */
  int32_t d_k, d_v;       /* must both be 128                                */
  int32_t unit;           /* QDR_UNIT_*                                      */
  int32_t gate;           /* QDR_GATE_*: form of the gate passed to the step */
  int32_t scale_mode;     /* QDR_SCALE_*                                     */
  int32_t fit_iters;      /* 0: column factor = clip-free range (V0);
                             1: plus one weighted least-squares refit (V1a);
                             must be 0 with QDR_SCALE_ROW_ABSMAX             */
  const uint8_t *kinds;   /* HOST: [num_heads] (UNIT_HEAD) or
                             [num_heads*128] (UNIT_ROW) of QDR_K_*; copied   */
  const float *omega;     /* HOST: [num_heads*128] row-impact weights,
                             finite, in [2^-40, 2^40]; ignored for
                             ROW_ABSMAX (may be NULL); copied                */
  int32_t scale_bits;     /* stored width of the factors r and c: 0 or 32 =
                             fp32; 16 = bfloat16 (compact storage; Review-SL,
                             compact-bits paragraph).  With 16 the row factor
                             and the clip-free column factor are rounded up to
                             bfloat16 before the codes are computed from
                             them, a refitted column factor is rounded to
                             nearest even, and the restore reads the stored
                             values                                           */
} qdr_pool_desc;

typedef struct {
  uint64_t slot_stride;        /* bytes between consecutive slots            */
  uint64_t total_bytes;        /* num_slots * slot_stride                    */
  int32_t num_slots, num_heads;
  const uint64_t *head_off;    /* HOST [num_heads]: block offset in a slot;
                                  owned by the pool                          */
  const uint32_t *head_bytes;  /* HOST [num_heads]: block size               */
  const uint32_t *code_bytes;  /* HOST [num_heads]: code bytes of a block    */
  void *base;                  /* device address of slot 0                   */
  double bits_per_value;       /* stored bits per state value, all included  */
} qdr_layout;

/* Device bytes needed for the packed states of a pool described by desc
 * (pure host computation).  Layout of one (slot, head) block: the code
 * stream of column j holds rows 0..127 as b-bit fields, cut into granules of
 * 16 B (UNIT_HEAD) or 4 B (UNIT_ROW); granule g of column j is at byte
 * (g*128 + j)*G; then r[128] fp32 and, for dual-axis scales, c[128] fp32
 * when the head has integer rows; blocks are padded to 256 B. */
qdr_status qdr_pool_bytes(const qdr_pool_desc *desc, size_t *bytes);

/* Create a pool on the current HIP device.  dev_mem == NULL: the library
 * allocates (and frees in destroy) the state memory; otherwise dev_mem must
 * hold at least qdr_pool_bytes() bytes, be 256-byte aligned and outlive the
 * pool.  The pool's small device tables (offsets, kinds, omega, error word)
 * are always allocated by the library.  State memory is zero-filled, which
 * is not a valid encoding of S = 0 for integer kinds: call qdr_slot_reset or
 * qdr_pack before stepping a slot.  Synchronises the device. */
qdr_status qdr_pool_create(const qdr_pool_desc *desc, void *dev_mem,
                           size_t dev_bytes, qdr_pool **out);
/* Free the pool (and its memory if the library allocated it).  Synchronises
 * the device first.  NULL is accepted. */
qdr_status qdr_pool_destroy(qdr_pool *pool);

/* Encode S = 0 into the n listed slots (codes 0, r = 1, c = 1). */
qdr_status qdr_slot_reset(qdr_pool *pool, const int32_t *slots, int32_t n,
                          void *stream);

/* Quantise dense fp32 states S[n][H][128][128] (row = key channel) into the
 * n listed slots: the requantisation tail of the step (scale fit, codes,
 * pack) applied to the given S (Tutorial §四). */
qdr_status qdr_pack(qdr_pool *pool, const int32_t *slots, int32_t n,
                    const float *S, void *stream);

/* Restore the n listed slots to dense fp32 S_out[n][H][128][128]:
 * X_ij = r_i c_j z_ij / q_i for integer rows, the stored value otherwise. */
qdr_status qdr_unpack(qdr_pool *pool, const int32_t *slots, int32_t n,
                      float *S_out, void *stream);

/* One fused decode step for B requests (Tutorial §二 and §四; order of work
 * per Review-SL, generation-time paragraph).  For every b < B with
 * slots[b] >= 0 and every head h:
 *   S' = D S_{t-1} restored from the packed slot, u = S'^T k,
 *   S_t = S' + beta k (v - u)^T  ( = (I - beta k k^T) D S_{t-1} + beta k v^T ),
 *   o = S_t^T q (before requantisation), then S_t is requantised into the
 *   slot in place.
 * q, k, v, o: [B][H][128] fp32; beta: [B][H]; gate: [B][H] (QDR_GATE_SCALAR,
 * linear alpha = exp(-g)) or [B][H][128] (QDR_GATE_DIAG, linear a_i).
 * Inputs are not checked for NaN or infinity: such values propagate through
 * the arithmetic of their own (request, head) -- its readout and its stored
 * block -- and leave every other head and request untouched. */
qdr_status qdr_decode_step(qdr_pool *pool, const int32_t *slots, int32_t B,
                           const float *q, const float *k, const float *v,
                           const float *beta, const float *gate, float *o,
                           void *stream);

/* The same step with bfloat16 q, k, v and o (compact I/O: half the bytes of
 * the fp32 vectors; Review (singularity-lens), compact-bits paragraph, counts
 * every stored byte).  q, k, v: [B][H][128] bfloat16 (uint16 bit patterns),
 * widened to fp32 exactly; beta and gate fp32 as in qdr_decode_step; o:
 * [B][H][128] bfloat16, the fp32 readout rounded to nearest, ties to even.
 * The state update and the stored state are those of qdr_decode_step on the
 * widened inputs.  Errors as qdr_decode_step. */
qdr_status qdr_decode_step_bf16(qdr_pool *pool, const int32_t *slots, int32_t B,
                                const uint16_t *q, const uint16_t *k,
                                const uint16_t *v, const float *beta,
                                const float *gate, uint16_t *o, void *stream);

/* The same step split over two streams (Tutorial §四, engineering paragraph:
 * the head output goes downstream first, and a second stream writes the
 * compressed state back so that the scale update overlaps model compute).
 *   1. on stream_readout: restore, gate, u and delta, o = S_t^T q -> o (the
 *      state is not written);
 *   2. on stream_writeback, ordered after 1 by an event: the whole step again
 *      (restore, update, refit, requantise, store) without writing o.
 * o and the stored state are bit-identical to qdr_decode_step's.  The
 * inputs (slots, q, k, v, beta, gate) must stay unchanged until
 * stream_writeback has finished.  Every later call on this pool, on any
 * stream, is ordered after the write-back by the library (an event recorded
 * on stream_writeback; qdr_read_raw / qdr_write_raw included).  Both streams
 * belong to the caller and must have the default priority; they may be the
 * same stream.  Calls on one pool from several host threads at once race.
 * Errors as qdr_decode_step, plus QDR_E_DEVICE if an event call fails. */
qdr_status qdr_decode_step_split(qdr_pool *pool, const int32_t *slots, int32_t B,
                                 const float *q, const float *k, const float *v,
                                 const float *beta, const float *gate, float *o,
                                 void *stream_readout, void *stream_writeback);

/* Layout of the pool (pointers stay valid until qdr_pool_destroy). */
qdr_status qdr_get_layout(const qdr_pool *pool, qdr_layout *out);

/* Copy the raw bytes of one slot (n = slot_stride) to or from HOST memory.
 * Synchronise `stream` before returning. */
qdr_status qdr_read_raw(qdr_pool *pool, int32_t slot, void *host_dst,
                        size_t n, void *stream);
qdr_status qdr_write_raw(qdr_pool *pool, int32_t slot, const void *host_src,
                         size_t n, void *stream);

/* Read and clear the device error word (bits QDR_DEVERR_*).  Synchronises
 * the device. */
qdr_status qdr_poll_device_error(qdr_pool *pool, uint32_t *flags);

/* Message describing the last failed call on this thread ("" if none). */
const char *qdr_last_error(void);

/* Diagnostic, not part of the decode step: enqueue on `stream` one wave
 * that runs iters x 256 fma instructions between two reads of the
 * shader-clock counter and of the constant 100 MHz counter, and stores
 * out[0..3] = {clock start, 100 MHz start, clock end, 100 MHz end} (out: a
 * device array of at least 5 uint64; out[4] holds a by-product).  The
 * shader clock in MHz is 100 (out[2] - out[0]) / (out[3] - out[1]); launched
 * on a second stream while decode steps run, it gives the clock the steps
 * run at.  QDR_E_INVAL for a null out or iters <= 0. */
qdr_status qdr_clock_probe(uint64_t *out, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QDR_H */
