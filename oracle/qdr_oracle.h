/*
 * qdr_oracle.h -- CPU oracle of the quantized gated delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the HIP
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or constant with the HIP library: the byte layout and the arithmetic are
 * written out here a second time, from the same written definition.
 *
 * Sources (the pages describing STEPQuant):
 *   [TUT]  tutorial "STEPQuant：取代 KV cache 的状态，6-bit 量化精度不掉"
 *          (bloombook.cn), sections 二 (gated delta rule, error recursion),
 *          三 (lifetime weight, row impact), 四 (allocation, pivots,
 *          dual-axis row/column factors, fused online kernel).
 *   [REV]  review "STEPQuant: When and Where Errors Matter in Delta-Rule
 *          Recurrent State Quantization" (ai-trend.me), Method and Key terms.
 *   [SLR]  review "STEPQuant：誤差の寿命と位置から設計するDelta則の再帰状態量子化"
 *          (singularity-lens.com), paragraphs on the uniform baseline, the
 *          dual-axis fit and the order of work at generation time.
 *
 * Every function states which passage it follows.  Where the pages leave a
 * step open (summation order, rounding, degenerate cases, byte layout) the
 * reading taken is stated at the function.
 *
 * Floating point: the state is fp32 (the pages' uncompressed baseline keeps
 * the recurrent state in FP32, [TUT] 一/五, [REV] Results).  All state
 * arithmetic below is IEEE binary32 with round-to-nearest-even, one rounding
 * per written operation, fused multiply-add only where fmaf() is written,
 * subnormals kept.  The file must be compiled with -ffp-contract=off.
 */
#ifndef QDR_ORACLE_H
#define QDR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage kinds of one key row.  The value is the bit width of one element. */
enum {
  ORK_INT2 = 2, ORK_INT4 = 4, ORK_INT6 = 6, ORK_INT8 = 8,
  ORK_FP16 = 16, ORK_FP32 = 32
};
enum { OR_UNIT_HEAD = 0, OR_UNIT_ROW = 1 };
enum { OR_SCALE_DUAL = 0, OR_SCALE_ROW_ABSMAX = 1 };
enum { OR_GATE_SCALAR = 0, OR_GATE_DIAG = 1 };

/* ---- IEEE binary16 (pivot storage) ------------------------------------- */
uint16_t or_f32_to_f16(float x);   /* round to nearest even, overflow -> inf */
float    or_f16_to_f32(uint16_t h);/* exact                                  */

/* ---- dense per-head arithmetic (generic dimension d, a power of two) ---- */
/*
 * A quantised head in "decoded" form: for row i of kind K,
 *   INT rows : e[i*d+j] holds the signed integer code z_ij (as int32 bits),
 *   FP16 rows: e[i*d+j] holds the binary16 bits,
 *   FP32 rows: e[i*d+j] holds the binary32 bits,
 * plus r[d] (row factors) and c[d] (column factors).
 */
void or_dequant(int d, const uint8_t *kinds, const uint32_t *e,
                const float *r, const float *c, const float *a,
                float *Sp);
void or_delta_update(int d, const float *Sp, const float *k, const float *v,
                     float beta, float *S, float *u);
void or_readout(int d, const float *S, const float *q, float *o);
/* m_j = sum_i |q_i| |S_ij| (double accumulation): the error scale of any
 * summation order of the readout, for checks only. */
void or_readout_magnitude(int d, const float *S, const float *q, float *m);
void or_requant(int d, const uint8_t *kinds, const float *S,
                const float *omega, int scale_mode, int fit_iters,
                int scale_bits, uint32_t *e, float *r, float *c,
                float *m_out);
float or_fold_sum(float *x, int n);

/* One whole step on a decoded head: dequant+gate, delta update, readout,
 * requantisation.  e/r/c are updated in place.  S_pre (optional, may be
 * NULL) receives the updated fp32 state before requantisation. */
void or_head_step(int d, const uint8_t *kinds, uint32_t *e, float *r,
                  float *c, const float *omega, int scale_mode,
                  int fit_iters, int scale_bits, const float *q, const float *k,
                  const float *v, float beta, const float *a, float *o,
                  float *S_pre);

/* ---- byte layout of one (slot, head) block, d = 128 --------------------- */
/* scale_bits: 32 stores r and c as binary32, 16 as bfloat16 (the upper 16
 * bits of the binary32 value, which the factors then are exactly). */
size_t or_block_bytes(const uint8_t *kinds, int unit, int scale_mode, int scale_bits);
size_t or_code_bytes(const uint8_t *kinds, int unit);
void or_encode_block(const uint8_t *kinds, int unit, int scale_mode, int scale_bits,
                     const uint32_t *e, const float *r, const float *c,
                     uint8_t *block);
void or_decode_block(const uint8_t *kinds, int unit, int scale_mode, int scale_bits,
                     const uint8_t *block, uint32_t *e, float *r, float *c);
/* bfloat16 rounding of the factors: up (smallest bfloat16 >= x, x >= 0) and
 * to nearest (ties to an even last bit). */
float or_bf16_up(float x);
float or_bf16_nearest(float x);

/* ---- whole pool (host memory image of the device pool) ------------------ */
typedef struct {
  int32_t num_slots, num_heads;
  int32_t unit, gate, scale_mode, fit_iters;
  const uint8_t *kinds;  /* [H] (UNIT_HEAD) or [H*128] (UNIT_ROW) */
  const float *omega;    /* [H*128]                               */
  int32_t scale_bits;    /* 32 (or 0): binary32 factors; 16: bfloat16 */
} or_pool_desc;

/* Per-head block offsets inside one slot, the slot stride and total bytes. */
int or_pool_layout(const or_pool_desc *desc, uint64_t *head_off,
                   uint64_t *slot_stride, uint64_t *total);

/* Step every (b, h) with slots[b] >= 0 in a host pool image.  Returns the
 * number of out-of-range slots (their o rows are zeroed; padding slots -1
 * also give zero o).  threads <= 1 runs on the calling thread.  o_mag
 * (optional, may be NULL): [B][H][128] readout magnitudes
 * (or_readout_magnitude of each updated state). */
int or_pool_step(const or_pool_desc *desc, uint8_t *pool,
                 const int32_t *slots, int32_t B, const float *q,
                 const float *k, const float *v, const float *beta,
                 const float *gate, float *o, int threads, float *o_mag);
/* Encode dense fp32 states S[n][H][128][128] into the listed slots. */
int or_pool_pack(const or_pool_desc *desc, uint8_t *pool,
                 const int32_t *slots, int32_t n, const float *S, int threads);
/* Decode the listed slots to dense fp32 S[n][H][128][128]. */
int or_pool_unpack(const or_pool_desc *desc, const uint8_t *pool,
                   const int32_t *slots, int32_t n, float *S, int threads);

#ifdef __cplusplus
}
#endif
#endif
