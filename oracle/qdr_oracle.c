/*
 * qdr_oracle.c -- CPU oracle of the quantized gated delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY (see qdr_oracle.h).  Plain loops in the order the
 * method states them; no blocking, no fusion, no vector intrinsics.  Build
 * with:  gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread -lm
 *
 * Page citations use the short names defined in qdr_oracle.h.
 */
#include "qdr_oracle.h"

#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define D128 128

/* ------------------------------------------------------------------------ */
/* small helpers                                                             */
/* ------------------------------------------------------------------------ */

static int kind_is_int(int kind) { return kind == ORK_INT2 || kind == ORK_INT4 ||
                                          kind == ORK_INT6 || kind == ORK_INT8; }

/* Largest code of a symmetric b-bit integer grid: 2^(b-1) - 1, i.e. 1, 7, 31
 * or 127.  Symmetric uniform integer grid of the baseline and of STEPQuant's
 * integer units ([SLR] uniform-baseline paragraph). */
static float kind_qmax(int kind) { return (float)((1 << (kind - 1)) - 1); }

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* ------------------------------------------------------------------------ */
/* IEEE binary16, written from the format definition.                       */
/* FP16 pivots keep the riskiest units in half precision ([TUT] 四,         */
/* [REV] Method).  Rounding: to nearest, ties to even; overflow gives inf.   */
/* ------------------------------------------------------------------------ */

uint16_t or_f32_to_f16(float x) {
  uint32_t bits = f2u(x);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  uint32_t ex = (bits >> 23) & 0xFFu;
  uint32_t frac = bits & 0x7FFFFFu;
  if (ex == 0xFFu) {                       /* inf or NaN */
    if (frac == 0) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | 0x7E00u | (frac >> 13));
  }
  if (ex == 0) return sign;                /* fp32 zero or subnormal: < 2^-126 */
  uint32_t m = frac | 0x800000u;           /* value = m * 2^(ex-150) */
  if (ex >= 113) {                         /* binary16 normal range or overflow */
    uint32_t h = ((ex - 112u) << 10) | (frac >> 13);
    uint32_t rem = frac & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
    if (h >= 0x7C00u) h = 0x7C00u;         /* overflow to infinity */
    return (uint16_t)(sign | h);
  }
  /* binary16 subnormal: count units of 2^-24, value/2^-24 = m * 2^(ex-126) */
  uint32_t shift = 126u - ex;              /* >= 14 */
  if (shift >= 32u) return sign;
  uint32_t n = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (n & 1u))) n += 1u;
  return (uint16_t)(sign | n);
}

float or_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t ex = (h >> 10) & 0x1Fu;
  uint32_t frac = h & 0x3FFu;
  if (ex == 0x1Fu) return u2f(sign | 0x7F800000u | (frac << 13));
  if (ex == 0) {                           /* zero or subnormal: frac * 2^-24 */
    float mag = (float)frac * 0x1p-24f;    /* exact: frac < 2^10 */
    return sign ? -mag : mag;
  }
  return u2f(sign | ((ex + 112u) << 23) | (frac << 13));
}

/* ------------------------------------------------------------------------ */
/* Pairwise sum used for the row magnitude m_i.                              */
/* The pages name the statistic (a row's mean absolute value, [SLR] dual-    */
/* axis paragraph; the row magnitude of [TUT] 四) but not a summation order. */
/* Reading taken: a balanced pairwise sum that repeatedly folds the upper    */
/* half of the vector onto the lower half: x_l += x_{l+n/2}, n halves, until */
/* one value remains.  n must be a power of two.  x is overwritten.          */
/* ------------------------------------------------------------------------ */
float or_fold_sum(float *x, int n) {
  while (n > 1) {
    n /= 2;
    for (int l = 0; l < n; ++l) x[l] = x[l] + x[l + n];
  }
  return x[0];
}

/* ------------------------------------------------------------------------ */
/* Step a2: restore the previous state and apply the gate.                   */
/*                                                                           */
/* Dual-axis form X_ij = r_i * c_j * z_ij ([TUT] 四).  Reading taken for     */
/* mixed per-row widths: z is measured in units of the row's largest code    */
/* q_i, X_ij = r_i c_j z_ij / q_i, so one column factor serves rows of any   */
/* width.  Gate D = a_i on row i: the head-shared scalar alpha (GDN) or the  */
/* per-key-channel diagonal (KDA) ([TUT] 二, [SLR] GDN/KDA paragraph);       */
/* D acts before the delta factor, so it scales the restored rows.           */
/* fp32 order:  rho_i = r_i / q_i;  g_i = a_i * rho_i;                       */
/*              S'_ij = (z_ij * g_i) * c_j                                   */
/* FP16 rows: S'_ij = a_i * h_ij.  FP32 rows: S'_ij = a_i * s_ij.            */
/* ------------------------------------------------------------------------ */
void or_dequant(int d, const uint8_t *kinds, const uint32_t *e,
                const float *r, const float *c, const float *a, float *Sp) {
  for (int i = 0; i < d; ++i) {
    int kind = kinds[i];
    if (kind_is_int(kind)) {
      float rho = r[i] / kind_qmax(kind);
      float g = a[i] * rho;
      for (int j = 0; j < d; ++j) {
        float z = (float)(int32_t)e[i * d + j];
        float zg = z * g;
        Sp[i * d + j] = zg * c[j];
      }
    } else if (kind == ORK_FP16) {
      for (int j = 0; j < d; ++j)
        Sp[i * d + j] = a[i] * or_f16_to_f32((uint16_t)e[i * d + j]);
    } else {
      for (int j = 0; j < d; ++j) Sp[i * d + j] = a[i] * u2f(e[i * d + j]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Steps a3-a4: the delta rule ([TUT] 二):                                   */
/*   S_t = (I - beta k k^T) D S_{t-1} + beta k v^T.                          */
/* With S' = D S_{t-1} and u = S'^T k this equals S' + beta k (v - u)^T,     */
/* which is the form evaluated:                                              */
/*   u_j = sum_i k_i S'_ij   (fused multiply-add chain, i ascending, from 0) */
/*   delta_j = v_j - u_j;  b_i = beta * k_i;  S_ij = fma(b_i, delta_j, S'_ij)*/
/* The chain order is a reading (the pages give none).                       */
/* ------------------------------------------------------------------------ */
void or_delta_update(int d, const float *Sp, const float *k, const float *v,
                     float beta, float *S, float *u) {
  float *delta = (float *)malloc(sizeof(float) * (size_t)d);
  for (int j = 0; j < d; ++j) {
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) acc = fmaf(k[i], Sp[i * d + j], acc);
    if (u) u[j] = acc;
    delta[j] = v[j] - acc;
  }
  for (int i = 0; i < d; ++i) {
    float b = beta * k[i];
    for (int j = 0; j < d; ++j) S[i * d + j] = fmaf(b, delta[j], Sp[i * d + j]);
  }
  free(delta);
}

/* ------------------------------------------------------------------------ */
/* Step a5: readout o = S_t^T q from the updated floating-point state,       */
/* before it is quantised again ([SLR] generation-time paragraph; the output */
/* is state times query, [TUT] 三).  Accumulated in double, then rounded.    */
/* ------------------------------------------------------------------------ */
void or_readout(int d, const float *S, const float *q, float *o) {
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += (double)q[i] * (double)S[i * d + j];
    o[j] = (float)acc;
  }
}

/* Absolute scale of the readout: m_j = sum_i |q_i| |S_ij|, accumulated in   */
/* double, then rounded.  Not part of the step: it is the scale of the       */
/* rounding error of any evaluation order of o_j = sum_i q_i S_ij            */
/* (|fl(x.y) - x.y| <= gamma_n |x|.|y|), which the checks of a readout that  */
/* sums in another order need when the sum cancels.                          */
void or_readout_magnitude(int d, const float *S, const float *q, float *m) {
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += fabs((double)q[i]) * fabs((double)S[i * d + j]);
    m[j] = (float)acc;
  }
}

/* ------------------------------------------------------------------------ */
/* Steps a6-a8: refit the scales and quantise the updated state.             */
/*                                                                           */
/* Row factor ([TUT] 四, [SLR] dual-axis paragraph):  r_i = m_i^(1/2) w_i^(-1/2)
 *   with m_i the row's mean absolute value and w_i = omega_i the fixed
 *   row-impact weight.  fp32: m_i = foldsum(|S_i.|) * (1/d) (exact power of
 *   two), nu_i = m_i / omega_i, r_i = sqrt(nu_i); r_i = 1 when nu_i == 0.
 * Uniform baseline ([SLR] uniform-baseline paragraph): scale from the key
 *   row's absolute maximum: r_i = max_j |S_ij|, r_i = 1 when that is below
 *   the smallest normal fp32; no column factor (c_j = 1).
 * Column factor ([TUT] 四, [REV] Method): fitted so the omega-weighted squared
 *   reconstruction error is small.  Reading taken (the fitting procedure is
 *   not given): V0, the smallest factor that needs no clipping,
 *   c_j = max_i |S_ij / r_i| over integer rows (1 when below the smallest
 *   normal fp32); optional V1a (fit_iters = 1): for the codes chosen with V0,
 *   the exact weighted least-squares factor
 *     c_j = sum_i omega_i r_i S_ij zeta_ij / sum_i omega_i r_i^2 zeta_ij^2
 *   with zeta = z / q_i and omega_i r_i^2 = m_i, so the weights are m_i;
 *   each sum is two fma chains, one per half of the rows, then added (order
 *   not given by the pages: reading taken).
 * Codes: z_ij = nearest integer (ties to even) to the exact real product
 *   Y_ij * w_ij, where Y_ij = S_ij * (1/r_i) and w_ij = (1/c0_j) * q_i, each
 *   rounded to fp32.  |z| <= q_i always holds, so no clipping is needed.
 * FP16 rows: binary16 of S.  FP32 rows: S itself.
 * Non-integer rows take no part in r or c; their r_i is stored as 0.
 */
/* ---- bfloat16 factors (compact scale storage, the compact-bits paragraph
 * of [SLR] counts 16-bit factors).  A bfloat16 value is a binary32 value
 * whose low 16 bits are zero.  Reading taken: the row factor and the
 * clip-free column factor are rounded UP before the codes are computed from
 * them (so |Y| <= 1 still holds and no code leaves +-q), a refitted column
 * factor is rounded to nearest; the restore uses the stored values. */
static float bf16_toward_zero(float x) { return u2f(f2u(x) & 0xFFFF0000u); }
static float bf16_away(float t) { return u2f(f2u(t) + 0x10000u); }  /* next bfloat16 away from 0 */

float or_bf16_up(float x) {
  float t = bf16_toward_zero(x);
  return (t < x) ? bf16_away(t) : t;
}

float or_bf16_nearest(float x) {
  float lo = bf16_toward_zero(x);
  if (lo == x) return x;
  float hi = bf16_away(lo);
  double dl = fabs((double)x - (double)lo), dh = fabs((double)hi - (double)x);
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (f2u(lo) & 0x10000u) ? hi : lo;
}

void or_requant(int d, const uint8_t *kinds, const float *S,
                const float *omega, int scale_mode, int fit_iters,
                int scale_bits, uint32_t *e, float *r, float *c,
                float *m_out) {
  const int b16 = scale_bits == 16;
  float *tmp = (float *)malloc(sizeof(float) * (size_t)d);
  float *ir = (float *)malloc(sizeof(float) * (size_t)d);
  float *m = (float *)malloc(sizeof(float) * (size_t)d);
  const float inv_d = 1.0f / (float)d;

  /* row factors, and the non-integer rows */
  for (int i = 0; i < d; ++i) {
    int kind = kinds[i];
    m[i] = 0.0f;
    ir[i] = 0.0f;
    if (kind == ORK_FP32) {
      for (int j = 0; j < d; ++j) e[i * d + j] = f2u(S[i * d + j]);
      r[i] = 0.0f;
      continue;
    }
    if (kind == ORK_FP16) {
      for (int j = 0; j < d; ++j) e[i * d + j] = or_f32_to_f16(S[i * d + j]);
      r[i] = 0.0f;
      continue;
    }
    if (scale_mode == OR_SCALE_DUAL) {
      for (int j = 0; j < d; ++j) tmp[j] = fabsf(S[i * d + j]);
      m[i] = or_fold_sum(tmp, d) * inv_d;
      float nu = m[i] / omega[i];
      r[i] = (nu == 0.0f) ? 1.0f : sqrtf(nu);
    } else {
      float mx = 0.0f;
      for (int j = 0; j < d; ++j) mx = fmaxf(mx, fabsf(S[i * d + j]));
      r[i] = (mx < FLT_MIN) ? 1.0f : mx;
    }
    if (b16) r[i] = or_bf16_up(r[i]);
    ir[i] = 1.0f / r[i];
  }

  /* column factors and codes */
  for (int j = 0; j < d; ++j) {
    float c0 = 1.0f;
    if (scale_mode == OR_SCALE_DUAL) {
      float mx = 0.0f;
      for (int i = 0; i < d; ++i)
        if (kind_is_int(kinds[i])) mx = fmaxf(mx, fabsf(S[i * d + j] * ir[i]));
      c0 = (mx < FLT_MIN) ? 1.0f : mx;
      if (b16) c0 = or_bf16_up(c0);
    }
    float ec = 1.0f / c0;
    /* refit sums: one fma chain over each half of the rows (rows 0..d/2-1
     * and d/2..d-1, each ascending from +0), then the two halves added */
    float num[2] = {0.0f, 0.0f}, den[2] = {0.0f, 0.0f};
    for (int i = 0; i < d; ++i) {
      int kind = kinds[i];
      if (!kind_is_int(kind)) continue;
      float q = kind_qmax(kind);
      float y = S[i * d + j] * ir[i];
      float w = ec * q;
      double z = rint((double)y * (double)w);   /* exact product, then RNE */
      e[i * d + j] = (uint32_t)(int32_t)z;
      if (fit_iters > 0) {
        const int half = i < d / 2 ? 0 : 1;
        float zeta = (float)z * (1.0f / q);
        float p = m[i] * zeta;
        num[half] = fmaf(p, y, num[half]);
        den[half] = fmaf(p, zeta, den[half]);
      }
    }
    const float num_all = num[0] + num[1], den_all = den[0] + den[1];
    c[j] = (fit_iters > 0 && den_all > 0.0f) ? num_all / den_all : c0;
    if (b16 && fit_iters > 0) c[j] = or_bf16_nearest(c[j]);
  }
  if (m_out) memcpy(m_out, m, sizeof(float) * (size_t)d);
  free(tmp);
  free(ir);
  free(m);
}

/* ------------------------------------------------------------------------ */
/* One decode step on a decoded head.  Order of work at generation time      */
/* ([SLR] generation-time paragraph): restore the previous state, update and */
/* read out in floating point, then quantise and store, so the error made    */
/* now first acts on the next step.                                          */
/* ------------------------------------------------------------------------ */
void or_head_step(int d, const uint8_t *kinds, uint32_t *e, float *r,
                  float *c, const float *omega, int scale_mode,
                  int fit_iters, int scale_bits, const float *q, const float *k,
                  const float *v, float beta, const float *a, float *o,
                  float *S_pre) {
  size_t nn = (size_t)d * (size_t)d;
  float *Sp = (float *)malloc(sizeof(float) * nn);
  float *S = (float *)malloc(sizeof(float) * nn);
  or_dequant(d, kinds, e, r, c, a, Sp);
  or_delta_update(d, Sp, k, v, beta, S, NULL);
  or_readout(d, S, q, o);
  if (S_pre) memcpy(S_pre, S, sizeof(float) * nn);
  or_requant(d, kinds, S, omega, scale_mode, fit_iters, scale_bits, e, r, c, NULL);
  free(Sp);
  free(S);
}

/* ------------------------------------------------------------------------ */
/* Byte layout of one (slot, head) block, d = 128.  The pages fix no layout; */
/* this is the layout chosen for the pool (its definition is restated here   */
/* independently of the device library):                                     */
/*  - the code stream of column j holds rows 0..127 in order, row i as a     */
/*    field of b_i bits (b = 2,4,6,8 integer codes, 16 binary16, 32          */
/*    binary32); stream bit p is bit p%8 of stream byte p/8;                 */
/*  - integer codes are stored as b-bit two's complement;                    */
/*  - the stream is cut into granules of G bytes (G = 16 for whole-head      */
/*    units, 4 for row units); rows 0..63 fill the first granules and rows   */
/*    64..127 start on a fresh granule, each half zero-padded to whole       */
/*    granules; granule g of column j sits at byte (g*128 + j)*G;            */
/*  - then, if any row is an integer row: r[128] fp32, and in dual-axis mode */
/*    c[128] fp32;                                                           */
/*  - the block is zero-padded to a multiple of 256 bytes.                   */
/* ------------------------------------------------------------------------ */
static int granule_bytes(int unit) { return unit == OR_UNIT_HEAD ? 16 : 4; }

static int any_int_row(const uint8_t *kinds) {
  for (int i = 0; i < D128; ++i)
    if (kind_is_int(kinds[i])) return 1;
  return 0;
}

/* granules of one half (rows lo..lo+63) of a column stream */
static size_t half_granules(const uint8_t *kinds, int unit, int lo) {
  size_t bits = 0;
  for (int i = lo; i < lo + 64; ++i) bits += kinds[i];
  size_t gbits = (size_t)granule_bytes(unit) * 8u;
  return (bits + gbits - 1) / gbits;
}

/* first stream bit of row i */
static size_t row_start_bit(const uint8_t *kinds, int unit, int i) {
  size_t p = 0;
  int lo = 0;
  if (i >= 64) {
    p = half_granules(kinds, unit, 0) * (size_t)granule_bytes(unit) * 8u;
    lo = 64;
  }
  for (int t = lo; t < i; ++t) p += kinds[t];
  return p;
}

size_t or_code_bytes(const uint8_t *kinds, int unit) {
  size_t ng = half_granules(kinds, unit, 0) + half_granules(kinds, unit, 64);
  return ng * D128 * (size_t)granule_bytes(unit);
}

static size_t factor_bytes(int scale_bits) { return scale_bits == 16 ? 2u : 4u; }

static size_t scale_bytes(const uint8_t *kinds, int scale_mode, int scale_bits) {
  if (!any_int_row(kinds)) return 0;
  return (scale_mode == OR_SCALE_DUAL ? 2u : 1u) * D128 * factor_bytes(scale_bits);
}

size_t or_block_bytes(const uint8_t *kinds, int unit, int scale_mode, int scale_bits) {
  size_t n = or_code_bytes(kinds, unit) + scale_bytes(kinds, scale_mode, scale_bits);
  return (n + 255u) / 256u * 256u;
}

/* byte n of column j's stream -> byte offset in the block */
static size_t stream_byte(int unit, int j, size_t n) {
  size_t G = (size_t)granule_bytes(unit);
  return ((n / G) * D128 + (size_t)j) * G + n % G;
}

static uint32_t field_of(int kind, uint32_t e) {
  if (kind_is_int(kind)) return e & ((1u << kind) - 1u);   /* low b bits of z */
  return e;   /* FP16 bits or FP32 bits */
}

/* one factor array at block + off: binary32, or the upper halves (bfloat16) */
static void put_factors(uint8_t *dst, const float *x, int scale_bits) {
  for (int i = 0; i < D128; ++i) {
    uint32_t u = f2u(x[i]);
    if (scale_bits == 16) {
      uint16_t h = (uint16_t)(u >> 16);
      memcpy(dst + 2 * i, &h, 2);
    } else {
      memcpy(dst + 4 * i, &u, 4);
    }
  }
}

static void get_factors(const uint8_t *src, float *x, int scale_bits) {
  for (int i = 0; i < D128; ++i) {
    if (scale_bits == 16) {
      uint16_t h;
      memcpy(&h, src + 2 * i, 2);
      x[i] = u2f((uint32_t)h << 16);
    } else {
      memcpy(&x[i], src + 4 * i, 4);
    }
  }
}

void or_encode_block(const uint8_t *kinds, int unit, int scale_mode, int scale_bits,
                     const uint32_t *e, const float *r, const float *c,
                     uint8_t *block) {
  size_t total = or_block_bytes(kinds, unit, scale_mode, scale_bits);
  memset(block, 0, total);
  for (int j = 0; j < D128; ++j) {
    for (int i = 0; i < D128; ++i) {
      int w = kinds[i];
      size_t p = row_start_bit(kinds, unit, i);
      uint32_t f = field_of(kinds[i], e[i * D128 + j]);
      for (int t = 0; t < w; ++t, ++p) {
        if ((f >> t) & 1u) block[stream_byte(unit, j, p / 8)] |= (uint8_t)(1u << (p % 8));
      }
    }
  }
  size_t off = or_code_bytes(kinds, unit);
  if (any_int_row(kinds)) {
    put_factors(block + off, r, scale_bits);
    if (scale_mode == OR_SCALE_DUAL) put_factors(block + off + D128 * factor_bytes(scale_bits), c, scale_bits);
  }
}

void or_decode_block(const uint8_t *kinds, int unit, int scale_mode, int scale_bits,
                     const uint8_t *block, uint32_t *e, float *r, float *c) {
  for (int j = 0; j < D128; ++j) {
    for (int i = 0; i < D128; ++i) {
      int w = kinds[i];
      size_t p = row_start_bit(kinds, unit, i);
      uint32_t f = 0;
      for (int t = 0; t < w; ++t, ++p)
        if ((block[stream_byte(unit, j, p / 8)] >> (p % 8)) & 1u) f |= 1u << t;
      if (kind_is_int(kinds[i]))   /* sign-extend the b-bit field */
        e[i * D128 + j] = (f & (1u << (w - 1))) ? (f | ~((1u << w) - 1u)) : f;
      else
        e[i * D128 + j] = f;
    }
  }
  size_t off = or_code_bytes(kinds, unit);
  for (int i = 0; i < D128; ++i) r[i] = 0.0f;
  for (int j = 0; j < D128; ++j) c[j] = 1.0f;
  if (any_int_row(kinds)) {
    get_factors(block + off, r, scale_bits);
    if (scale_mode == OR_SCALE_DUAL) get_factors(block + off + D128 * factor_bytes(scale_bits), c, scale_bits);
  }
}

/* ------------------------------------------------------------------------ */
/* Pool: (num_slots) slots; one slot holds every head's block back to back.  */
/* The slot table maps requests to slots ((5B+1) slots per the serving       */
/* memory accounting quoted in the zhichai.net discussion).                  */
/* ------------------------------------------------------------------------ */
/* stored factor width of a pool (0 means binary32) */
static int SB(const or_pool_desc *desc) { return desc->scale_bits == 16 ? 16 : 32; }

static void head_kinds(const or_pool_desc *desc, int h, uint8_t *out) {
  for (int i = 0; i < D128; ++i)
    out[i] = desc->unit == OR_UNIT_HEAD ? desc->kinds[h]
                                        : desc->kinds[(size_t)h * D128 + i];
}

int or_pool_layout(const or_pool_desc *desc, uint64_t *head_off,
                   uint64_t *slot_stride, uint64_t *total) {
  uint8_t kinds[D128];
  uint64_t off = 0;
  for (int h = 0; h < desc->num_heads; ++h) {
    head_kinds(desc, h, kinds);
    if (head_off) head_off[h] = off;
    off += or_block_bytes(kinds, desc->unit, desc->scale_mode, SB(desc));
  }
  if (slot_stride) *slot_stride = off;
  if (total) *total = off * (uint64_t)desc->num_slots;
  return 0;
}

typedef struct {
  const or_pool_desc *desc;
  uint8_t *pool;
  const uint8_t *cpool;
  const uint64_t *head_off;
  uint64_t stride;
  const int32_t *slots;
  int32_t nreq;
  const float *q, *k, *v, *beta, *gate;
  float *o;
  float *o_mag;            /* optional: readout magnitude per (b, h, j) */
  const float *S_in;
  float *S_out;
  int op;                  /* 0 step, 1 pack, 2 unpack */
  int64_t first, last;     /* item range [first, last) over nreq*H */
  int bad;
} work_t;

static void run_items(work_t *w) {
  const or_pool_desc *desc = w->desc;
  const int H = desc->num_heads;
  const size_t nn = (size_t)D128 * D128;
  uint8_t kinds[D128];
  uint32_t *e = (uint32_t *)malloc(sizeof(uint32_t) * nn);
  float *S = (float *)malloc(sizeof(float) * nn);
  float r[D128], c[D128], a[D128];
  for (int64_t it = w->first; it < w->last; ++it) {
    int32_t b = (int32_t)(it / H);
    int h = (int)(it % H);
    int32_t slot = w->slots[b];
    size_t vec = ((size_t)b * H + (size_t)h) * D128;
    if (slot < 0 || slot >= desc->num_slots) {
      if (slot >= desc->num_slots || slot < -1) w->bad++;
      if (w->op == 0) memset(w->o + vec, 0, sizeof(float) * D128);
      if (w->op == 0 && w->o_mag) memset(w->o_mag + vec, 0, sizeof(float) * D128);
      if (w->op == 2) memset(w->S_out + ((size_t)b * H + h) * nn, 0, sizeof(float) * nn);
      continue;
    }
    head_kinds(desc, h, kinds);
    size_t boff = (size_t)slot * w->stride + w->head_off[h];
    if (w->op == 0) {
      const float *omega = desc->omega + (size_t)h * D128;
      or_decode_block(kinds, desc->unit, desc->scale_mode, SB(desc), w->pool + boff, e, r, c);
      for (int i = 0; i < D128; ++i)
        a[i] = desc->gate == OR_GATE_SCALAR ? w->gate[(size_t)b * H + h] : w->gate[vec + i];
      or_head_step(D128, kinds, e, r, c, omega, desc->scale_mode, desc->fit_iters, SB(desc),
                   w->q + vec, w->k + vec, w->v + vec, w->beta[(size_t)b * H + h], a,
                   w->o + vec, w->o_mag ? S : NULL);
      if (w->o_mag) or_readout_magnitude(D128, S, w->q + vec, w->o_mag + vec);
      or_encode_block(kinds, desc->unit, desc->scale_mode, SB(desc), e, r, c, w->pool + boff);
    } else if (w->op == 1) {
      const float *omega = desc->omega + (size_t)h * D128;
      or_requant(D128, kinds, w->S_in + ((size_t)b * H + h) * nn, omega, desc->scale_mode,
                 desc->fit_iters, SB(desc), e, r, c, NULL);
      or_encode_block(kinds, desc->unit, desc->scale_mode, SB(desc), e, r, c, w->pool + boff);
    } else {
      for (int i = 0; i < D128; ++i) a[i] = 1.0f;
      or_decode_block(kinds, desc->unit, desc->scale_mode, SB(desc), w->cpool + boff, e, r, c);
      or_dequant(D128, kinds, e, r, c, a, w->S_out + ((size_t)b * H + h) * nn);
    }
  }
  free(e);
  free(S);
}

static void *thread_main(void *arg) { run_items((work_t *)arg); return NULL; }

static int run_pool(work_t *proto, int threads) {
  const int H = proto->desc->num_heads;
  uint64_t *head_off = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)H);
  uint64_t stride = 0;
  or_pool_layout(proto->desc, head_off, &stride, NULL);
  proto->head_off = head_off;
  proto->stride = stride;
  int64_t items = (int64_t)proto->nreq * H;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  work_t *ws = (work_t *)calloc((size_t)threads, sizeof(work_t));
  pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
  for (int t = 0; t < threads; ++t) {
    ws[t] = *proto;
    ws[t].first = items * t / threads;
    ws[t].last = items * (t + 1) / threads;
    ws[t].bad = 0;
  }
  if (threads == 1) {
    run_items(&ws[0]);
  } else {
    for (int t = 0; t < threads; ++t) pthread_create(&tid[t], NULL, thread_main, &ws[t]);
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
  }
  int bad = 0;
  for (int t = 0; t < threads; ++t) bad += ws[t].bad;
  free(ws);
  free(tid);
  free(head_off);
  /* a slot listed for every head counts once per request */
  return H > 0 ? bad / H : 0;
}

int or_pool_step(const or_pool_desc *desc, uint8_t *pool,
                 const int32_t *slots, int32_t B, const float *q,
                 const float *k, const float *v, const float *beta,
                 const float *gate, float *o, int threads, float *o_mag) {
  work_t w;
  memset(&w, 0, sizeof w);
  w.desc = desc; w.pool = pool; w.slots = slots; w.nreq = B;
  w.q = q; w.k = k; w.v = v; w.beta = beta; w.gate = gate; w.o = o; w.o_mag = o_mag;
  w.op = 0;
  return run_pool(&w, threads);
}

int or_pool_pack(const or_pool_desc *desc, uint8_t *pool,
                 const int32_t *slots, int32_t n, const float *S, int threads) {
  work_t w;
  memset(&w, 0, sizeof w);
  w.desc = desc; w.pool = pool; w.slots = slots; w.nreq = n; w.S_in = S;
  w.op = 1;
  return run_pool(&w, threads);
}

int or_pool_unpack(const or_pool_desc *desc, const uint8_t *pool,
                   const int32_t *slots, int32_t n, float *S, int threads) {
  work_t w;
  memset(&w, 0, sizeof w);
  w.desc = desc; w.cpool = pool; w.slots = slots; w.nreq = n; w.S_out = S;
  w.op = 2;
  return run_pool(&w, threads);
}
