#pragma once
// qdr_device.h -- CDNA4 (gfx950) kernels of the quantized gated delta-rule
// decode step.
//
// One workgroup of 128 threads (two wave64s) owns one (request, head) 128x128
// state.  Wave w holds key rows 64w..64w+63; lane l holds value columns l and
// l+64 of those rows, so the whole fp32 tile lives in 128 VGPRs per lane:
//   * column sums (u = S'^T k, o = S^T q, the column maximum of the scale fit)
//     are lane-local fma chains;
//   * row sums (the row magnitude m_i) are a lane-local pair add followed by a
//     transpose-reduce: v_permlane32_swap, v_permlane16_swap, then one LDS
//     hop for the last sixteen partials;
//   * every per-row scalar (gate * row factor, k_i, beta*k_i, q_i, 1/r_i) is
//     broadcast from LDS, so VALU instructions never exceed the one-SGPR limit.
// Codes stream in and out as 16-byte granules laid out so that one wave
// instruction touches 1 KiB of consecutive bytes.
//
// Arithmetic order (must match the written specification bit for bit):
//   restore  rho_i = r_i / q_i, g_i = a_i * rho_i, S'_ij = (z_ij * g_i) * c_j
//   update   u_j = fma chain over i ascending, delta_j = v_j - u_j,
//            b_i = beta * k_i, S_ij = fma(b_i, delta_j, S'_ij)
//   scales   m_i = foldsum_j |S_ij| * 2^-7, r_i = sqrt(m_i / omega_i) (1 if the
//            quotient is 0), Y = S * (1/r_i), c0_j = max_i |Y_ij| (1 if below
//            2^-126), z = nearest-even(Y * ((1/c0_j) * q)) of the exact product
// Page references: gated delta rule and gate forms, tutorial
// "STEPQuant：取代 KV cache 的状态，6-bit 量化精度不掉" §二; dual-axis factors,
// pivots and the fused online kernel, same tutorial §四; restore / update /
// read out / quantise order, review "STEPQuant：誤差の寿命と位置から設計する
// Delta則の再帰状態量子化", generation-time paragraph.
#include <float.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdr_internal.h"

namespace qdr {

namespace {

// 1.5 * 2^23: adding it to |x| < 2^22 leaves round-to-nearest-even(x) in the
// low mantissa bits (two's complement), so fma(Y, w, kMagic) both rounds the
// exact product Y*w and yields the code's bit pattern.
constexpr float kMagic = 12582912.0f;

// Scheduling fences between groups of rows keep the unrolled loops from
// hoisting whole phases (which would hold every unpacked code next to the
// tile); LDS and global reads may still move up, so the next group's
// row scalars are fetched while the current group computes.
#define QDR_FENCE() __builtin_amdgcn_sched_barrier(0x0120)

template <int BITS>
struct Kind {
  static constexpr bool is_int = BITS <= 8;
  static constexpr int qmax_i = is_int ? (1 << (BITS - 1)) - 1 : 0;
  static constexpr int NG = BITS / 2;   // 16-byte granules per column half
  static constexpr int NW = BITS * 2;   // 32-bit words per column half
};

__device__ __forceinline__ float rn_div(float a, float b) { return __fdiv_rn(a, b); }

// Pins x to an fp32 register: an empty asm statement with a read-write VGPR
// operand.  Without it the compiler folds fp16_round(fma(a, b, c)) into one
// mixed-precision fma that rounds the exact result to fp16 once, which
// differs from rounding to fp32 first (the state is fp32) at fp16 ties.
__device__ __forceinline__ float pin_f32(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Correctly rounded square root of a finite x >= 0.  v_sqrt_f32 is accurate
// to one ulp; the neighbours s-ulp and s+ulp are then tested exactly: for
// adjacent floats a < b, a*b equals the squared midpoint minus (b-a)^2/4, and
// no float lies strictly between the two, so the sign of the single-rounded
// residual x - a*b (an fma) tells on which side of the midpoint sqrt(x) lies.
// Inputs below 2^-100 are scaled by 2^64 first so the residuals stay
// representable.  (A square root is never exactly halfway between floats.)
__device__ __forceinline__ float rn_sqrt(float x) {
  const bool tiny = x < 0x1p-100f;
  const float xs = tiny ? x * 0x1p64f : x;
  float s = __builtin_amdgcn_sqrtf(xs);
  const float s_dn = __uint_as_float(__float_as_uint(s) - 1u);
  const float s_up = __uint_as_float(__float_as_uint(s) + 1u);
  const float r_dn = __builtin_fmaf(-s_dn, s, xs);
  const float r_up = __builtin_fmaf(-s_up, s, xs);
  s = (r_dn <= 0.0f) ? s_dn : s;
  s = (r_up > 0.0f) ? s_up : s;
  return tiny ? s * 0x1p-32f : s;
}

// b-bit field number `ii` of a column-half stream held in w[] (two's
// complement for integer kinds, raw bits otherwise).
template <int BITS>
__device__ __forceinline__ uint32_t field_bits(const uint32_t *w, int ii) {
  const int p = ii * BITS, d = p >> 5, s = p & 31;
  if (BITS == 32) return w[d];
  if (s + BITS <= 32) return w[d] >> s;
  return __builtin_amdgcn_alignbit(w[d + 1], w[d], s);
}

// n/16 for the 4-bit two's complement integer n in the low nibble of byte
// SEL of w: v_cvt_off_f32_i4 (exact: n/16 has at most 4 significant bits)
// reading its operand through an SDWA byte select.
template <int SEL>
__device__ __forceinline__ float nibble_over16(uint32_t w) {
  float r;
  if (SEL == 0) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if (SEL == 1) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if (SEL == 2) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  else asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}

// INT4 field ii of a column-half stream as z/16 (nibble 2k of a word is the
// low nibble of byte k, nibble 2k+1 the low nibble of byte k after a 4-bit
// shift of the whole word).
__device__ __forceinline__ float int4_field_over16(const uint32_t *w, int ii) {
  const int d = ii >> 3, nib = ii & 7;
  const uint32_t x = (nib & 1) ? (w[d] >> 4) : w[d];
  switch (nib >> 1) {
    case 0: return nibble_over16<0>(x);
    case 1: return nibble_over16<1>(x);
    case 2: return nibble_over16<2>(x);
    default: return nibble_over16<3>(x);
  }
}

// Sign-extended low `width` bits of x (v_bfe_i32 with a wave-uniform width
// operand).  Written as a single instruction so that the result is known to
// the compiler only as a signed 32-bit value.
__device__ __forceinline__ int32_t sext_low(uint32_t x, uint32_t width) {
  int32_t r;
  asm("v_bfe_i32 %0, %1, 0, %2" : "=v"(r) : "v"(x), "s"(width));
  return r;
}

template <int BITS>
__device__ __forceinline__ float field_int_as_float(const uint32_t *w, int ii) {
  const int p = ii * BITS, d = p >> 5, s = p & 31;
  if (BITS == 8) return (float)(int)(int8_t)(uint8_t)(w[d] >> s);
  int32_t x;
  if (s + BITS <= 32)
    x = __builtin_amdgcn_sbfe((int32_t)w[d], s, BITS);
  else
    x = __builtin_amdgcn_sbfe((int32_t)__builtin_amdgcn_alignbit(w[d + 1], w[d], s), 0, BITS);
  return (float)x;
}

// Append field `ii` (low BITS bits of f) to the output stream: funnel shifts
// bring the new bits in from the top, so bits above BITS never reach memory.
template <int BITS>
__device__ __forceinline__ void put_field(uint32_t *out, uint32_t &acc, uint32_t f, int ii) {
  const int p = ii * BITS, d = p >> 5, s = p & 31;
  if (BITS == 32) { out[d] = f; return; }
  if (s + BITS < 32) {
    acc = __builtin_amdgcn_alignbit(f, acc, BITS);
  } else if (s + BITS == 32) {
    acc = __builtin_amdgcn_alignbit(f, acc, BITS);
    out[d] = acc;
  } else {
    acc = __builtin_amdgcn_alignbit(f, acc, 32 - s);
    out[d] = acc;
    // the next word starts from f alone: whatever lies below f in the
    // window is shifted out before that word is complete, so the word does
    // not depend on this one (shorter dependency chains)
    acc = __builtin_amdgcn_alignbit(f, 0u, BITS);
  }
}

// Block accesses go through a buffer resource (base and size of the block in
// SGPRs): a code granule is (scalar offset of granule row g of this wave) +
// (one 32-bit lane offset), so no per-granule 64-bit vector address stays
// live between the loads and the stores, and accesses past the block end are
// dropped by the hardware range check.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) dword access on CDNA

// Code granules are read once per step: nontemporal (nt) loads.
// A lane offset past every block's buffer range: a raw buffer load there
// returns zeros without touching memory.
constexpr uint32_t kBeyondBuffer = 0x80000000u;

__device__ __forceinline__ uint4 load_granule(rsrc_t rs, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// A 16-byte store may read its data registers after the next instructions
// have issued.  The compiler keeps those registers untouched for the
// required wait state only when the store has no scalar offset register (it
// takes a store with an SGPR soffset to have read its data already); on this
// GPU that does not hold -- an overwrite right behind such a store reached
// memory for some lanes -- so the whole offset goes into the lane offset and
// soffset is the constant 0.
__device__ __forceinline__ void store_granule(rsrc_t rs, uint4 t, uint32_t voff, uint32_t soff) {
  __attribute__((ext_vector_type(4))) unsigned int v = {t.x, t.y, t.z, t.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff + soff, 0, 2);   // nontemporal: written once per step
}

__device__ __forceinline__ float load_f32(rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
}

__device__ __forceinline__ void store_f32(rsrc_t rs, float x, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32((int)__float_as_uint(x), rs, voff, soff, 0);
}

__device__ __forceinline__ void store_u32(rsrc_t rs, uint32_t x, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32((int)x, rs, voff, soff, 0);
}

// ---- Scale storage.  The SCALE template argument: bit 0 clear = dual-axis
// factors (r and c), set = per-row absmax (r only); bit 1 set = the factors
// are stored as bfloat16 instead of fp32.
constexpr bool dual(int scale) { return (scale & 1) == 0; }
constexpr bool sc16(int scale) { return (scale & 2) != 0; }

// bfloat16 factors: the row factor and the clip-free column factor round up
// (toward +inf; x >= 0 finite), so every |Y| <= 1 and every code stays within
// +-q; a refitted column factor rounds to nearest, ties to even.  The
// quantiser then uses the rounded value, and the restore reads the same one.
__device__ __forceinline__ float bf16_up(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t t = u & 0xFFFF0000u;
  return __uint_as_float((u & 0xFFFFu) ? t + 0x10000u : t);
}

__device__ __forceinline__ float bf16_nearest(float x) {
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// Element i of a factor array that starts at byte `base` of the block.
template <bool B16>
__device__ __forceinline__ float load_sc(rsrc_t rs, uint32_t i, uint32_t base) {
  if constexpr (B16) {
    const uint32_t h = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, i * 2u, base, 0);
    return __uint_as_float(h << 16);
  } else {
    return load_f32(rs, i * 4u, base);
  }
}

// x must be a bfloat16 value when B16 (its low 16 bits are zero).
template <bool B16>
__device__ __forceinline__ void store_sc(rsrc_t rs, float x, uint32_t i, uint32_t base) {
  if constexpr (B16) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(__float_as_uint(x) >> 16), rs, i * 2u, base, 0);
  else store_f32(rs, x, i * 4u, base);
}

// Store one column half (this wave's 64 rows of column j) as 16-byte granules.
// soff0: byte offset of this wave's first granule row; voff = j*16.
template <int BITS>
__device__ __forceinline__ void store_column(rsrc_t rs, const uint32_t *ow, uint32_t voff, uint32_t soff0) {
#pragma unroll
  for (int g = 0; g < Kind<BITS>::NG; ++g) {
    uint4 t;
    t.x = ow[4 * g + 0]; t.y = ow[4 * g + 1]; t.z = ow[4 * g + 2]; t.w = ow[4 * g + 3];
    store_granule(rs, t, voff, soff0 + (uint32_t)g * (kDim * 16));
  }
}

__device__ __forceinline__ float4 lds4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// The lane index (0..63), computed afresh with v_mbcnt where it is used: the
// byte offsets of the final stores would otherwise stay live in registers
// from the item's loads to its stores, across the whole tile.
__device__ __forceinline__ uint32_t lane_now() {
  uint32_t r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The fp32 tile of one wave: lane l holds columns l and l + 64 of the wave's
// 64 rows; four consecutive rows of a column share one 4-register vector
// (v[c][g][e] = row 4g + e, column l + 64c).
struct Tile {
  v4f v[2][16];
  __device__ __forceinline__ float get(int c, int ii) const { return v[c][ii >> 2][ii & 3]; }
  __device__ __forceinline__ void set(int c, int ii, float x) { v[c][ii >> 2][ii & 3] = x; }
};

// Row reduction of |S| over the 128 columns of each of this wave's 64 rows.
// SUM: the fold-by-halves tree over the 128 columns (pairs j/j+64 are the
// lane's own two columns; then j/j+32 by
// permlane32_swap, j/j+16 by permlane16_swap, j/j+8 .. j/j+1 after one LDS
// transpose).  MAX: the same tree with max.  Returns the value of row
// 64w + lane.  red: this wave's [64][20] LDS scratch.
template <bool MAX>
__device__ __forceinline__ float row_reduce(const Tile &S, float (*red)[20], int lane) {
  // rows are taken four at a time so that only a handful of partials are
  // live next to the tile: rows 4s..4s+3 -> two permlane32 partials -> one
  // permlane16 partial holding row 4s + {0,2,1,3}[lane/16] for column
  // residue lane%16, written to LDS.
  const int G = lane >> 4, n = lane & 15;
  const int rsub = (G == 0) ? 0 : (G == 1) ? 2 : (G == 2) ? 1 : 3;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    float h1[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 4 * s + 2 * t, r1 = r0 + 1;
      const float p0 = MAX ? fmaxf(fabsf(S.get(0, r0)), fabsf(S.get(1, r0))) : fabsf(S.get(0, r0)) + fabsf(S.get(1, r0));
      const float p1 = MAX ? fmaxf(fabsf(S.get(0, r1)), fabsf(S.get(1, r1))) : fabsf(S.get(0, r1)) + fabsf(S.get(1, r1));
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
      const float x = __uint_as_float(sw[0]), y = __uint_as_float(sw[1]);
      h1[t] = MAX ? fmaxf(x, y) : x + y;
    }
    auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h1[0]), __float_as_uint(h1[1]), false, false);
    const float x = __uint_as_float(sw[0]), y = __uint_as_float(sw[1]);
    red[4 * s + rsub][n] = MAX ? fmaxf(x, y) : x + y;
    if (s & 1) QDR_FENCE();
  }
  __builtin_amdgcn_wave_barrier();
  // the first fold (i with i + 8) as the partials arrive, so at most eight
  // of them are live next to the tile
  float x[8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float4 t0 = lds4(&red[lane][4 * i]);
    const float4 t1 = lds4(&red[lane][4 * i + 8]);
    x[4 * i + 0] = MAX ? fmaxf(t0.x, t1.x) : t0.x + t1.x;
    x[4 * i + 1] = MAX ? fmaxf(t0.y, t1.y) : t0.y + t1.y;
    x[4 * i + 2] = MAX ? fmaxf(t0.z, t1.z) : t0.z + t1.z;
    x[4 * i + 3] = MAX ? fmaxf(t0.w, t1.w) : t0.w + t1.w;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int half = 4; half >= 1; half >>= 1) {
#pragma unroll
    for (int i = 0; i < half; ++i) x[i] = MAX ? fmaxf(x[i], x[i + half]) : x[i] + x[i + half];
  }
  return x[0];
}


// Restore this wave's 64 rows of both lane columns into S (gate included).
// CHAIN also runs acc_c = fma(x_i, S'_ic, acc_c) over those rows in order.
// OFF4 (INT4 only): the codes are converted as z/16 and gsh holds 16 g_i, so
// z' * (16 g) is the same real number as z * g and rounds identically.
template <int BITS, bool CHAIN, bool OFF4 = false>
__device__ __forceinline__ void restore_rows(Tile &S, float (&acc)[2],
                                             const uint32_t (&wd)[2][Kind<BITS>::NW],
                                             const float (&colc)[2], const float *gsh,
                                             const float *xsh, int row0) {
#pragma unroll
  for (int i4 = 0; i4 < 16; ++i4) {
    const float4 g4 = lds4(&gsh[row0 + 4 * i4]);
    float4 x4 = {0, 0, 0, 0};
    if (CHAIN) x4 = lds4(&xsh[row0 + 4 * i4]);
    const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
    const float xx[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = 4 * i4 + e;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float sp;
        if (Kind<BITS>::is_int) {
          const float zf = OFF4 ? int4_field_over16(wd[c], ii) : field_int_as_float<BITS>(wd[c], ii);
          sp = (zf * gg[e]) * colc[c];
        } else if (BITS == 16) {
          sp = gg[e] * __half2float(__ushort_as_half((unsigned short)(field_bits<16>(wd[c], ii) & 0xFFFFu)));
        } else {
          sp = gg[e] * __uint_as_float(field_bits<32>(wd[c], ii));
        }
        S.set(c, ii, sp);
        if (CHAIN) acc[c] = __builtin_fmaf(xx[e], sp, acc[c]);
      }
    }
    QDR_FENCE();
  }
}

// acc_c = fma(x_i, S_ic, acc_c) over this wave's 64 rows, in order.
__device__ __forceinline__ void chain_rows(const Tile &S, float (&acc)[2], const float *xsh, int row0) {
#pragma unroll
  for (int i4 = 0; i4 < 16; ++i4) {
    const float4 x4 = lds4(&xsh[row0 + 4 * i4]);
    const float xx[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[0] = __builtin_fmaf(xx[e], S.get(0, 4 * i4 + e), acc[0]);
      acc[1] = __builtin_fmaf(xx[e], S.get(1, 4 * i4 + e), acc[1]);
    }
    QDR_FENCE();
  }
}

// The rank-1 delta update of this wave's tile: S_ij = fma(b_i, delta_j, S_ij).
// bsh: the wave's b table (b_i of rows row0 ..).
__device__ __forceinline__ void delta_update(Tile &S, const float (&dl)[2], const float *bsh) {
#pragma unroll
  for (int i4 = 0; i4 < 16; ++i4) {
    const float4 b4 = lds4(bsh + 4 * i4);
    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S.set(0, 4 * i4 + e, __builtin_fmaf(bb[e], dl[0], S.get(0, 4 * i4 + e)));
      S.set(1, 4 * i4 + e, __builtin_fmaf(bb[e], dl[1], S.get(1, 4 * i4 + e)));
    }
    QDR_FENCE();
  }
}

// Calls f(i4, x4) on the 16 float4 groups of a 64-entry per-row LDS table in
// order, each group's read issued A groups before its use (in the row-unit
// kernel an LDS read issued in its own group's turn would stall its wave).
template <int A, class F>
__device__ __forceinline__ void row_groups(const float *t, F &&f) {
  float4 q[16];
#pragma unroll
  for (int g = 0; g < A; ++g) q[g] = lds4(t + 4 * g);
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    if (g + A < 16) q[g + A] = lds4(t + 4 * (g + A));
    f(g, q[g]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// chain_rows with its table reads issued A groups ahead (row_groups)
template <int A>
__device__ __forceinline__ void chain_rows_ahead(const Tile &S, float (&acc)[2], const float *xsh, int row0) {
  row_groups<A>(xsh + row0, [&](int i4, const float4 x4) {
    const float xx[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[0] = __builtin_fmaf(xx[e], S.get(0, 4 * i4 + e), acc[0]);
      acc[1] = __builtin_fmaf(xx[e], S.get(1, 4 * i4 + e), acc[1]);
    }
  });
}

// DPP row move of x (dpp_ctrl CTRL, all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the wave's 64 lanes, returned to every lane (used for the readout
// only, so the summation order is free): DPP butterflies inside each 16-lane
// row (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror), then the four row sums from lanes 0, 16, 32 and 48.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

// ---- q, k, v and o: fp32, or bfloat16 in the bfloat16-I/O step mode.
// A bfloat16 input widens to fp32 exactly; o narrows with round to nearest,
// ties to even (NaN stays NaN).
// The step's per-lane inputs: k and q of row `row`, v of columns l and l+64.
template <bool BF16>
__device__ __forceinline__ void load_qkv(const LaunchArgs &P, size_t bh, int row, int l, float &kr, float &qr,
                                         float (&vc)[2]) {
  const size_t base = bh * kDim;
  if constexpr (BF16) {
    const uint16_t *k16 = reinterpret_cast<const uint16_t *>(P.k) + base;
    const uint16_t *q16 = reinterpret_cast<const uint16_t *>(P.q) + base;
    const uint16_t *v16 = reinterpret_cast<const uint16_t *>(P.v) + base;
    const uint32_t a = k16[row], b = q16[row], c = v16[l], d = v16[l + 64];
    kr = __uint_as_float(a << 16);
    qr = __uint_as_float(b << 16);
    vc[0] = __uint_as_float(c << 16);
    vc[1] = __uint_as_float(d << 16);
  } else {
    kr = P.k[base + row];
    qr = P.q[base + row];
    vc[0] = P.v[base + l];
    vc[1] = P.v[base + 64 + l];
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool BF16>
__device__ __forceinline__ void out_o(const LaunchArgs &P, size_t idx, float x) {
  if constexpr (BF16) reinterpret_cast<uint16_t *>(P.o)[idx] = bf16_rne(x);
  else P.o[idx] = x;
}

// What a mode does: is_step -- the whole step with the store; has_readout --
// reads q, k, v, beta, gate and computes the readout; writes_o -- stores it;
// restores -- rebuilds S from codes; io16 -- q, k, v and o in bfloat16.
constexpr bool is_step(int m) { return m == MODE_STEP || m == MODE_STEP_BF16 || m == MODE_WRITEBACK; }
constexpr bool has_readout(int m) { return is_step(m) || m == MODE_READOUT; }
constexpr bool restores(int m) { return has_readout(m) || m == MODE_UNPACK; }
constexpr bool writes_o(int m) { return has_readout(m) && m != MODE_WRITEBACK; }
constexpr bool io16(int m) { return m == MODE_STEP_BF16; }

struct SharedCore {
  float g[kDim];     // restore factor a_i * r_i / q_i (or a_i for float kinds)
  float k[kDim];
  float b[kDim];     // beta * k_i
  float q[kDim];
  float ir[kDim];    // 1 / r_i
  float m[kDim];     // row magnitude (refit weights)
  float x[kDim];     // u hand-off, then o partial of wave 1
  float d[kDim];     // delta, then refit numerator hand-off
  float y[kDim];     // refit denominator hand-off
  float cmax[2][kDim];
  float qm[kDim];    // row units: largest code of the row's grid (0 for float rows)
  float iq[kDim];    // row units: 1/qm (0 for float rows)
  float qb[2];       // each wave's part of sum_i q_i b_i
};

struct Shared : SharedCore {
  float red[2][64][20];   // row-reduction transpose scratch, one block per wave
};

}  // namespace

// --------------------------------------------------------------------------
// Whole-head kernel: every row of the head has kind BITS.
// MODE_STEP: restore, gate, delta update, readout, requantise, store.
// MODE_READOUT: restore, gate, u and delta, readout only (no store).
// MODE_STEP_BF16: MODE_STEP with bfloat16 q, k, v and o.
// MODE_WRITEBACK: MODE_STEP without the o store (the second half of the
// two-stream step).
// MODE_PACK: requantise S_in.  MODE_UNPACK: restore into S_out.
// MODE_RESET: requantise S = 0.
// --------------------------------------------------------------------------
// Waves per SIMD the register allocation targets: three for the dual-axis
// integer kernels (their 128-register tile plus working set fits in 168
// VGPRs), two where it does not (float kinds, the refit variant, the
// row-absmax baseline).
template <int BITS, int MODE, int SCALE, int FIT>
struct Occupancy {
  static constexpr int waves = (BITS <= 8 && FIT == 0 && dual(SCALE)) ? 3 : 2;
};
// The row-unit kernel: three waves per SIMD except the pack of dense states
// (up to 9 registers over the three-wave budget).
template <int MODE>
struct RowsOccupancy {
  static constexpr int waves = (MODE == MODE_PACK) ? 2 : 3;
};

// The work of one (request b, head h) of kind BITS; sh is the workgroup's
// LDS block; w the wave of this lane (0 or 1, uniform).
template <int BITS, int MODE, int GATE, int SCALE, int FIT>
__device__ __forceinline__ void head_body(const LaunchArgs &P, Shared &sh, const int b, const int h,
                                          const uint64_t head_off, const uint32_t code_bytes, const int w) {
  using K = Kind<BITS>;
  constexpr bool INT = K::is_int;
  constexpr float QMAX = (float)K::qmax_i;
  // INT4 codes convert as z/16 (one SDWA instruction each); the 16 moves into
  // the row factor.  Dual-axis row factors are at most sqrt(FLT_MAX / 2^-40),
  // so 16 g_i stays finite; the row-absmax baseline keeps the plain path.
  constexpr bool OFF4 = (BITS == 4) && dual(SCALE);
  constexpr bool SC16 = sc16(SCALE);
  constexpr uint32_t SCB = SC16 ? 2u : 4u;   // bytes per stored factor
  constexpr float GSCALE = OFF4 ? 16.0f : 1.0f;

  const int l = threadIdx.x & 63;
  const int row = 64 * w + l;
  const size_t bh = (size_t)b * P.H + h;
  const int slot = P.slots[b];

  if (slot < 0 || slot >= P.num_slots) {
    if (slot != -1 && row == 0) atomicOr(P.err, 1u);
    if (writes_o(MODE) && w == 0 && P.o != nullptr) {
      out_o<io16(MODE)>(P, bh * kDim + l, 0.0f);     // wave 0 and 1 cover columns 0..127
      out_o<io16(MODE)>(P, bh * kDim + 64 + l, 0.0f);
    }
    if (MODE == MODE_UNPACK) {
      float *dst = P.S_out + bh * kDim * kDim;
      for (int i = 0; i < 64; ++i) { dst[(64 * w + i) * kDim + l] = 0.0f; dst[(64 * w + i) * kDim + 64 + l] = 0.0f; }
    }
    return;
  }
  uint8_t *blk = P.pool + (size_t)slot * P.slot_stride + head_off;
  const uint32_t blk_bytes = code_bytes + (INT ? (dual(SCALE) ? 2u : 1u) * kDim * SCB : 0u);
  const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(blk, 0, (int)blk_bytes, kRsrcWord3);
  const uint32_t half_off = (uint32_t)w * K::NG * (kDim * 16);   // this wave's first granule row
  const uint32_t r_off = code_bytes;                              // r[128]
  const uint32_t c_off = code_bytes + kDim * SCB;                 // c[128]

  Tile S;
  float colc[2] = {1.0f, 1.0f};

  // ---------------- load codes (both columns of this lane, this wave's rows)
  uint32_t wd[2][K::NW];
  if (restores(MODE)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int g = 0; g < K::NG; ++g) {
        const uint4 t = load_granule(rs, (uint32_t)(l + 64 * c) * 16u, half_off + (uint32_t)g * (kDim * 16));
        wd[c][4 * g + 0] = t.x; wd[c][4 * g + 1] = t.y; wd[c][4 * g + 2] = t.z; wd[c][4 * g + 3] = t.w;
      }
    }
  }
  // the rest of the item's loads, all issued before the first wait: the
  // row's readout weight (a load at its use, after the restore, would add a
  // memory round trip), the gate, the factors, q/k/v and beta
  const float omega_row = (INT && dual(SCALE)) ? (P.omega + (size_t)h * kDim)[row] : 1.0f;
  float a_row = 1.0f;
  if (has_readout(MODE)) a_row = (GATE == 0) ? P.gate[bh] : (P.gate + bh * kDim)[row];
  float r_raw = 1.0f;
  if (restores(MODE) && INT) {
    r_raw = load_sc<SC16>(rs, (uint32_t)l, r_off + (uint32_t)w * 64u * SCB);
    if (dual(SCALE)) {
      colc[0] = load_sc<SC16>(rs, (uint32_t)l, c_off);
      colc[1] = load_sc<SC16>(rs, (uint32_t)l + 64u, c_off);
    }
  }
  float vcol[2] = {0.0f, 0.0f};
  float kr = 0.0f, qr = 0.0f, beta_b = 0.0f;
  if (has_readout(MODE)) {
    load_qkv<io16(MODE)>(P, bh, row, l, kr, qr, vcol);
    beta_b = P.beta[bh];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---------------- per-row scalars of this lane's row, broadcast via LDS
  if (restores(MODE)) sh.g[row] = INT ? (a_row * rn_div(r_raw, QMAX)) * GSCALE : a_row;
  const float b_row = beta_b * kr;
  if (has_readout(MODE)) {
    sh.k[row] = kr;
    sh.b[row] = b_row;
    sh.q[row] = qr;
    if (w == 1) {
      // v waits in the delta slots (wave 1 forms delta there)
      sh.d[l] = vcol[0];
      sh.d[l + 64] = vcol[1];
    }
  }
  // omega waits in the row's 1/r slot (overwritten by 1/r), so neither it
  // nor v holds a register across the restore and the update
  if (INT && dual(SCALE)) sh.ir[row] = omega_row;
  if (has_readout(MODE)) {
    // each wave's part of q . beta k (order free: readout only), now, so
    // that q and beta k hold no registers across the restore
    const float qb_part = wave_sum(qr * b_row);
    if (l == 0) sh.qb[w] = qb_part;
  }
  __builtin_amdgcn_wave_barrier();

  // ---------------- restore (and gate).  In a step the two waves balance the
  // sequential key projection u = S'^T k (rows 0..63 by wave 0, then rows
  // 64..127 by wave 1) against the readout part S'^T q of their own rows:
  // wave 0 runs its half of u inside the restore and its q part after the
  // hand-off, wave 1 the other way round.
  float acc1[2] = {0.0f, 0.0f};
  if (has_readout(MODE))
    restore_rows<BITS, true, OFF4>(S, acc1, wd, colc, sh.g, (w == 0) ? sh.k : sh.q, 64 * w);
  else if (MODE == MODE_UNPACK)
    restore_rows<BITS, false, OFF4>(S, acc1, wd, colc, sh.g, sh.g, 64 * w);

  if (MODE == MODE_UNPACK) {
    float *dst = P.S_out + bh * kDim * kDim;
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) {
      dst[(64 * w + ii) * kDim + l] = S.get(0, ii);
      dst[(64 * w + ii) * kDim + 64 + l] = S.get(1, ii);
    }
    return;
  }

  if (MODE == MODE_PACK) {
    const float *src = P.S_in + bh * kDim * kDim;
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) {
      S.set(0, ii, src[(64 * w + ii) * kDim + l]);
      S.set(1, ii, src[(64 * w + ii) * kDim + 64 + l]);
    }
  }
  if (MODE == MODE_RESET) {
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) { S.set(0, ii, 0.0f); S.set(1, ii, 0.0f); }
  }

  // ---------------- delta update, and the readout as soon as delta is known
  // (tolerance-checked, any summation order):
  //   o = S_t^T q = S'^T q + (q . b) delta,
  // wave 1's part of S'^T q handed to wave 0 with delta
  if (has_readout(MODE)) {
    if (w == 0) { sh.x[l] = acc1[0]; sh.x[l + 64] = acc1[1]; }
    __syncthreads();
    float acc2[2] = {0.0f, 0.0f};
    if (w == 1) { acc2[0] = sh.x[l]; acc2[1] = sh.x[l + 64]; }
    // (the write-back stores no readout: wave 0 skips its S'^T q part)
    if (!(MODE == MODE_WRITEBACK && w == 0)) chain_rows(S, acc2, (w == 0) ? sh.q : sh.k, 64 * w);
    if (w == 1) {
      sh.d[l] = sh.d[l] - acc2[0];
      sh.d[l + 64] = sh.d[l + 64] - acc2[1];
      sh.x[l] = acc1[0];          // wave 1's readout part; wave 0's u part has been read
      sh.x[l + 64] = acc1[1];
    }
    __syncthreads();
    float dl[2] = {sh.d[l], sh.d[l + 64]};
    if (writes_o(MODE) && w == 0 && P.o != nullptr) {
      const float qb_all = sh.qb[0] + sh.qb[1];
      out_o<io16(MODE)>(P, bh * kDim + l, (acc2[0] + sh.x[l]) + qb_all * dl[0]);
      out_o<io16(MODE)>(P, bh * kDim + 64 + l, (acc2[1] + sh.x[l + 64]) + qb_all * dl[1]);
    }
    // readout-first launch: the state is neither updated nor stored (the
    // write-back launch does it)
    if constexpr (MODE == MODE_READOUT) return;
    delta_update(S, dl, &sh.b[64 * w]);
  }

  // ---------------- requantise
  if (INT) {
    // row factor
    float r_row, m_row = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    if (dual(SCALE)) {
      m_row = row_reduce<false>(S, sh.red[w], l) * 0.0078125f;
      const float nu = rn_div(m_row, sh.ir[row]);   // omega of the row
      r_row = (nu == 0.0f) ? 1.0f : rn_sqrt(nu);
    } else {
      const float mx = row_reduce<true>(S, sh.red[w], l);
      r_row = (mx < FLT_MIN) ? 1.0f : mx;
    }
    if constexpr (SC16) r_row = bf16_up(r_row);
    sh.ir[row] = rn_div(1.0f, r_row);
    if (FIT) sh.m[row] = m_row;
    store_sc<SC16>(rs, r_row, lane_now(), r_off + (uint32_t)w * 64u * SCB);
    __builtin_amdgcn_wave_barrier();

    // Y = S / r (in place) and the column maximum
    // (two partial maxima per column, rows 4s+{0,1} and 4s+{2,3}: the
    // maximum is exact in any order, and four independent chains keep the
    // dependent v_max3 latency off the critical path)
    float cm[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
#pragma unroll
    for (int i4 = 0; i4 < 16; ++i4) {
      const float4 r4 = lds4(&sh.ir[64 * w + 4 * i4]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float y = S.get(c, 4 * i4 + e) * rr[e];
          S.set(c, 4 * i4 + e, y);
          cm[c][e >> 1] = fmaxf(cm[c][e >> 1], fabsf(y));
        }
      }
      QDR_FENCE();
    }
    float c0[2] = {1.0f, 1.0f};
    if (dual(SCALE)) {
      sh.cmax[w][l] = fmaxf(cm[0][0], cm[0][1]);
      sh.cmax[w][l + 64] = fmaxf(cm[1][0], cm[1][1]);
    }
    __syncthreads();
    if (dual(SCALE)) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float mx = fmaxf(sh.cmax[0][l + 64 * c], sh.cmax[1][l + 64 * c]);
        c0[c] = (mx < FLT_MIN) ? 1.0f : mx;
        if constexpr (SC16) c0[c] = bf16_up(c0[c]);
      }
    }
    float wq[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) wq[c] = dual(SCALE) ? rn_div(1.0f, c0[c]) * QMAX : QMAX;

    // codes: both columns at once (two independent packing chains), then store
    float nacc[2] = {0.0f, 0.0f}, dacc[2] = {0.0f, 0.0f};
    constexpr float INVQ = INT ? 1.0f / (QMAX > 0.0f ? QMAX : 1.0f) : 0.0f;
    {
      uint32_t ow[2][K::NW];
      uint32_t pacc[2] = {0u, 0u};
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4) {
        float mm[4] = {0, 0, 0, 0};
        if (FIT) {
          const float4 m4 = lds4(&sh.m[64 * w + 4 * i4]);
          mm[0] = m4.x; mm[1] = m4.y; mm[2] = m4.z; mm[3] = m4.w;
        }
        uint32_t tb[2][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = 4 * i4 + e;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float t = __builtin_fmaf(S.get(c, ii), wq[c], kMagic);
            tb[c][e] = __float_as_uint(t);
            if (BITS != 8) put_field<BITS>(ow[c], pacc[c], __float_as_uint(t), ii);
            if (FIT) {
              const float zeta = (t - kMagic) * INVQ;
              const float pz = mm[e] * zeta;
              nacc[c] = __builtin_fmaf(pz, S.get(c, ii), nacc[c]);
              dacc[c] = __builtin_fmaf(pz, zeta, dacc[c]);
            }
          }
        }
        if (BITS == 8) {
          // the low byte of each t is its two's complement code: gather the
          // four bytes of rows 4*i4 .. 4*i4+3 with three byte permutes
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t lo = __builtin_amdgcn_perm(tb[c][1], tb[c][0], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(tb[c][3], tb[c][2], 0x0c0c0400u);
            ow[c][i4] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
        }
        QDR_FENCE();
      }
      const uint32_t ln = lane_now();
#pragma unroll
      for (int c = 0; c < 2; ++c) store_column<BITS>(rs, ow[c], (ln + 64u * c) * 16u, half_off);
    }
    // column factor
    if (dual(SCALE)) {
      if (!FIT) {
        if (w == 0) {
          const uint32_t ln = lane_now();
          store_sc<SC16>(rs, c0[0], ln, c_off);
          store_sc<SC16>(rs, c0[1], ln + 64u, c_off);
        }
      } else {
        if (w == 0) {
          sh.d[l] = nacc[0]; sh.d[l + 64] = nacc[1];
          sh.y[l] = dacc[0]; sh.y[l + 64] = dacc[1];
        }
        __syncthreads();
        if (w == 1) {
          // each wave summed its own rows; the halves are added in row order
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float nn = sh.d[l + 64 * c] + nacc[c], dd = sh.y[l + 64 * c] + dacc[c];
            float cf = (dd > 0.0f) ? rn_div(nn, dd) : c0[c];
            if constexpr (SC16) cf = bf16_nearest(cf);
            store_sc<SC16>(rs, cf, lane_now() + 64u * c, c_off);
          }
        }
      }
    }
  } else {
    // FP16 / FP32 rows: store the updated values themselves
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t ow[K::NW];
      uint32_t pacc = 0;
#pragma unroll
      for (int ii = 0; ii < 64; ++ii) {
        uint32_t f;
        if (BITS == 16) f = (uint32_t)__half_as_ushort(__float2half_rn(pin_f32(S.get(c, ii))));
        else f = __float_as_uint(S.get(c, ii));
        put_field<BITS>(ow, pacc, f, ii);
      }
      store_column<BITS>(rs, ow, (lane_now() + 64u * c) * 16u, half_off);
    }
  }
}

// One storage kind per launch: block = (request, entry of head_list).
template <int BITS, int MODE, int GATE, int SCALE, int FIT>
__global__ void __launch_bounds__(128)
__attribute__((amdgpu_waves_per_eu(Occupancy<BITS, MODE, SCALE, FIT>::waves)))
k_head(const LaunchArgs P) {
  __shared__ Shared sh;
  const int item = blockIdx.x;
  const int b = item / P.n_list;
  const ListEntry &e = P.head_list[item - b * P.n_list];
  // v_readfirstlane is convergent, so these reads stay ahead of the padding /
  // bad-slot branch (which stores): the entry is then read by one scalar load
  // before anything is written, not by a vector load after the branch.
  const uint64_t off = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(e.info.off >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)e.info.off);
  const uint32_t code_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)e.info.code_bytes);
  head_body<BITS, MODE, GATE, SCALE, FIT>(P, sh, b, e.h, off, code_bytes,
                                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
}

// Every integer kind in one launch.  head_list interleaves the integer heads
// of the different widths in proportion to their counts, so each compute
// unit runs a mix of them at any time: the narrow widths are bound by vector
// ALU work and the wide ones by HBM traffic, and mixed they overlap instead
// of running as separate back-to-back launches.  The kind is read per block
// (uniform across the workgroup), so the branch below is scalar.
template <int MODE, int GATE, int SCALE, int FIT>
__global__ void __launch_bounds__(128)
__attribute__((amdgpu_waves_per_eu(Occupancy<8, MODE, SCALE, FIT>::waves)))
k_head_int(const LaunchArgs P) {
  __shared__ Shared sh;
  const int item = blockIdx.x;
  const int b = item / P.n_list;
  const ListEntry &e = P.head_list[item - b * P.n_list];
  // the entry's words through v_readfirstlane (scalar loads ahead of the
  // padding branch, see k_head)
  const uint32_t *ew = reinterpret_cast<const uint32_t *>(&e);
  uint32_t wv[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) wv[t] = (uint32_t)__builtin_amdgcn_readfirstlane((int)ew[t]);
  const uint64_t off = ((uint64_t)wv[1] << 32) | wv[0];
  const uint32_t code_bytes = wv[2];
  const int kind = (int)((wv[3] >> 16) & 0xFFu);
  const int h = (int)wv[4];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kind == 6) head_body<6, MODE, GATE, SCALE, FIT>(P, sh, b, h, off, code_bytes, w);
  else if (kind == 8) head_body<8, MODE, GATE, SCALE, FIT>(P, sh, b, h, off, code_bytes, w);
  else if (kind == 4) head_body<4, MODE, GATE, SCALE, FIT>(P, sh, b, h, off, code_bytes, w);
  else head_body<2, MODE, GATE, SCALE, FIT>(P, sh, b, h, off, code_bytes, w);
}

// Row i's program word, broadcast from lane i of the per-lane table register
// (i is a compile-time lane index: one v_readlane into a scalar register).
__device__ __forceinline__ uint32_t row_lane(uint32_t xs_v, int i) {
  return (uint32_t)__builtin_amdgcn_readlane((int)xs_v, i);
}
// fields of a program word: LDS byte offset of the field's first word, the
// width of a 2..16-bit field, the repack's completing shift (low 5 bits)
__device__ __forceinline__ uint32_t rp_base(uint32_t e) { return e & (kRowCompletes - 512u); }
__device__ __forceinline__ uint32_t rp_width(uint32_t e) { return (e >> 4) & 30u; }
__device__ __forceinline__ uint32_t rp_pack_shift(uint32_t e) { return 0u - e; }

// Append one field of `kind` bits (1..16) at stream bit `off` of a
// column-half stream to the two column windows of a lane.  A window holds
// the last 32 stream bits written, newest at the top: the funnel shift by the
// width brings the field's low `kind` bits in from the top.  When the field
// reaches or crosses the end of its word, that word -- the window shifted by
// the bits that were missing -- is written to LDS (out: [word][column] of the
// half).  Whatever is left below the field after a crossing is shifted out
// before the next word completes.
__device__ __forceinline__ void append_field(uint32_t *out, int l, uint32_t (&win)[2], uint32_t f0,
                                             uint32_t f1, uint32_t off, uint32_t kind) {
  const uint32_t sft = off & 31u;
  if (sft + kind >= 32u) {
    uint32_t *o = out + (off >> 5) * kDim + l;
    o[0] = __builtin_amdgcn_alignbit(f0, win[0], 32u - sft);
    o[64] = __builtin_amdgcn_alignbit(f1, win[1], 32u - sft);
  }
  win[0] = __builtin_amdgcn_alignbit(f0, win[0], kind);
  win[1] = __builtin_amdgcn_alignbit(f1, win[1], kind);
}

// --------------------------------------------------------------------------
// Row-unit kernel: each key row has its own kind (per-key-channel allocation
// of the KDA variant, review "STEPQuant: When and Where Errors Matter in
// Delta-Rule Recurrent State Quantization", Method).  Same thread mapping and
// arithmetic as k_head.  Row widths are data, so:
//   * each wave stages its half of the column streams in LDS; lane l holds
//     the program word of row l of the half (word offset | width code | bit
//     offset) in a vector register, loaded once with the codes, and each
//     row's word is broadcast with v_readlane into a scalar register whose
//     fields serve as instruction operands.  (Scalar loads of the
//     tables inside the loops would share the LDS wait counter, so every LDS
//     wait there would also wait for a table load from L2; only the
//     repack's append pass, which reads no LDS, takes the words by scalar
//     loads.);
//   * R1 restores every row as an integer row (a funnel shift of two words,
//     then one sign-extending extract of the row's width), straight-line;
//     rows stored as FP16/FP32 pivots are redone in uniform branches (R2)
//     only when the half holds any;
//   * repacking: every value becomes its code bits in place (P1), pivot rows
//     take their stored bits from an LDS stash, then each row's field is
//     appended to per-column register windows (P2); the word a field ends in
//     is written to LDS at once (a later field of the same word overwrites
//     it), and the half goes out with 16-byte stores.  Halves holding FP32
//     rows append in uniform branches instead.
// LDS: each wave's region holds the staged words of its half (one spare row
// so the second word of a funnel shift stays in range); after the restore it
// serves as the row reduction's scratch, the pivot stash and the output
// image of the half.
// --------------------------------------------------------------------------
template <int MODE, int GATE, int SCALE, int FIT>
__global__ void __launch_bounds__(128)
// three waves per SIMD (168 VGPRs): the third wave covers the LDS and memory
// latency of the per-row extraction (config 5: 8.63 -> 6.86 ms with the
// clip-free fit, 10.64 -> 8.06 ms with the refit, against two waves)
__attribute__((amdgpu_waves_per_eu(RowsOccupancy<MODE>::waves)))
k_rows(const LaunchArgs P) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_codes[];   // 16-byte aligned: staged with ds_write_b128
  __shared__ SharedCore sh;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int row = 64 * w + l;
  const int item = blockIdx.x;
  const int b = item / P.n_list;
  const ListEntry &ent = P.head_list[item - b * P.n_list];
  // read the whole entry ahead of the bad-slot branch (see k_head)
  uint32_t ev[5];
  {
    const uint32_t *ew = reinterpret_cast<const uint32_t *>(&ent);
#pragma unroll
    for (int t = 0; t < 5; ++t) ev[t] = (uint32_t)__builtin_amdgcn_readfirstlane((int)ew[t]);
  }
  const uint64_t blk_off = ((uint64_t)ev[1] << 32) | ev[0];
  const uint32_t code_bytes = ev[2];
  const int words0 = (int)(ev[3] & 0xFFu), words1 = (int)((ev[3] >> 8) & 0xFFu);
  const int has_int = (int)(ev[3] >> 24);
  const int h = (int)ev[4];
  const size_t bh = (size_t)b * P.H + h;
  const int slot = P.slots[b];

  if (slot < 0 || slot >= P.num_slots) {
    if (slot != -1 && tid == 0) atomicOr(P.err, 1u);
    if (writes_o(MODE) && w == 0 && P.o != nullptr) {
      out_o<io16(MODE)>(P, bh * kDim + l, 0.0f);
      out_o<io16(MODE)>(P, bh * kDim + 64 + l, 0.0f);
    }
    if (MODE == MODE_UNPACK) {
      float *dst = P.S_out + bh * kDim * kDim;
      for (int i = 0; i < 64; ++i) { dst[(64 * w + i) * kDim + l] = 0.0f; dst[(64 * w + i) * kDim + 64 + l] = 0.0f; }
    }
    return;
  }
  uint8_t *blk = P.pool + (size_t)slot * P.slot_stride + blk_off;
  constexpr bool SC16 = sc16(SCALE);
  constexpr uint32_t SCB = SC16 ? 2u : 4u;   // bytes per stored factor
  const uint32_t blk_bytes = code_bytes + (has_int ? (dual(SCALE) ? 2u : 1u) * kDim * SCB : 0u);
  const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(blk, 0, (int)blk_bytes, kRsrcWord3);
  const int nwords = (w == 0) ? words0 : words1;                    // words per column, this half
  const uint32_t half_off = (w == 0) ? 0u : (uint32_t)words0 * (kDim * 4);
  const uint32_t half_bytes = (uint32_t)nwords * (kDim * 4);
  const uint32_t r_off = code_bytes, c_off = code_bytes + kDim * SCB;
  uint32_t *codes = lds_codes + (size_t)w * P.region_rows * kDim;   // [word][column]
  uint8_t *codes8 = reinterpret_cast<uint8_t *>(codes);
  const uint32_t lane_byte = (uint32_t)l * 4u;                       // column l of word 0
  // rows (restore) and table groups (other passes) whose LDS reads are in
  // flight ahead of their use, within the three-wave register budget (the
  // refit's extra sums leave room for one)
  constexpr int kAhead = FIT ? 1 : 2;
  // ---------------- every load of the item goes out here, ahead of the
  // first wait: the row programs and row data, then the code chunks (the HBM
  // stream).  (Loads issued after a wait, or behind a branch on loaded data,
  // would each add a memory round trip.)
  // this half's row programs: lane l loads row 64w + l's entries
  const RowProg *prog = P.row_prog + (size_t)h * kDim + 64 * w;
  const uint32_t xs_v = prog[l].xs;
  const int my_kind = (int)prog[l].z;
  const float omega_row = dual(SCALE) ? (P.omega + (size_t)h * kDim)[row] : 1.0f;
  float a_row = 1.0f;
  if (has_readout(MODE)) a_row = (GATE == 0) ? P.gate[bh] : (P.gate + bh * kDim)[row];
  // factors: r of every row (pivot rows' entries are read and ignored), c of
  // the lane's two columns; a head without integer rows stores none
  float r_raw = 1.0f;
  float colc[2] = {1.0f, 1.0f};
  if (restores(MODE) && has_int) {
    r_raw = load_sc<SC16>(rs, (uint32_t)l, r_off + (uint32_t)w * 64u * SCB);
    if (dual(SCALE)) {
      colc[0] = load_sc<SC16>(rs, (uint32_t)l, c_off);
      colc[1] = load_sc<SC16>(rs, (uint32_t)l + 64u, c_off);
    }
  }
  float vcol[2] = {0.0f, 0.0f};
  float kr = 0.0f, qr = 0.0f, beta_b = 0.0f;
  if (has_readout(MODE)) {
    load_qkv<io16(MODE)>(P, bh, row, l, kr, qr, vcol);
    beta_b = P.beta[bh];
  }
  // code chunks of this half (1 KiB per wave instruction), the first eight
  // unconditionally: lanes past the end of the half, and chunks past the
  // last, take an offset beyond the buffer's range, which reads zeros
  // without a memory access (so a last chunk of one word row also zeroes the
  // spare row)
  const uint32_t nchunks = (half_bytes + 1023u) >> 10;
  uint4 chunk[8];
  if (restores(MODE)) {
#pragma unroll
    for (uint32_t u = 0; u < 8u; ++u) {
      const uint32_t boff = u * 1024u + (uint32_t)l * 16u;
      chunk[u] = load_granule(rs, boff < half_bytes ? boff : kBeyondBuffer, half_off);
    }
  }
  // keep the scheduler from hoisting a use of the loaded data (and its wait)
  // above the loads
  __builtin_amdgcn_sched_barrier(0);

  // ---------------- per-row scalars of this lane's row
  const bool my_int = my_kind <= 8;
  const float my_q = my_int ? (float)((1 << (my_kind - 1)) - 1) : 0.0f;
  // rows of this half stored as FP16/FP32 pivots, and as FP32 (bit ii = row 64w+ii)
  const uint64_t pivots = __ballot(!my_int);
  const uint64_t fp32_rows = __ballot(my_kind == 32);
  sh.qm[row] = my_q;
  if (FIT) sh.iq[row] = my_int ? rn_div(1.0f, my_q) : 0.0f;
  if (restores(MODE)) sh.g[row] = my_int ? a_row * rn_div(r_raw, my_q) : a_row;
  const float b_row = beta_b * kr;
  if (has_readout(MODE)) {
    sh.k[row] = kr;
    sh.b[row] = b_row;
    sh.q[row] = qr;
    // v waits in the delta slots (wave 1 forms delta there) and omega in the
    // 1/r slot (overwritten by 1/r), so neither holds a register meanwhile
    if (w == 1) { sh.d[l] = vcol[0]; sh.d[l + 64] = vcol[1]; }
  }
  if (dual(SCALE)) sh.ir[row] = omega_row;

  // ---------------- stage the code words in LDS: the first eight chunks
  // from registers, any further ones (halves over 8 KiB) in batches of eight
  // loads ahead of their writes
  Tile S;
  if (restores(MODE)) {
#pragma unroll
    for (uint32_t u = 0; u < 8u; ++u)
      if (u < nchunks) *reinterpret_cast<uint4 *>(codes8 + u * 1024u + (uint32_t)l * 16u) = chunk[u];
    for (uint32_t g0 = 8u; g0 < nchunks; g0 += 8u) {
      uint4 t[8];
#pragma unroll
      for (uint32_t u = 0; u < 8u; ++u) {
        const uint32_t boff = (g0 + u) * 1024u + (uint32_t)l * 16u;
        t[u] = load_granule(rs, boff < half_bytes ? boff : kBeyondBuffer, half_off);
      }
#pragma unroll
      for (uint32_t u = 0; u < 8u; ++u)
        if (g0 + u < nchunks) *reinterpret_cast<uint4 *>(codes8 + (g0 + u) * 1024u + (uint32_t)l * 16u) = t[u];
    }
    codes[nwords * kDim + l] = 0u;
    codes[nwords * kDim + 64 + l] = 0u;
  }
  __builtin_amdgcn_wave_barrier();

  // ---------------- restore (and gate).  R1: every row as an integer row,
  // R2: pivot rows redone (only when the half has any), R3: the first chain
  // (u over rows 0..63 in wave 0, the S'^T q part of rows 64..127 in wave 1)
  // in row order.
  float acc1[2] = {0.0f, 0.0f};
  if (restores(MODE)) {
    // the staged words of row ii + kAhead are read while row ii is restored,
    // so a row's LDS reads have kAhead rows of work to land in (read in the
    // row's turn, each row would wait out its own LDS latency)
    uint32_t pe_q[64], wq[64][4];
    float4 gq[16];
    auto fetch = [&](int ii) {
      pe_q[ii] = row_lane(xs_v, ii);
      const uint32_t *wp = reinterpret_cast<const uint32_t *>(codes8 + (rp_base(pe_q[ii]) | lane_byte));
      wq[ii][0] = wp[0]; wq[ii][1] = wp[64]; wq[ii][2] = wp[kDim]; wq[ii][3] = wp[kDim + 64];
      if ((ii & 3) == 0) gq[ii >> 2] = lds4(&sh.g[64 * w + ii]);
    };
#pragma unroll
    for (int ii = 0; ii < kAhead; ++ii) fetch(ii);
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) {
      const float4 g4 = gq[ii >> 2];
      const float gi = ((ii & 3) == 0) ? g4.x : ((ii & 3) == 1) ? g4.y : ((ii & 3) == 2) ? g4.z : g4.w;
      const uint32_t pe = pe_q[ii];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // FP32 rows have width 0 here (and give 0); R2 redoes them
        const int32_t z = sext_low(__builtin_amdgcn_alignbit(wq[ii][2 + c], wq[ii][c], pe), rp_width(pe));
        S.set(c, ii, ((float)z * gi) * colc[c]);
      }
      if (ii + kAhead < 64) fetch(ii + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (pivots != 0) {
      // pivot rows are rare: test eight rows at a time, then the rows of a
      // group that holds any
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) {
        if (((pivots >> (8 * g8)) & 0xFFu) == 0u) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ii = 8 * g8 + e;
          if (!((pivots >> ii) & 1u)) continue;
          const uint32_t pe = row_lane(xs_v, ii);
          const bool f32row = (fp32_rows >> ii) & 1u;
          const uint32_t *wp = reinterpret_cast<const uint32_t *>(codes8 + (rp_base(pe) | lane_byte));
          const float gi = sh.g[64 * w + ii];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t f = __builtin_amdgcn_alignbit(wp[kDim + 64 * c], wp[64 * c], pe);
            S.set(c, ii, gi * (f32row ? __uint_as_float(f)
                                      : __half2float(__ushort_as_half((unsigned short)(f & 0xFFFFu)))));
          }
        }
      }
    }
    // (the write-back stores no readout: wave 1 skips its S'^T q part)
    if (has_readout(MODE) && !(MODE == MODE_WRITEBACK && w == 1))
      chain_rows_ahead<kAhead>(S, acc1, (w == 0) ? sh.k : sh.q, 64 * w);
  }

  if (MODE == MODE_UNPACK) {
    float *dst = P.S_out + bh * kDim * kDim;
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) {
      dst[(64 * w + ii) * kDim + l] = S.get(0, ii);
      dst[(64 * w + ii) * kDim + 64 + l] = S.get(1, ii);
    }
    return;
  }
  if (MODE == MODE_PACK) {
    const float *src = P.S_in + bh * kDim * kDim;
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) {
      S.set(0, ii, src[(64 * w + ii) * kDim + l]);
      S.set(1, ii, src[(64 * w + ii) * kDim + 64 + l]);
    }
  }
  if (MODE == MODE_RESET) {
#pragma unroll
    for (int ii = 0; ii < 64; ++ii) { S.set(0, ii, 0.0f); S.set(1, ii, 0.0f); }
  }

  // ---------------- delta update (same hand-off as k_head)
  float oq[2] = {0.0f, 0.0f};
  float dl[2] = {0.0f, 0.0f};
  if (has_readout(MODE)) {
    if (w == 0) { sh.x[l] = acc1[0]; sh.x[l + 64] = acc1[1]; }
    const float qb_part = wave_sum(qr * b_row);
    if (l == 0) sh.qb[w] = qb_part;
    __syncthreads();
    float acc2[2] = {0.0f, 0.0f};
    if (w == 1) { acc2[0] = sh.x[l]; acc2[1] = sh.x[l + 64]; }
    if (!(MODE == MODE_WRITEBACK && w == 0)) chain_rows_ahead<kAhead>(S, acc2, (w == 0) ? sh.q : sh.k, 64 * w);
    if (w == 1) {
      sh.d[l] = sh.d[l] - acc2[0];
      sh.d[l + 64] = sh.d[l + 64] - acc2[1];
      // wave 1's readout part goes where wave 0's u part was (already read)
      sh.x[l] = acc1[0];
      sh.x[l + 64] = acc1[1];
    } else {
      oq[0] = acc2[0]; oq[1] = acc2[1];
    }
    __syncthreads();
    dl[0] = sh.d[l];
    dl[1] = sh.d[l + 64];
    // the readout, o = S'^T q + (q . b) delta (tolerance-checked, any
    // summation order), written as soon as delta is known
    if (writes_o(MODE) && w == 0 && P.o != nullptr) {
      const float qb_all = sh.qb[0] + sh.qb[1];
      out_o<io16(MODE)>(P, bh * kDim + l, (oq[0] + sh.x[l]) + qb_all * dl[0]);
      out_o<io16(MODE)>(P, bh * kDim + 64 + l, (oq[1] + sh.x[l + 64]) + qb_all * dl[1]);
    }
    // readout-first launch: the state is neither updated nor stored (the
    // write-back launch does it)
    if constexpr (MODE == MODE_READOUT) return;
    row_groups<kAhead>(&sh.b[64 * w], [&](int i4, const float4 b4) {
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 4 * i4 + e;
        S.set(0, ii, __builtin_fmaf(bb[e], dl[0], S.get(0, ii)));
        S.set(1, ii, __builtin_fmaf(bb[e], dl[1], S.get(1, ii)));
      }
    });
  }


  // ---------------- row factors (integer rows only use them)
  // (the row reduction's scratch aliases the staged words: both waves have
  // passed the barrier after their restore, so no staged word is read again)
  float (*red)[20] = reinterpret_cast<float (*)[20]>(codes);
  float r_row = 0.0f, m_row = 0.0f;
  if (dual(SCALE)) {
    m_row = row_reduce<false>(S, red, l) * 0.0078125f;
    const float nu = rn_div(m_row, sh.ir[row]);   // omega of the row
    r_row = (nu == 0.0f) ? 1.0f : rn_sqrt(nu);
  } else {
    const float mx = row_reduce<true>(S, red, l);
    r_row = (mx < FLT_MIN) ? 1.0f : mx;
  }
  if constexpr (SC16) r_row = bf16_up(r_row);
  if (!my_int) { r_row = 0.0f; m_row = 0.0f; }
  // Pivot rows leave their stored bits (fp16 or fp32 of S) in LDS now (the
  // row reduction's scratch is free), so the Y pass can zero them (factor 0):
  // they add nothing to the column maximum or the refit sums, and their code
  // bits are replaced by the stash afterwards.
  uint32_t *stash = codes;   // [pivot rank][column]
  if (pivots != 0) {
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      if (((pivots >> (8 * g8)) & 0xFFu) == 0u) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ii = 8 * g8 + e;
        if (!((pivots >> ii) & 1u)) continue;
        const bool f32row = (fp32_rows >> ii) & 1u;
        const int rank = __builtin_popcountll(pivots & ((1ull << ii) - 1ull));
#pragma unroll
        for (int c = 0; c < 2; ++c)
          stash[rank * 128 + l + 64 * c] = f32row ? __float_as_uint(S.get(c, ii))
                                                  : (uint32_t)__half_as_ushort(__float2half_rn(pin_f32(S.get(c, ii))));
      }
    }
  }
  sh.ir[row] = my_int ? rn_div(1.0f, r_row) : 0.0f;
  sh.m[row] = m_row;
  // factors are stored as soon as they are known (every read of the block
  // was issued and waited for before the restore)
  if (has_int) store_sc<SC16>(rs, r_row, (uint32_t)l, r_off + (uint32_t)w * 64u * SCB);
  __builtin_amdgcn_wave_barrier();

  // Y = S / r in place (integer rows; pivot rows become 0), and the column
  // maximum, to which only integer rows contribute
  float cm[2] = {0.0f, 0.0f};
  row_groups<kAhead>(&sh.ir[64 * w], [&](int i4, const float4 r4) {
    const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = 4 * i4 + e;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float y = S.get(c, ii) * rr[e];
        S.set(c, ii, y);
        cm[c] = fmaxf(cm[c], fabsf(y));
      }
    }
  });
  float c0[2] = {1.0f, 1.0f};
  if (dual(SCALE)) {
    sh.cmax[w][l] = cm[0];
    sh.cmax[w][l + 64] = cm[1];
  }
  __syncthreads();
  if (dual(SCALE)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float mx = fmaxf(sh.cmax[0][l + 64 * c], sh.cmax[1][l + 64 * c]);
      c0[c] = (mx < FLT_MIN) ? 1.0f : mx;
      if constexpr (SC16) c0[c] = bf16_up(c0[c]);
    }
  }
  float ec[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) ec[c] = dual(SCALE) ? rn_div(1.0f, c0[c]) : 1.0f;
  if (dual(SCALE) && has_int && !FIT && w == 0) {
    store_sc<SC16>(rs, c0[0], (uint32_t)l, c_off);
    store_sc<SC16>(rs, c0[1], (uint32_t)l + 64u, c_off);
  }

  // ---------------- codes.  Pivot rows first leave their stored bits (fp16
  // or fp32 of S) in LDS; P1 turns every value into its code bits in place
  // (straight-line); P2 appends each row's field to the column windows in
  // row order and stores every completed word.
  // V1a refit sums: each wave runs an fma chain over its own integer rows in
  // ascending order; wave 1 adds wave 0's sums to its own at the end
  float nacc[2] = {0.0f, 0.0f}, dacc[2] = {0.0f, 0.0f};
  // code bits replace the values in place (the tile holds the bit patterns)
  row_groups<kAhead>(&sh.qm[64 * w], [&](int i4, const float4 q4) {
    const float qq[4] = {q4.x, q4.y, q4.z, q4.w};
    float4 m4 = {0, 0, 0, 0}, iq4 = {0, 0, 0, 0};
    if (FIT) { m4 = lds4(&sh.m[64 * w + 4 * i4]); iq4 = lds4(&sh.iq[64 * w + 4 * i4]); }
    const float mm[4] = {m4.x, m4.y, m4.z, m4.w};
    const float iqq[4] = {iq4.x, iq4.y, iq4.z, iq4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = 4 * i4 + e;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float y = S.get(c, ii);
        const float t = __builtin_fmaf(y, ec[c] * qq[e], kMagic);
        if (FIT) {
          // pivot rows: 1/q is stored as 0, so they add exact zeros
          const float zeta = (t - kMagic) * iqq[e];
          const float pz = mm[e] * zeta;
          nacc[c] = __builtin_fmaf(pz, y, nacc[c]);
          dacc[c] = __builtin_fmaf(pz, zeta, dacc[c]);
        }
        S.set(c, ii, t);
      }
    }
  });
  if (FIT && dual(SCALE)) {
    if (w == 0) {
      sh.d[l] = nacc[0]; sh.d[l + 64] = nacc[1];
      sh.y[l] = dacc[0]; sh.y[l + 64] = dacc[1];
    }
    __syncthreads();
  }
  if (pivots != 0) {
    // pivot rows: their stored bits replace the code bits
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      if (((pivots >> (8 * g8)) & 0xFFu) == 0u) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ii = 8 * g8 + e;
        if (!((pivots >> ii) & 1u)) continue;
        const int rank = __builtin_popcountll(pivots & ((1ull << ii) - 1ull));
        S.set(0, ii, __uint_as_float(stash[rank * 128 + l]));
        S.set(1, ii, __uint_as_float(stash[rank * 128 + l + 64]));
      }
    }
  }
  {
    // the completed words go to the wave's LDS region (the stash has been
    // read), then out with 16-byte stores, 1 KiB of the half per instruction
    uint32_t win[2] = {0u, 0u};   // the last 32 stream bits written, per column
    if (fp32_rows == 0) {
      // every field is at most 16 bits wide: straight-line appends; a field
      // that completes its word (the program word's flag, a uniform branch)
      // also writes that word.  A word left incomplete by the last field is
      // written by the final flush.
      // this pass reads no LDS, so the program words come in by scalar loads
      // (constant address space), eight rows per load, one batch ahead,
      // instead of a v_readlane per row
      typedef __attribute__((address_space(4))) const uint32_t cu32;
      cu32 *pw = (cu32 *)(uintptr_t)prog;   // {xs, z} per row
      uint32_t pb[2][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[0][e] = pw[2 * e];
#pragma unroll
      for (int b8 = 0; b8 < 8; ++b8) {
        if (b8 + 1 < 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[(b8 + 1) & 1][e] = pw[2 * (8 * (b8 + 1) + e)];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ii = 8 * b8 + e;
          const uint32_t pe = pb[b8 & 1][e];
          const uint32_t t0 = __float_as_uint(S.get(0, ii)), t1 = __float_as_uint(S.get(1, ii));
          if (pe & kRowCompletes) {
            uint32_t *o = reinterpret_cast<uint32_t *>(codes8 + (rp_base(pe) | lane_byte));
            o[0] = __builtin_amdgcn_alignbit(t0, win[0], rp_pack_shift(pe));
            o[64] = __builtin_amdgcn_alignbit(t1, win[1], rp_pack_shift(pe));
          }
          win[0] = __builtin_amdgcn_alignbit(t0, win[0], rp_width(pe));
          win[1] = __builtin_amdgcn_alignbit(t1, win[1], rp_width(pe));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < 64; ++ii) {
        const uint32_t pe = row_lane(xs_v, ii);
        const uint32_t off = (rp_base(pe) >> 4) + (pe & 31u);   // stream bit of the field in this half
        const uint32_t t0 = __float_as_uint(S.get(0, ii)), t1 = __float_as_uint(S.get(1, ii));
        if ((fp32_rows >> ii) & 1u) {   // an FP32 row: its two 16-bit halves in turn
          append_field(codes, l, win, t0, t1, off, 16u);
          append_field(codes, l, win, t0 >> 16, t1 >> 16, off + 16u, 16u);
        } else {
          append_field(codes, l, win, t0, t1, off, rp_width(pe));
        }
      }
    }
    // a partly filled last word: its bits sit at the top of the window;
    // shift them down with zeros above (the padding of the half)
    const uint32_t plast = row_lane(xs_v, 63);
    const uint32_t end = (rp_base(plast) >> 4) + (plast & 31u) + (((fp32_rows >> 63) & 1u) ? 32u : rp_width(plast));
    const uint32_t rem = end & 31u;
    if (rem != 0u) {
      uint32_t *o = codes + (end >> 5) * kDim + l;
      o[0] = __builtin_amdgcn_alignbit(0u, win[0], 32u - rem);
      o[64] = __builtin_amdgcn_alignbit(0u, win[1], 32u - rem);
    }
    __builtin_amdgcn_wave_barrier();
    // eight LDS reads ahead of their stores, as in the staging
    const uint32_t nchunks = (half_bytes + 1023u) >> 10;
    for (uint32_t g0 = 0; g0 < nchunks; g0 += 8u) {
      uint4 t[8];
#pragma unroll
      for (uint32_t u = 0; u < 8u; ++u)
        if (g0 + u < nchunks) t[u] = *reinterpret_cast<const uint4 *>(codes8 + (g0 + u) * 1024u + (uint32_t)l * 16u);
#pragma unroll
      for (uint32_t u = 0; u < 8u; ++u) {
        const uint32_t boff = (g0 + u) * 1024u + (uint32_t)l * 16u;
        if (g0 + u < nchunks && boff < half_bytes) store_granule(rs, t[u], boff, half_off);
      }
    }
  }

  // ---------------- refitted column factors
  if (FIT && dual(SCALE) && has_int) {
    if (w == 1) {
      // wave 0's sums (rows 0..63) plus wave 1's (rows 64..127)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float nn = sh.d[l + 64 * c] + nacc[c], dd = sh.y[l + 64 * c] + dacc[c];
        float cf = (dd > 0.0f) ? rn_div(nn, dd) : c0[c];
        if constexpr (SC16) cf = bf16_nearest(cf);
        store_sc<SC16>(rs, cf, (uint32_t)l + 64u * c, c_off);
      }
    }
  }

}

// --------------------------------------------------------------------------
// launch helpers (instantiated per storage kind in the qdr_head_*.hip units)
// --------------------------------------------------------------------------
namespace {

// Calls f(GATE, SCALE, FIT) -- each a std::integral_constant -- with the
// template arguments of the pool: the gate form, the scale mode and width
// (SCALE bit 0: row absmax, bit 1: bfloat16 factors) and the refit (dual-axis
// scales only).
template <class F>
void with_variant(const PoolConfig &cfg, F &&f) {
  using std::integral_constant;
  const bool diag = cfg.gate == 1, fit = cfg.fit_iters > 0;
  const int s = (cfg.scale_mode == 0 ? 0 : 1) | (cfg.scale_bits == 16 ? 2 : 0);
  auto go = [&](auto g) {
    switch (s) {
      case 0:
        if (fit) f(g, integral_constant<int, 0>{}, integral_constant<int, 1>{});
        else f(g, integral_constant<int, 0>{}, integral_constant<int, 0>{});
        break;
      case 1: f(g, integral_constant<int, 1>{}, integral_constant<int, 0>{}); break;
      case 2:
        if (fit) f(g, integral_constant<int, 2>{}, integral_constant<int, 1>{});
        else f(g, integral_constant<int, 2>{}, integral_constant<int, 0>{});
        break;
      default: f(g, integral_constant<int, 3>{}, integral_constant<int, 0>{}); break;
    }
  };
  if (diag) go(integral_constant<int, 1>{});
  else go(integral_constant<int, 0>{});
}

template <int BITS, int MODE>
hipError_t launch_head_kind(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)n * a.n_list)), block(128);
  if (grid.x == 0) return hipSuccess;
  if (!Kind<BITS>::is_int) {   // float kinds store no factors
    if (cfg.gate == 1) hipLaunchKernelGGL((k_head<BITS, MODE, 1, 0, 0>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_head<BITS, MODE, 0, 0, 0>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  with_variant(cfg, [&](auto G, auto S, auto Fi) {
    hipLaunchKernelGGL((k_head<BITS, MODE, decltype(G)::value, decltype(S)::value, decltype(Fi)::value>), grid,
                       block, 0, st, a);
  });
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_head_int_mode(const PoolConfig &cfg, const LaunchArgs &a, int n, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)n * a.n_list)), block(128);
  if (grid.x == 0) return hipSuccess;
  with_variant(cfg, [&](auto G, auto S, auto Fi) {
    hipLaunchKernelGGL((k_head_int<MODE, decltype(G)::value, decltype(S)::value, decltype(Fi)::value>), grid,
                       block, 0, st, a);
  });
  return hipGetLastError();
}

// Every mode of the whole-head kernel for one storage kind.
template <int BITS>
hipError_t launch_head_modes(const PoolConfig &cfg, const LaunchArgs &a, int n, int mode, hipStream_t st) {
  switch (mode) {
    case MODE_STEP: return launch_head_kind<BITS, MODE_STEP>(cfg, a, n, st);
    case MODE_READOUT: return launch_head_kind<BITS, MODE_READOUT>(cfg, a, n, st);
    case MODE_STEP_BF16: return launch_head_kind<BITS, MODE_STEP_BF16>(cfg, a, n, st);
    case MODE_WRITEBACK: return launch_head_kind<BITS, MODE_WRITEBACK>(cfg, a, n, st);
    case MODE_PACK: return launch_head_kind<BITS, MODE_PACK>(cfg, a, n, st);
    case MODE_UNPACK: return launch_head_kind<BITS, MODE_UNPACK>(cfg, a, n, st);
    default: return launch_head_kind<BITS, MODE_RESET>(cfg, a, n, st);
  }
}

}  // namespace

}  // namespace qdr
