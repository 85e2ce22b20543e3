/*
 * oracle_sanitize.c -- drives every entry point of the CPU oracle
 * (oracle/qdr_oracle.c) over small pools of every storage kind, unit,
 * gate form, scale mode, factor width and refit option, on one thread and
 * on several, so that an AddressSanitizer / UndefinedBehaviorSanitizer
 * build of the oracle sees every code path the tests use.  Test
 * infrastructure: built and run by tests/test_sanitizers.py.
 *
 * Prints "ok <n>" (n = pool steps run) and exits 0; any sanitizer report
 * aborts with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/qdr_oracle.h"

#define D 128

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {   /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float uniform(void) { return (float)((next_u32() >> 8) * (1.0 / 16777216.0)); }
static float normal(void) {
  float a = uniform() + 1e-7f, b = uniform();
  return sqrtf(-2.0f * logf(a)) * cosf(6.2831853f * b);
}

static const uint8_t kKinds[6] = {2, 4, 6, 8, 16, 32};

static int run_pool(int unit, int gate, int scale_mode, int fit, int scale_bits, int threads) {
  const int H = 3, slots_n = 4, B = 3;
  uint8_t *kinds = malloc(unit == OR_UNIT_HEAD ? H : H * D);
  float *omega = malloc(sizeof(float) * H * D);
  for (int i = 0; i < (unit == OR_UNIT_HEAD ? H : H * D); ++i) kinds[i] = kKinds[next_u32() % 6];
  if (unit == OR_UNIT_ROW) kinds[D + 9] = 32;          /* at least one FP32 row */
  for (int i = 0; i < H * D; ++i) omega[i] = expf(normal());
  or_pool_desc desc = {slots_n, H, unit, gate, scale_mode, fit, kinds, omega, scale_bits};
  uint64_t head_off[3], stride = 0, total = 0;
  if (or_pool_layout(&desc, head_off, &stride, &total) != 0) return -1;
  uint8_t *pool = calloc(total, 1);
  float *S = malloc(sizeof(float) * slots_n * H * D * D);
  for (size_t i = 0; i < (size_t)slots_n * H * D * D; ++i) S[i] = normal() * 3.0f;
  /* FP16 rows stay inside the binary16 range; one zero row, one zero head */
  memset(S + (size_t)D * 7, 0, sizeof(float) * D);
  memset(S + (size_t)D * D * 2, 0, sizeof(float) * D * D);
  int32_t all[4] = {0, 1, 2, 3};
  or_pool_pack(&desc, pool, all, slots_n, S, threads);
  const size_t nv = (size_t)B * H * D;
  float *q = malloc(sizeof(float) * nv), *k = malloc(sizeof(float) * nv), *v = malloc(sizeof(float) * nv);
  float *beta = malloc(sizeof(float) * B * H), *g = malloc(sizeof(float) * nv), *o = malloc(sizeof(float) * nv);
  float *om = malloc(sizeof(float) * nv);
  int32_t slots[3] = {2, -1, 0};
  int steps = 0;
  for (int t = 0; t < 4; ++t) {
    for (size_t i = 0; i < nv; ++i) { q[i] = normal() * 0.1f; k[i] = normal() * 0.09f; v[i] = normal(); g[i] = 0.5f + 0.5f * uniform(); }
    for (int i = 0; i < B * H; ++i) beta[i] = uniform();
    if (t == 3) slots[1] = 9;                            /* an out-of-range slot is reported */
    const int bad = or_pool_step(&desc, pool, slots, B, q, k, v, beta, g, o, threads, (t & 1) ? om : NULL);
    if (bad != (t == 3 ? 1 : 0)) return -2;
    ++steps;
  }
  or_pool_unpack(&desc, pool, all, slots_n, S, threads);
  /* single-head entry points and the block codec */
  uint8_t hk[D];
  for (int i = 0; i < D; ++i) hk[i] = unit == OR_UNIT_HEAD ? kinds[1] : kinds[D + i];
  uint32_t *e = calloc(D * D, 4);
  float r[D], c[D], m[D], oo[D], *Spre = malloc(sizeof(float) * D * D);
  for (int i = 0; i < D; ++i) for (int j = 0; j < D; ++j) if (hk[i] == 16) S[i * D + j] = fminf(fmaxf(S[i * D + j], -6e4f), 6e4f);
  or_requant(D, hk, S, omega + D, scale_mode, fit, scale_bits, e, r, c, m);
  uint8_t *blk = calloc(or_block_bytes(hk, unit, scale_mode, scale_bits), 1);
  or_encode_block(hk, unit, scale_mode, scale_bits, e, r, c, blk);
  or_decode_block(hk, unit, scale_mode, scale_bits, blk, e, r, c);
  or_head_step(D, hk, e, r, c, omega + D, scale_mode, fit, scale_bits, q, k, v, 0.5f, g, oo, Spre);
  float fs[D];
  for (int i = 0; i < D; ++i) fs[i] = normal();
  (void)or_fold_sum(fs, D);
  for (uint32_t h = 0; h < 65536; h += 97) (void)or_f32_to_f16(or_f16_to_f32((uint16_t)h));
  (void)or_bf16_up(3.3f);
  (void)or_bf16_nearest(3.3f);
  free(blk); free(Spre); free(e);
  free(q); free(k); free(v); free(beta); free(g); free(o); free(om);
  free(S); free(pool); free(kinds); free(omega);
  return steps;
}

int main(void) {
  int total = 0;
  for (int unit = 0; unit < 2; ++unit)
    for (int gate = 0; gate < 2; ++gate)
      for (int mode = 0; mode < 2; ++mode)
        for (int fit = 0; fit < 2; ++fit)
          for (int sb = 16; sb <= 32; sb += 16)
            for (int th = 1; th <= 3; th += 2) {
              if (fit && mode == OR_SCALE_ROW_ABSMAX) continue;
              const int n = run_pool(unit, gate, mode, fit, sb, th);
              if (n < 0) {
                fprintf(stderr, "failed: unit %d gate %d mode %d fit %d sb %d threads %d (%d)\n",
                        unit, gate, mode, fit, sb, th, n);
                return 1;
              }
              total += n;
            }
  printf("ok %d\n", total);
  return 0;
}
