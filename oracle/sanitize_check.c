/*
 * sanitize_check.c -- drives every entry point of the CPU oracle (csa2_oracle.c) once on
 * small, ragged inputs so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitized.py: gcc -fsanitize=address,undefined) reports any
 * out-of-bounds access, use of uninitialised heap, overflow or invalid shift in the oracle.
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself.  It checks no values (the pins in
 * tests/ do that); it only exercises the code paths: both compression ratios, static and
 * per-token pooling weights, Full and candidate scoring, the block selection with a pool
 * that does and does not cover every block, ties, NaN scores, -1 padded Top-K rows, empty
 * and clamped windows, FP8 window rings, the MXFP4 query and HISA block means.
 * Inputs come from a fixed linear congruential generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "csa2_oracle.h"

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}
static float next_f(void) { return ((float)(next_u32() >> 8) / 16777216.0f) * 2.0f - 1.0f; }
static uint16_t bf16_of(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

int main(void) {
  /* scalar formats over every code */
  double acc = 0.0;
  for (int c = 0; c < 16; c++) acc += csa2o_e2m1_value(c);
  for (int b = 0; b < 256; b++) acc += isnan(csa2o_e4m3_value(b)) ? 0.0 : csa2o_e4m3_value(b);
  for (int b = 0; b < 255; b++) acc += csa2o_e8m0_value(b) > 0.0 ? 1.0 : 0.0;
  const float probes[] = {0.0f, 1e-30f, 1e-8f, 0.25f, 1.0f, 6.0f, 448.0f, 2688.0f, 1e30f, INFINITY};
  for (int i = 0; i < 10; i++) {
    acc += csa2o_e4m3_encode(probes[i]) + csa2o_e8m0_scale_code(probes[i]) + csa2o_e8m0_scale_code_e4m3(probes[i]);
    acc += csa2o_e2m1_encode(probes[i], 1.0) + csa2o_e2m1_encode(-probes[i], 0.5);
  }
  acc += (double)csa2o_entry_bytes(512, 16) + (double)csa2o_entry_bytes(128, 32) + (double)csa2o_swa_fp8_row_bytes();

  /* stage 1: both ratios, static and per-token weights */
  const int64_t n = 70;
  for (int m = 1; m <= 2; m++) {
    for (int per_token = 0; per_token <= 1; per_token++) {
      uint16_t *lat = xmalloc(sizeof(uint16_t) * n * m * 512);
      float *pw = xmalloc(sizeof(float) * n * m * 512);
      int64_t *pos = xmalloc(sizeof(int64_t) * n);
      float *cs = xmalloc(sizeof(float) * n * 64);
      uint16_t *w = xmalloc(sizeof(uint16_t) * 128 * 512);
      uint8_t *kv = xmalloc((size_t)n * 288), *ix = xmalloc((size_t)n * 68);
      float *pooled = xmalloc(sizeof(float) * n * 512), *rot = xmalloc(sizeof(float) * n * 512);
      float *kp = xmalloc(sizeof(float) * n * 128);
      for (int64_t i = 0; i < n * m * 512; i++) lat[i] = bf16_of(3.0f * next_f());
      for (int64_t i = 0; i < n * m * 512; i++) pw[i] = 0.01f + fabsf(next_f());
      for (int64_t i = 0; i < n; i++) pos[i] = i * m + 977;
      for (int64_t i = 0; i < 128 * 512; i++) w[i] = bf16_of(next_f() / 22.6f);
      csa2o_rope_table(pos, n, 160000.0, cs);
      csa2o_compress_pack(lat, n, m, m == 1 && per_token ? NULL : pw, per_token, cs, w, kv, ix, pooled, rot, kp);
      csa2o_compress_pack(lat, n, m, pw, per_token, cs, w, kv, ix, NULL, NULL, NULL);
      double d512[512], d128[128];
      csa2o_dequant_kv(kv + 288 * (n - 1), d512);
      csa2o_dequant_idx(ix + 68 * (n - 1), d128);
      acc += d512[511] + d128[127] + pooled[0] + rot[511] + kp[127];
      free(lat), free(pw), free(pos), free(cs), free(w), free(kv), free(ix), free(pooled), free(rot), free(kp);
    }
  }

  /* stages 2-4 over two ragged sequences: 300 and 37 entries (the pool covers every block of
   * the second one and not of the first with M = 16) */
  const int32_t n_q = 2, rows = 337, width = 300, M = 16, K = 24;
  uint8_t *kv = xmalloc((size_t)rows * 288), *ix = xmalloc((size_t)rows * 68);
  for (int64_t i = 0; i < (int64_t)rows * 288; i++) kv[i] = (uint8_t)next_u32();
  for (int64_t i = 0; i < (int64_t)rows * 68; i++) ix[i] = (uint8_t)next_u32();
  for (int32_t r = 0; r < rows; r++) {
    for (int g = 0; g < 32; g++) kv[r * 288 + 256 + g] = (uint8_t)(0x20 + next_u32() % 25);
    for (int g = 0; g < 4; g++) ix[r * 68 + 64 + g] = (uint8_t)(120 + next_u32() % 10);
  }
  uint16_t *q_idx = xmalloc(sizeof(uint16_t) * n_q * 32 * 128);
  float *hw = xmalloc(sizeof(float) * n_q * 32);
  for (int i = 0; i < n_q * 32 * 128; i++) q_idx[i] = bf16_of(next_f() / 11.3f);
  for (int i = 0; i < n_q * 32; i++) hw[i] = next_f() / 5.7f;
  const int64_t base[2] = {0, 300};
  const int32_t nvis[2] = {300, 37};
  float *s = xmalloc(sizeof(float) * n_q * width);
  csa2o_index_score(q_idx, hw, ix, base, nvis, NULL, 0, n_q, width, s);
  uint8_t *q4 = xmalloc((size_t)n_q * 32 * 68);
  csa2o_quantize_q_mxfp4(q_idx, n_q * 32, q4);
  csa2o_index_score_fp4q(q4, hw, ix, base, nvis, NULL, 0, n_q, width, s);
  s[5] = s[6];          /* a tie */
  s[7] = NAN;           /* NaN ranks as -inf */
  int32_t *pool = xmalloc(sizeof(int32_t) * n_q * M), *topk = xmalloc(sizeof(int32_t) * n_q * K);
  csa2o_block_topk(s, n_q, width, nvis, NULL, 8, M, K, pool, topk);
  csa2o_block_topk(s, n_q, width, nvis, NULL, 8, M, K, NULL, topk);
  csa2o_topk_bruteforce(s, n_q, width, nvis, K, topk);
  float *sc = xmalloc(sizeof(float) * n_q * 8 * M);
  csa2o_index_score(q_idx, hw, ix, base, nvis, pool, M, n_q, 8 * M, sc);
  csa2o_index_score_fp4q(q4, hw, ix, base, nvis, pool, M, n_q, 8 * M, sc);
  csa2o_block_topk(sc, n_q, 8 * M, nvis, pool, 8, M, K, NULL, topk);
  /* HISA: block means of sequence 0, their scores and the pool from them */
  uint8_t *means = xmalloc((size_t)((300 + 7) / 8) * 68);
  csa2o_block_mean_pack(ix, 300, 8, means);
  const int32_t nbw = (300 + 7) / 8, nv1[1] = {300};
  const int64_t b0[1] = {0};
  const int32_t nmeans[1] = {nbw};
  float *sb = xmalloc(sizeof(float) * nbw);
  csa2o_index_score(q_idx, hw, means, b0, nmeans, NULL, 0, 1, nbw, sb);
  csa2o_pool_from_block_scores(sb, 1, nbw, nv1, 8, M, pool);

  /* stage 4: topk row 1 padded with -1, window lengths 128 and 0 (a query with only entries),
   * bf16 rows and FP8 rings */
  for (int i = 0; i < K; i += 3) topk[K + i] = -1;
  uint16_t *q = xmalloc(sizeof(uint16_t) * n_q * 64 * 512);
  for (int i = 0; i < n_q * 64 * 512; i++) q[i] = bf16_of(next_f());
  const int32_t swa_rows = 256;
  uint16_t *swa = xmalloc(sizeof(uint16_t) * swa_rows * 512);
  for (int i = 0; i < swa_rows * 512; i++) swa[i] = bf16_of(next_f());
  const int64_t swa_start[2] = {0, 128};
  const int32_t swa_len[2] = {128, 0};
  float *out = xmalloc(sizeof(float) * n_q * 64 * 512), *lse = xmalloc(sizeof(float) * n_q * 64);
  csa2o_sparse_attn(q, kv, base, topk, K, swa, swa_start, swa_len, 0.0441941738f, out, lse, n_q);
  csa2o_sparse_attn(q, kv, base, topk, K, swa, swa_start, swa_len, 0.0441941738f, out, NULL, n_q);
  uint8_t *swa8 = xmalloc((size_t)swa_rows * 584);
  csa2o_swa_fp8_pack(swa, swa_rows, swa8);
  double d512[512];
  csa2o_dequant_swa_fp8(swa8 + 584 * 7, d512);
  const int64_t ring_start[2] = {100, 128 + 5};
  csa2o_sparse_attn_swa_fp8(q, kv, base, topk, K, swa8, 0, swa_start, swa_len, 0.0441941738f, out, lse, n_q);
  csa2o_sparse_attn_swa_fp8(q, kv, base, topk, K, swa8, 128, ring_start, swa_len, 0.0441941738f, out, lse, n_q);
  acc += out[0] + lse[0] + d512[0] + sb[0];

  free(kv), free(ix), free(q_idx), free(hw), free(s), free(q4), free(pool), free(topk), free(sc), free(means);
  free(sb), free(q), free(swa), free(out), free(lse), free(swa8);
  printf("oracle exercised (checksum %g)\n", acc);
  return 0;
}
