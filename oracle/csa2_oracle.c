/*
 * csa2_oracle.c -- plain, single-threaded CPU oracle for the CSA2 global branch.
 *
 * TEST INFRASTRUCTURE ONLY (see csa2_oracle.h).  Built with -O2 -ffp-contract=off and
 * without fast-math so every fp32 operation below is one IEEE round-to-nearest op.
 *
 * What it computes, step by step, in the order the pages give it:
 *   compressor pooling   [DF] §4.2 compressor equation; [ZB] §2.3.1 (no overlap, no
 *                        absolute position embedding; m = 1 is per-token projection)
 *   RoPE then quantise   [ZB] §2.4.4 (quantise after RoPE, same format for NoPE/RoPE)
 *   main-KV FP4          [ZB] §2.4.4, [DF] §4.4-4.5: E2M1 with one E4M3 scale per 16
 *   indexer-K            [ZB] §2.3.1 (indexer K projected from the main-KV entry),
 *                        [DF] §4.4: MXFP4 = E2M1 with one E8M0 scale per 32
 *   indexer scores       [ZB] §3.3.2 (indexer query with per-head weights)
 *   block max / pool     [ZB] §2.3.4 (pad with -inf, amax over blocks of 8, newest
 *                        block forced to +inf, expand selected blocks, truncate to width),
 *                        [DF] §4.7 pool equations (g_r, TopM, union)
 *   Top-K                [ZB] model table index_topk = 512
 *   sparse attention     [ZB] §3.3.2.1 (key = value = c, one softmax over the selected
 *                        entries joined with the SWA keys)
 *
 * Readings of points the pages leave open (each also listed in the design notes):
 *   - pooling uses normalised weights a_i = w_i / sum(w), then sum a_i x_i (ascending i);
 *     mathematically the compressor equation, and equal weights give exactly the mean.
 *   - RoPE on channels 448..511 in adjacent pairs (448+2i, 449+2i), angle from a table.
 *   - E4M3 scale = nearest-even E4M3 of fp32(amax / 6), saturating at 448; S = 0 -> all
 *     codes 0.  Element code = grid point nearest to |e| / S (exact), ties to even code,
 *     saturating at 6; sign bit only on a non-zero code.
 *   - E8M0 scale code = floor(log2 amax) - 2 + 127 clamped to [0, 254]; amax = 0 -> 0.
 *   - indexer K = ascending fmaf chain over the 512 post-RoPE fp32 channels.
 *   - score = sum_h w_h * max(0, q_h . k): the lightning-indexer form; no extra scale.
 *   - ties in block and entry selection go to the lower index; NaN ranks as -inf.
 *   - attention logit = scale * q_h . key over all 512 dims; value = the same key.
 */
#include "csa2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define D_LAT 512
#define D_ROPE 64
#define D_NOPE (D_LAT - D_ROPE)
#define IDX_HEADS 32
#define IDX_DIM 128
#define N_HEADS 64
#define KV_BYTES 288
#define IDX_BYTES 68

static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int64_t csa2o_entry_bytes(int64_t D, int64_t G) { return D / 2 + D / G; }

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ formats */

double csa2o_e2m1_value(int code4) {
  double v = kE2M1[code4 & 7];
  return (code4 & 8) ? -v : v;
}

double csa2o_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return NAN;
  /* normal: (1 + m/8) 2^(e-7); subnormal: (m/8) 2^(-6) */
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

double csa2o_e8m0_value(int byte) {
  if ((byte & 255) == 255) return NAN;
  return ldexp(1.0, (byte & 255) - 127);
}

/* Nearest non-negative E4M3 value by scanning every finite code, ties to the even code. */
int csa2o_e4m3_encode(double x) {
  if (!(x < 448.0)) return 0x7E; /* saturate (also +inf / NaN) */
  if (x <= 0.0) return 0x00;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    double d = fabs(x - csa2o_e4m3_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Nearest grid point g*S to |e| over g in {0,0.5,1,1.5,2,3,4,6}, ties to the even code. */
int csa2o_e2m1_encode(float e, double S) {
  if (!(S > 0.0)) return 0;
  double a = fabs((double)e);
  int best = 0;
  if (a >= 6.0 * S) {
    best = 7;
  } else {
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
      double d = fabs(a - kE2M1[c] * S);
      if (d < bestd || (d == bestd && (c & 1) == 0)) {
        best = c;
        bestd = d;
      }
    }
  }
  return (e < 0.0f && best != 0) ? (best | 8) : best;
}

int csa2o_e8m0_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0;
  if (isinf(amax)) return 254; /* a group holding an infinity takes the largest finite scale */
  int ex;
  frexpf(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
  int code = (ex - 1) - 2 + 127;
  if (code < 0) code = 0;
  if (code > 254) code = 254;
  return code;
}

/* ------------------------------------------------------------------ RoPE table */

void csa2o_rope_table(const int64_t *pos, int64_t n, double theta, float *out) {
  for (int64_t j = 0; j < n; j++) {
    for (int i = 0; i < D_ROPE / 2; i++) {
      double inv_freq = pow(theta, -(double)(2 * i) / (double)D_ROPE);
      double ang = (double)pos[j] * inv_freq;
      out[j * D_ROPE + i] = (float)cos(ang);
      out[j * D_ROPE + D_ROPE / 2 + i] = (float)sin(ang);
    }
  }
}

/* ------------------------------------------------------------------ stage 1 */

static void pack_nibbles(const int *codes, int n, uint8_t *dst) {
  for (int b = 0; b < n / 2; b++) dst[b] = (uint8_t)((codes[2 * b] & 15) | ((codes[2 * b + 1] & 15) << 4));
}

void csa2o_compress_pack(const uint16_t *latent, int64_t n_entries, int m, const float *pool_w,
                         int per_token_w, const float *rope_cs, const uint16_t *w_idx, uint8_t *kv_out,
                         uint8_t *idx_out, float *pooled, float *rotated, float *kproj) {
  float c[D_LAT];
  float k[IDX_DIM];
  int codes[D_LAT];
  for (int64_t j = 0; j < n_entries; j++) {
    /* a1: c_j[ch] = sum_i a_i[ch] x_{m j + i}[ch], a_i = w_i / sum_i' w_i'.  The weights
     * are static per channel ([m, 512]) or, with per_token_w, one row per latent token
     * ([n_entries * m, 512]: the gate of token m j + i is row m j + i), the same formula
     * ([DF] §4.2 remarks that the pooling weights may be projected from the input). */
    const float *w = (per_token_w && m > 1) ? pool_w + (j * m) * D_LAT : pool_w;
    for (int ch = 0; ch < D_LAT; ch++) {
      const uint16_t *x = latent + (j * m) * D_LAT + ch;
      if (m == 1) {
        c[ch] = bf16_to_f32(x[0]);
      } else {
        float wsum = w[ch];
        for (int i = 1; i < m; i++) wsum = wsum + w[i * D_LAT + ch];
        float acc = (w[ch] / wsum) * bf16_to_f32(x[0]);
        for (int i = 1; i < m; i++) acc = acc + (w[i * D_LAT + ch] / wsum) * bf16_to_f32(x[i * D_LAT]);
        c[ch] = acc;
      }
    }
    if (pooled) memcpy(pooled + j * D_LAT, c, sizeof c);

    /* a2: rotate the 64-channel rope tail in adjacent pairs */
    const float *cs = rope_cs + j * D_ROPE;
    for (int i = 0; i < D_ROPE / 2; i++) {
      float x0 = c[D_NOPE + 2 * i], x1 = c[D_NOPE + 2 * i + 1];
      float co = cs[i], si = cs[D_ROPE / 2 + i];
      float t0 = x0 * co, t1 = x1 * si, t2 = x0 * si, t3 = x1 * co;
      c[D_NOPE + 2 * i] = t0 - t1;
      c[D_NOPE + 2 * i + 1] = t2 + t3;
    }
    if (rotated) memcpy(rotated + j * D_LAT, c, sizeof c);

    /* a3: main KV, 32 groups of 16 channels, E4M3 scale + E2M1 codes */
    uint8_t *kv = kv_out + j * KV_BYTES;
    for (int g = 0; g < D_LAT / 16; g++) {
      float amax = 0.0f;
      for (int i = 0; i < 16; i++) {
        float a = fabsf(c[16 * g + i]);
        if (a > amax) amax = a;
      }
      float s_raw = amax / 6.0f;
      int sc = csa2o_e4m3_encode((double)s_raw);
      double S = csa2o_e4m3_value(sc);
      kv[256 + g] = (uint8_t)sc;
      for (int i = 0; i < 16; i++) codes[16 * g + i] = csa2o_e2m1_encode(c[16 * g + i], S);
    }
    pack_nibbles(codes, D_LAT, kv);

    /* a4: indexer K = W_idx c (ascending fmaf chain), then MXFP4 in 4 groups of 32 */
    for (int o = 0; o < IDX_DIM; o++) {
      float acc = 0.0f;
      for (int ch = 0; ch < D_LAT; ch++) acc = fmaf(bf16_to_f32(w_idx[o * D_LAT + ch]), c[ch], acc);
      k[o] = acc;
    }
    if (kproj) memcpy(kproj + j * IDX_DIM, k, sizeof k);
    uint8_t *ix = idx_out + j * IDX_BYTES;
    for (int g = 0; g < IDX_DIM / 32; g++) {
      float amax = 0.0f;
      for (int i = 0; i < 32; i++) {
        float a = fabsf(k[32 * g + i]);
        if (a > amax) amax = a;
      }
      int sc = csa2o_e8m0_scale_code(amax);
      double X = csa2o_e8m0_value(sc);
      ix[64 + g] = (uint8_t)sc;
      for (int i = 0; i < 32; i++) codes[32 * g + i] = csa2o_e2m1_encode(k[32 * g + i], X);
    }
    pack_nibbles(codes, IDX_DIM, ix);
  }
}

void csa2o_dequant_kv(const uint8_t *e, double *out) {
  for (int ch = 0; ch < D_LAT; ch++) {
    int code = (e[ch / 2] >> (4 * (ch & 1))) & 15;
    out[ch] = csa2o_e2m1_value(code) * csa2o_e4m3_value(e[256 + ch / 16]);
  }
}

void csa2o_dequant_idx(const uint8_t *e, double *out) {
  for (int ch = 0; ch < IDX_DIM; ch++) {
    int code = (e[ch / 2] >> (4 * (ch & 1))) & 15;
    out[ch] = csa2o_e2m1_value(code) * csa2o_e8m0_value(e[64 + ch / 32]);
  }
}

/* ------------------------------------------------------------------ stage 2 */

/* s = sum_h w_h max(0, q_h . k): q given as exact doubles [32 x 128] */
static double index_score_one(const double *q, const float *w, const uint8_t *entry) {
  double k[IDX_DIM];
  csa2o_dequant_idx(entry, k);
  double s = 0.0;
  for (int h = 0; h < IDX_HEADS; h++) {
    double dot = 0.0;
    for (int d = 0; d < IDX_DIM; d++) dot += q[h * IDX_DIM + d] * k[d];
    if (dot > 0.0) s += (double)w[h] * dot; /* ReLU, then the per-head weight */
  }
  return s;
}

static void index_score_rows(const double *qd, const float *head_w, const uint8_t *idx_cache,
                             const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                             int32_t M, int32_t n_q, int32_t width, float *scores) {
  for (int32_t t = 0; t < n_q; t++) {
    const double *q = qd + (int64_t)t * IDX_HEADS * IDX_DIM;
    const float *w = head_w + (int64_t)t * IDX_HEADS;
    float *row = scores + (int64_t)t * width;
    for (int32_t p = 0; p < width; p++) row[p] = -INFINITY;
    int32_t nvis = q_nvis[t];
    if (!pool_blocks) {
      for (int32_t j = 0; j < nvis && j < width; j++)
        row[j] = (float)index_score_one(q, w, idx_cache + (q_base[t] + j) * IDX_BYTES);
    } else {
      for (int32_t slot = 0; slot < M; slot++) {
        int32_t b = pool_blocks[(int64_t)t * M + slot];
        if (b < 0) continue;
        for (int o = 0; o < 8; o++) {
          int64_t j = (int64_t)b * 8 + o;
          if (j >= nvis || slot * 8 + o >= width) continue;
          row[slot * 8 + o] = (float)index_score_one(q, w, idx_cache + (q_base[t] + j) * IDX_BYTES);
        }
      }
    }
  }
}

void csa2o_index_score(const uint16_t *q_idx, const float *head_w, const uint8_t *idx_cache,
                       const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                       int32_t M, int32_t n_q, int32_t width, float *scores) {
  const int64_t nv = (int64_t)n_q * IDX_HEADS * IDX_DIM;
  double *qd = (double *)malloc(sizeof(double) * (size_t)(nv > 0 ? nv : 1));
  for (int64_t i = 0; i < nv; i++) qd[i] = (double)bf16_to_f32(q_idx[i]);
  index_score_rows(qd, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, n_q, width, scores);
  free(qd);
}

/* ------------------------------------------------------------------ FP4 indexer query */

/* The indexer query in MXFP4 ([ZB] §2.4.4: DeepSeek-V4 already trains the indexer Q and K
 * for FP4; the format is OCP MXFP4): each head's 128 channels are packed like an
 * indexer-K entry -- E2M1 codes, channel 2b in the low nibble of byte b, one E8M0 scale
 * per 32 channels by the MX rule -- into 68 bytes.  n_vec = n_q * 32 head vectors. */
void csa2o_quantize_q_mxfp4(const uint16_t *q_bf16, int64_t n_vec, uint8_t *out) {
  int codes[IDX_DIM];
  for (int64_t v = 0; v < n_vec; v++) {
    const uint16_t *x = q_bf16 + v * IDX_DIM;
    uint8_t *o = out + v * IDX_BYTES;
    for (int g = 0; g < IDX_DIM / 32; g++) {
      float amax = 0.0f;
      for (int i = 0; i < 32; i++) {
        float a = fabsf(bf16_to_f32(x[32 * g + i]));
        if (a > amax) amax = a;
      }
      int sc = csa2o_e8m0_scale_code(amax);
      double X = csa2o_e8m0_value(sc);
      o[64 + g] = (uint8_t)sc;
      for (int i = 0; i < 32; i++) codes[32 * g + i] = csa2o_e2m1_encode(bf16_to_f32(x[32 * g + i]), X);
    }
    pack_nibbles(codes, IDX_DIM, o);
  }
}

/* Stage 2 with the MXFP4 query: the same score, q_h the dequantised head vector. */
void csa2o_index_score_fp4q(const uint8_t *q_fp4, const float *head_w, const uint8_t *idx_cache,
                            const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                            int32_t M, int32_t n_q, int32_t width, float *scores) {
  const int64_t nh = (int64_t)n_q * IDX_HEADS;
  double *qd = (double *)malloc(sizeof(double) * (size_t)(nh > 0 ? nh * IDX_DIM : 1));
  for (int64_t v = 0; v < nh; v++) csa2o_dequant_idx(q_fp4 + v * IDX_BYTES, qd + v * IDX_DIM);
  index_score_rows(qd, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, n_q, width, scores);
  free(qd);
}

/* ------------------------------------------------------------------ stage 3 */

typedef struct {
  double key; /* score, NaN mapped to -inf */
  int64_t id; /* block id or entry id (for the tie rule) */
} ranked_t;

/* descending key, then ascending id */
static int cmp_rank(const void *a, const void *b) {
  const ranked_t *x = (const ranked_t *)a, *y = (const ranked_t *)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x < y) ? -1 : (x > y);
}

static double rank_key(float s) { return isnan(s) ? -INFINITY : (double)s; }

/* take the first min(n, K) of a ranked list, write their ids ascending, pad with -1 */
static void emit_sorted(ranked_t *r, int64_t n, int32_t K, int32_t *out) {
  qsort(r, (size_t)n, sizeof *r, cmp_rank);
  int32_t take = (int32_t)(n < K ? n : K);
  for (int32_t i = 0; i < take; i++) out[i] = (int32_t)r[i].id;
  qsort(out, (size_t)take, sizeof *out, cmp_i32);
  for (int32_t i = take; i < K; i++) out[i] = -1;
}

void csa2o_block_topk(const float *scores, int32_t n_q, int32_t width, const int32_t *q_nvis,
                      const int32_t *pool_blocks, int32_t block, int32_t M, int32_t K,
                      int32_t *pool_out, int32_t *topk_out) {
  int32_t *pool = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
  ranked_t *cand = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)(width > 0 ? width : 1));
  for (int32_t t = 0; t < n_q; t++) {
    const float *row = scores + (int64_t)t * width;
    int32_t nvis = q_nvis[t];
    int64_t nc = 0;
    if (!pool_blocks) {
      if (nvis > width) nvis = width; /* a row holds at most width scores */
      if (nvis < 0) nvis = 0;         /* a negative count sees nothing */
      /* g_r = max of block r over visible positions (padding = -inf) */
      int32_t nb = (nvis + block - 1) / block;
      ranked_t *g = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)(nb > 0 ? nb : 1));
      for (int32_t r = 0; r < nb; r++) {
        double mx = -INFINITY;
        for (int32_t o = 0; o < block; o++) {
          int32_t j = r * block + o;
          double v = (j < nvis) ? rank_key(row[j]) : -INFINITY;
          if (v > mx) mx = v;
        }
        g[r].key = mx;
        g[r].id = r;
      }
      if (nb > 0) g[nb - 1].key = INFINITY; /* the newest block always takes a slot */
      emit_sorted(g, nb, M, pool);
      free(g);
      if (pool_out) memcpy(pool_out + (int64_t)t * M, pool, sizeof(int32_t) * (size_t)M);
      /* pool = union of selected blocks, truncated to the visible width */
      for (int32_t s = 0; s < M; s++) {
        if (pool[s] < 0) continue;
        for (int32_t o = 0; o < block; o++) {
          int32_t j = pool[s] * block + o;
          if (j >= nvis) continue;
          cand[nc].key = rank_key(row[j]);
          cand[nc].id = j;
          nc++;
        }
      }
    } else {
      const int32_t *pb = pool_blocks + (int64_t)t * M;
      for (int32_t s = 0; s < M; s++) {
        if (pb[s] < 0) continue;
        for (int32_t o = 0; o < block; o++) {
          int64_t j = (int64_t)pb[s] * block + o;
          if (j >= nvis || s * block + o >= width) continue;
          cand[nc].key = rank_key(row[s * block + o]);
          cand[nc].id = j;
          nc++;
        }
      }
    }
    emit_sorted(cand, nc, K, topk_out + (int64_t)t * K);
  }
  free(cand);
  free(pool);
}

void csa2o_topk_bruteforce(const float *scores, int32_t n_q, int32_t width, const int32_t *q_nvis,
                           int32_t K, int32_t *topk_out) {
  ranked_t *cand = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)(width > 0 ? width : 1));
  for (int32_t t = 0; t < n_q; t++) {
    int32_t n = q_nvis[t] < width ? q_nvis[t] : width;
    if (n < 0) n = 0;
    for (int32_t j = 0; j < n; j++) {
      cand[j].key = rank_key(scores[(int64_t)t * width + j]);
      cand[j].id = j;
    }
    emit_sorted(cand, n, K, topk_out + (int64_t)t * K);
  }
  free(cand);
}

/* ------------------------------------------------------------------ HISA block means */

/* HISA's coarse filter ([ZB] §2.3.4, the HISA paragraphs): the prefix is cut into blocks of
 * consecutive positions and every block keeps the mean of its indexer keys, an auxiliary
 * for the search (the token keys stay).  The mean is taken over the exact dequantised keys
 * of the block's entries: an fp32 sum in ascending position order (what a running sum of a
 * decoding block holds), then one fp32 division by the entry count (a partial last block
 * divides by its own count).  It is stored in the indexer-K format (MXFP4, 68 bytes) by the
 * same rules as the indexer keys. */
static void pack_mxfp4_128(const float *x, uint8_t *o) {
  int codes[IDX_DIM];
  for (int g = 0; g < IDX_DIM / 32; g++) {
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
      float a = fabsf(x[32 * g + i]);
      if (a > amax) amax = a;
    }
    int sc = csa2o_e8m0_scale_code(amax);
    double X = csa2o_e8m0_value(sc);
    o[64 + g] = (uint8_t)sc;
    for (int i = 0; i < 32; i++) codes[32 * g + i] = csa2o_e2m1_encode(x[32 * g + i], X);
  }
  pack_nibbles(codes, IDX_DIM, o);
}

void csa2o_block_mean_pack(const uint8_t *idx_cache, int64_t n_entries, int32_t block, uint8_t *out) {
  double k[IDX_DIM];
  float sum[IDX_DIM], mean[IDX_DIM];
  const int64_t nb = (n_entries + block - 1) / block;
  for (int64_t b = 0; b < nb; b++) {
    const int64_t j0 = b * block;
    const int64_t j1 = (j0 + block < n_entries) ? j0 + block : n_entries;
    for (int64_t j = j0; j < j1; j++) {
      csa2o_dequant_idx(idx_cache + j * IDX_BYTES, k); /* exact in fp32 */
      for (int d = 0; d < IDX_DIM; d++) sum[d] = (j == j0) ? (float)k[d] : sum[d] + (float)k[d];
    }
    const float cnt = (float)(j1 - j0);
    for (int d = 0; d < IDX_DIM; d++) mean[d] = sum[d] / cnt;
    pack_mxfp4_128(mean, out + b * IDX_BYTES);
  }
}

/* The candidate pool from caller-given block scores (HISA: the scores of the block means):
 * the M blocks with the largest scores among the ceil(min(nvis, nbw*block)/block) visible
 * blocks, the newest visible block forced in as in the HSI pool ([ZB] §2.3.4 boundary
 * policy), ties to the lower block, NaN as -inf; ascending, padded with -1. */
void csa2o_pool_from_block_scores(const float *bscores, int32_t n_q, int32_t nbw, const int32_t *q_nvis,
                                  int32_t block, int32_t M, int32_t *pool_out) {
  ranked_t *g = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)(nbw > 0 ? nbw : 1));
  for (int32_t t = 0; t < n_q; t++) {
    int64_t nvis = q_nvis[t];
    if (nvis > (int64_t)nbw * block) nvis = (int64_t)nbw * block;
    if (nvis < 0) nvis = 0;
    const int32_t nb = (int32_t)((nvis + block - 1) / block);
    for (int32_t r = 0; r < nb; r++) {
      g[r].key = rank_key(bscores[(int64_t)t * nbw + r]);
      g[r].id = r;
    }
    if (nb > 0) g[nb - 1].key = INFINITY;
    emit_sorted(g, nb, M, pool_out + (int64_t)t * M);
  }
  free(g);
}

/* ------------------------------------------------------------------ stage 4 */

/* ------------------------------------------------------------------ FP8 window rows */

/* A window row in FP8 ([ZB] §2.4.4 and [SR] "FP4 Main KV Cache": the sliding-window KV
 * keeps FP8 precision; [ZB] §3.1 and [DF] §4.6 give DeepSeek-V4's FP8 KV entry as 448 FP8 NoPE
 * channels + 64 BF16 RoPE channels + 8 bytes of FP8 scales = 584 B, the layout taken
 * here): bytes [0, 448) E4M3 codes of channels 0..447, [448, 576) the BF16 bits of
 * channels 448..511, [576, 583) one E8M0 scale per 64 NoPE channels, byte 583 zero.
 * Scale: the OCP MX rule with E4M3's largest exponent (8), X = 2^(floor(log2 amax) - 8);
 * element: nearest-even E4M3 of x / X, saturating at 448, sign only on non-zero codes. */
int64_t csa2o_swa_fp8_row_bytes(void) { return D_NOPE + 2 * D_ROPE + 8; }

int csa2o_e8m0_scale_code_e4m3(float amax) {
  if (!(amax > 0.0f)) return 0;
  if (isinf(amax)) return 254; /* a group holding an infinity takes the largest finite scale */
  int ex;
  frexpf(amax, &ex); /* floor(log2 amax) = ex - 1 */
  int code = (ex - 1) - 8 + 127;
  if (code < 0) code = 0;
  if (code > 254) code = 254;
  return code;
}

void csa2o_swa_fp8_pack(const uint16_t *rows, int64_t n, uint8_t *out) {
  const int64_t rb = csa2o_swa_fp8_row_bytes();
  for (int64_t r = 0; r < n; r++) {
    const uint16_t *x = rows + r * D_LAT;
    uint8_t *o = out + r * rb;
    for (int g = 0; g < D_NOPE / 64; g++) {
      float amax = 0.0f;
      for (int c = 64 * g; c < 64 * g + 64; c++) {
        float a = fabsf(bf16_to_f32(x[c]));
        if (a > amax) amax = a;
      }
      const int code = csa2o_e8m0_scale_code_e4m3(amax);
      o[D_NOPE + 2 * D_ROPE + g] = (uint8_t)code;
      for (int c = 64 * g; c < 64 * g + 64; c++) {
        const double v = (double)bf16_to_f32(x[c]);
        const int e = csa2o_e4m3_encode(ldexp(fabs(v), 127 - code));
        o[c] = (uint8_t)((v < 0.0 && e != 0) ? (e | 0x80) : e);
      }
    }
    for (int c = D_NOPE; c < D_LAT; c++) {
      o[D_NOPE + 2 * (c - D_NOPE)] = (uint8_t)(x[c] & 0xFF);
      o[D_NOPE + 2 * (c - D_NOPE) + 1] = (uint8_t)(x[c] >> 8);
    }
    o[rb - 1] = 0;
  }
}

void csa2o_dequant_swa_fp8(const uint8_t *row, double *out) {
  for (int c = 0; c < D_NOPE; c++)
    out[c] = csa2o_e4m3_value(row[c]) * csa2o_e8m0_value(row[D_NOPE + 2 * D_ROPE + c / 64]);
  for (int c = D_NOPE; c < D_LAT; c++) {
    const uint16_t b = (uint16_t)(row[D_NOPE + 2 * (c - D_NOPE)] | (row[D_NOPE + 2 * (c - D_NOPE) + 1] << 8));
    out[c] = (double)bf16_to_f32(b);
  }
}

/* ------------------------------------------------------------------ stage 4 */

/* one window row into doubles: bf16 rows, or FP8 rows when swa8 != NULL */
typedef struct {
  const uint16_t *swa;
  const uint8_t *swa8;
  int64_t ring;
} window_src;

/* Window row r of a window that starts at row `start`.  Without a ring the rows are
 * consecutive.  With a ring of R rows the buffer is a sequence of rings (one per
 * sequence); the window stays inside the ring holding `start` and wraps at its end. */
static void window_row(const window_src *w, int64_t start, int32_t r, double *out) {
  int64_t row = start + r;
  if (w->ring > 0) {
    const int64_t seg = start - start % w->ring;
    row = seg + (start - seg + r) % w->ring;
  }
  if (w->swa8 != NULL) {
    csa2o_dequant_swa_fp8(w->swa8 + row * csa2o_swa_fp8_row_bytes(), out);
  } else {
    const uint16_t *r = w->swa + row * D_LAT;
    for (int d = 0; d < D_LAT; d++) out[d] = (double)bf16_to_f32(r[d]);
  }
}

static void sparse_attn_core(const uint16_t *q, const uint8_t *kv_cache, const int64_t *q_base,
                             const int32_t *topk, int32_t K, const window_src *win,
                             const int64_t *swa_start, const int32_t *swa_len, float scale,
                             float *out, float *lse, int32_t n_q) {
  int32_t cap = K + 128;
  double *keys = (double *)malloc(sizeof(double) * (size_t)cap * D_LAT);
  double *logit = (double *)malloc(sizeof(double) * (size_t)cap);
  double o[D_LAT];
  for (int32_t t = 0; t < n_q; t++) {
    /* gather: selected entries (dequantised exactly), then the window rows */
    int32_t nk = 0;
    for (int32_t i = 0; i < K; i++) {
      int32_t id = topk[(int64_t)t * K + i];
      if (id < 0) continue;
      csa2o_dequant_kv(kv_cache + (q_base[t] + id) * KV_BYTES, keys + (int64_t)nk * D_LAT);
      nk++;
    }
    int32_t nw = swa_len[t] < 128 ? swa_len[t] : 128;
    for (int32_t r = 0; r < nw; r++) {
      window_row(win, swa_start[t], r, keys + (int64_t)nk * D_LAT);
      nk++;
    }
    for (int h = 0; h < N_HEADS; h++) {
      const uint16_t *qh = q + ((int64_t)t * N_HEADS + h) * D_LAT;
      float *oh = out + ((int64_t)t * N_HEADS + h) * D_LAT;
      if (nk == 0) {
        for (int d = 0; d < D_LAT; d++) oh[d] = 0.0f;
        if (lse) lse[(int64_t)t * N_HEADS + h] = -INFINITY;
        continue;
      }
      double mx = -INFINITY;
      for (int32_t k = 0; k < nk; k++) {
        double dot = 0.0;
        for (int d = 0; d < D_LAT; d++) dot += (double)bf16_to_f32(qh[d]) * keys[(int64_t)k * D_LAT + d];
        logit[k] = (double)scale * dot;
        if (logit[k] > mx) mx = logit[k];
      }
      double z = 0.0;
      for (int d = 0; d < D_LAT; d++) o[d] = 0.0;
      for (int32_t k = 0; k < nk; k++) {
        double p = exp(logit[k] - mx);
        z += p;
        for (int d = 0; d < D_LAT; d++) o[d] += p * keys[(int64_t)k * D_LAT + d];
      }
      for (int d = 0; d < D_LAT; d++) oh[d] = (float)(o[d] / z);
      if (lse) lse[(int64_t)t * N_HEADS + h] = (float)(mx + log(z));
    }
  }
  free(logit);
  free(keys);
}

void csa2o_sparse_attn(const uint16_t *q, const uint8_t *kv_cache, const int64_t *q_base,
                       const int32_t *topk, int32_t K, const uint16_t *swa,
                       const int64_t *swa_start, const int32_t *swa_len, float scale,
                       float *out, float *lse, int32_t n_q) {
  const window_src w = {swa, NULL, 0};
  sparse_attn_core(q, kv_cache, q_base, topk, K, &w, swa_start, swa_len, scale, out, lse, n_q);
}

void csa2o_sparse_attn_swa_fp8(const uint16_t *q, const uint8_t *kv_cache, const int64_t *q_base,
                               const int32_t *topk, int32_t K, const uint8_t *swa8, int64_t swa_ring,
                               const int64_t *swa_start, const int32_t *swa_len, float scale,
                               float *out, float *lse, int32_t n_q) {
  const window_src w = {NULL, swa8, swa_ring};
  sparse_attn_core(q, kv_cache, q_base, topk, K, &w, swa_start, swa_len, scale, out, lse, n_q);
}
