/*
 * csa2_oracle.h -- plain, single-threaded CPU oracle for the CSA2 global-branch
 * hot path (compress + FP4 pack, lightning-indexer scoring, hierarchical block
 * Top-K, sparse latent attention with the sliding window).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the test-suite, the smoke entry point and the bench's
 * CPU-baseline leg use it.  It shares no source with the HIP library.
 *
 * Page abbreviations used in every citation below:
 *   [ZB] zartbot.github.io  "DeepSeek-V4.1 Flash: 把 KV Cache 压缩推到极致"
 *   [DF] dilfish.github.io  "4. 层维度(下):CSA2 与每 token 890 字节"
 *   [SR] sarnas.ru          "DeepSeek-V4.1 Flash: как устроено сжатие KV-кэша"
 *   [SW] s1mplewind.github.io "deepseek-v4.1-技术报告学习"
 *
 * Conventions (all arrays are host memory, row-major, owned by the caller):
 *   bf16 values are passed as their raw uint16 bit patterns.
 *   Main-KV entry: 288 bytes = 256 payload bytes (512 E2M1 nibbles, channel
 *   2b in the low nibble of byte b) + 32 E4M3 scale bytes (one per 16 channels).
 *   Indexer-K entry: 68 bytes = 64 payload bytes (same nibble order) + 4 E8M0
 *   scale bytes (one per 32 channels).
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- sizes: [DF] §4.4, entry-size equation b(D,G) = D/2 + D/G ---------------- */
int64_t csa2o_entry_bytes(int64_t D, int64_t G);

/* ---- scalar formats ([ZB] §2.4.4, [DF] §4.4/§4.5) ------------------------------ */
double csa2o_e2m1_value(int code4);          /* 4-bit code: sign bit 3, magnitude 0..7 */
double csa2o_e4m3_value(int byte);           /* OCP E4M3FN; 0x7F/0xFF -> NaN            */
double csa2o_e8m0_value(int byte);           /* 2^(byte-127); 255 -> NaN                */
int    csa2o_e4m3_encode(double x);          /* x >= 0: nearest, ties to even, sat. 448 */
int    csa2o_e2m1_encode(float e, double S); /* nearest of |e| on {0..6}*S, ties even   */
int    csa2o_e8m0_scale_code(float amax);    /* MX rule: floor(log2 amax) - 2 + 127     */

/* ---- RoPE table: cos then sin of pos * theta^(-2i/64), i = 0..31, out[n, 64] ---- */
void csa2o_rope_table(const int64_t *pos, int64_t n, double theta, float *out);

/* ---- stage 1: compressor + RoPE + FP4 pack + indexer-K projection + MXFP4 pack --
 * latent   : bf16 [n_entries * m, 512] (complete groups only)
 * pool_w   : fp32 non-negative weights (unused when m == 1): [m, 512] per channel, or with
 *            per_token_w != 0 one row per latent token, [n_entries * m, 512]
 * rope_cs  : fp32 [n_entries, 64] (cos[32], sin[32]) at each entry's position
 * w_idx    : bf16 [128, 512] indexer-K projection
 * kv_out   : [n_entries, 288]; idx_out : [n_entries, 68]
 * pooled/rotated/kproj (each may be NULL): fp32 intermediates [n, 512] / [n, 512] / [n, 128]. */
void csa2o_compress_pack(const uint16_t *latent, int64_t n_entries, int m,
                         const float *pool_w, int per_token_w, const float *rope_cs, const uint16_t *w_idx,
                         uint8_t *kv_out, uint8_t *idx_out,
                         float *pooled, float *rotated, float *kproj);

/* exact dequantisation of one entry into doubles */
void csa2o_dequant_kv(const uint8_t *entry288, double *out512);
void csa2o_dequant_idx(const uint8_t *entry68, double *out128);

/* ---- stage 2: lightning-indexer scores ------------------------------------------
 * s(t, j) = sum_h w[t,h] * max(0, q[t,h,:] . k_j), double accumulation, stored fp32.
 * q_idx [n_q, 32, 128] bf16; head_w [n_q, 32]; idx_cache flat [*, 68];
 * entry j of query t lives at row q_base[t] + j; j < q_nvis[t] is visible.
 * pool_blocks == NULL: scores[t, j] for j < nvis, -inf elsewhere (row stride width).
 * else pool_blocks [n_q, M] (block ids, -1 pad): scores[t, 8*slot + o] is the score
 * of entry 8*pool[slot] + o, -inf when the slot is empty or the entry not visible. */
void csa2o_index_score(const uint16_t *q_idx, const float *head_w, const uint8_t *idx_cache,
                       const int64_t *q_base, const int32_t *q_nvis,
                       const int32_t *pool_blocks, int32_t M, int32_t n_q, int32_t width,
                       float *scores);

/* ---- stage 3: block max -> top-M block pool -> Top-K -----------------------------
 * Full mode (pool_blocks == NULL): pool over all visible blocks, newest block +inf,
 * Top-K among pool positions.  pool_out may be NULL.
 * Candidate mode (pool_blocks != NULL): Top-K among the pool positions of scores
 * laid out as in csa2o_index_score.  Outputs ascending, padded with -1. */
void csa2o_block_topk(const float *scores, int32_t n_q, int32_t width, const int32_t *q_nvis,
                      const int32_t *pool_blocks, int32_t block, int32_t M, int32_t K,
                      int32_t *pool_out, int32_t *topk_out);

/* brute-force Top-K over the visible row, no pool (for the equivalence pin) */
void csa2o_topk_bruteforce(const float *scores, int32_t n_q, int32_t width, const int32_t *q_nvis,
                           int32_t K, int32_t *topk_out);

/* ---- stage 4: sparse latent attention joined with the sliding window -------------
 * q [n_q, 64, 512] bf16; keys = values = dequantised entries q_base[t] + topk[t, i]
 * (i < K, skipping -1) followed by swa rows swa_start[t] .. + swa_len[t] - 1.
 * out [n_q, 64, 512] fp32; lse (may be NULL) [n_q, 64] natural-log partition. */
void csa2o_sparse_attn(const uint16_t *q, const uint8_t *kv_cache, const int64_t *q_base,
                       const int32_t *topk, int32_t K, const uint16_t *swa,
                       const int64_t *swa_start, const int32_t *swa_len, float scale,
                       float *out, float *lse, int32_t n_q);

/* ---- FP4 indexer query ([ZB] §2.4.4: FP4 indexer Q and K; OCP MXFP4) ---------------
 * q head vectors packed exactly like indexer-K entries (68 B: 64 B of E2M1 codes, 4 E8M0
 * scales); the score is stage 2's with q_h dequantised. */
void csa2o_quantize_q_mxfp4(const uint16_t *q_bf16, int64_t n_vec, uint8_t *out68);
void csa2o_index_score_fp4q(const uint8_t *q_fp4, const float *head_w, const uint8_t *idx_cache,
                            const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                            int32_t M, int32_t n_q, int32_t width, float *scores);

/* ---- HISA block-mean keys ([ZB] §2.3.4, HISA: block means of the indexer keys as a search
 * auxiliary; block-level coarse scoring, then token-level scoring of the expanded blocks) --
 * out[b] (68 B, indexer-K format) = MXFP4 of (fp32 ascending sum of the exact dequantised
 * keys of entries b*block .. min(b*block+block, n)-1) / count, for b < ceil(n / block). */
void csa2o_block_mean_pack(const uint8_t *idx_cache, int64_t n_entries, int32_t block, uint8_t *out);
/* pool = top-M of bscores [n_q, nbw] over the visible blocks, newest visible block forced in,
 * ties to the lower block, NaN as -inf; ascending, -1 padded (pool_out [n_q, M]). */
void csa2o_pool_from_block_scores(const float *bscores, int32_t n_q, int32_t nbw, const int32_t *q_nvis,
                                  int32_t block, int32_t M, int32_t *pool_out);

/* ---- FP8 window rows (the sliding-window KV kept in FP8: [ZB] §2.4.4, [SR] "FP4 Main
 * KV Cache"; the 584-byte FP8 KV entry of [ZB] §3.1 and [DF] §4.6) ------------------------
 * row: [0,448) E4M3 codes of channels 0..447 | [448,576) BF16 bits of channels 448..511 |
 * [576,583) E8M0 scale per 64 NoPE channels | byte 583 = 0.
 * Scale X = 2^(floor(log2 amax) - 8) (OCP MX rule, E4M3 emax 8); codes nearest-even of
 * x / X, saturating at 448, sign only on non-zero codes. */
int64_t csa2o_swa_fp8_row_bytes(void);
int csa2o_e8m0_scale_code_e4m3(float amax);
void csa2o_swa_fp8_pack(const uint16_t *rows_bf16, int64_t n, uint8_t *out);
void csa2o_dequant_swa_fp8(const uint8_t *row, double *out512);
/* stage 4 with an FP8 window cache: window row r of query t is swa_start[t] + r when
 * swa_ring == 0; when swa_ring = R > 0 the buffer is a sequence of rings of R rows (one per
 * sequence) and the window wraps inside the ring that holds row swa_start[t]:
 * row = s + (swa_start[t] - s + r) mod R with s = swa_start[t] - swa_start[t] mod R. */
void csa2o_sparse_attn_swa_fp8(const uint16_t *q, const uint8_t *kv_cache, const int64_t *q_base,
                               const int32_t *topk, int32_t K, const uint8_t *swa8, int64_t swa_ring,
                               const int64_t *swa_start, const int32_t *swa_len, float scale,
                               float *out, float *lse, int32_t n_q);

#ifdef __cplusplus
}
#endif
#endif
