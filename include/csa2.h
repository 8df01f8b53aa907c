/*
 * csa2.h -- C ABI of libcsa2.so: the CSA2 global-attention hot path with an FP4 KV
 * cache, as hand-written HIP kernels for MI355X (gfx950).
 *
 * Page abbreviations used in the citations:
 *   [ZB] zartbot.github.io   "DeepSeek-V4.1 Flash: 把 KV Cache 压缩推到极致"
 *   [DF] dilfish.github.io   "4. 层维度(下):CSA2 与每 token 890 字节"
 *   [SR] sarnas.ru           "DeepSeek-V4.1 Flash: как устроено сжатие KV-кэша"
 *
 * General contract
 *   - Tensor pointers are DEVICE pointers owned by the caller unless a parameter says
 *     "host".  Arrays are dense and row-major.  bf16 values travel as uint16 bit
 *     patterns.  The library never allocates, frees or synchronises device memory at run
 *     time.  Its global state: on each GPU, the fixed 32 MiB scratch array of
 *     csa2_block_topk_noalloc (a __device__ array that exists from library load to process
 *     end; only that call uses it); on the host, per-device caches of occupancy figures (how
 *     many workgroups of a kernel fit on the device) and of that array's device address,
 *     held in atomics and written with the same value by whichever call computes them
 *     first.  Calls on different streams and host threads are independent, except that
 *     overlapping csa2_block_topk_noalloc calls on one GPU share its array.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *     is asynchronous on it.  A kernel fault surfaces at the caller's next sync.
 *   - Return value: CSA2_OK (0) or a negative status.  Argument errors are detected on
 *     the host before anything is launched; CSA2_ERR_HIP reports a launch failure.
 *   - Fixed method constants (from the model table of [ZB] §1.2): latent width 512 =
 *     448 NoPE + 64 RoPE channels, 64 attention heads, 32 indexer heads x 128 dims,
 *     block 8, at most 2048 pool blocks, Top-K at most 512, window at most 128 rows,
 *     compression ratio m in {1, 2} ([DF] §4.2).
 *
 * Cache entry formats (bit-exact; [ZB] §2.4.4, [DF] §4.4 entry-size equation b(D,G))
 *   main KV  (288 B): bytes 0..255 hold 512 E2M1 codes, channel 2b in the low nibble
 *            of byte b (sign in the nibble's bit 3); bytes 256..287 hold one OCP E4M3
 *            scale per 16 channels.  Rows must be 16-byte aligned (288 = 18 x 16).
 *   indexer K (68 B per entry): 128 E2M1 codes in the same nibble order (64 payload
 *            bytes) and one E8M0 scale per 32 channels (MXFP4, 4 bytes).  The cache
 *            holds entries in tiles of 32 (2176 B per tile, tile t = entries 32t .. 32t +
 *            31): payload bytes 16p .. 16p + 15 of the tile's entry e (plane p = 0..3, the
 *            codes of channels 32p .. 32p + 31) at tile byte 512p + 16e, its 4 scale bytes
 *            at tile byte 2048 + 4e.  Entry j is thus at tile j / 32, slot j % 32, and a
 *            cache holding entries 0 .. n - 1 takes ceil(n / 32) x 2176 bytes.  A 68-byte
 *            record (the MXFP4 query of csa2_quantize_q_mxfp4) is the same entry as 64
 *            payload bytes in channel order followed by the 4 scale bytes.  The cache base
 *            must be 16-byte aligned.  HISA's block-mean cache uses the same layout.
 *   FP8 window row (584 B; the window KV kept in FP8, [ZB] §2.4.4, in DeepSeek-V4's FP8
 *            KV entry layout, [ZB] §3.1 and [DF] §4.6 equation 448 x 1 + 64 x 2 + 8):
 *            bytes 0..447 OCP E4M3 codes of channels 0..447; bytes 448..575 the bf16 bits
 *            of channels 448..511 (little-endian); bytes 576..582 one E8M0 scale per 64
 *            channels, X = 2^(floor(log2 amax) - 8) clamped to codes [0, 254] (the OCP MX
 *            rule with E4M3's largest exponent; 254 for a group holding an infinity);
 *            byte 583 zero.  Codes are nearest-even E4M3 of x / X saturating at 448
 *            (magnitudes in (448 X, 512 X) clip), the sign only on non-zero codes.  The
 *            buffer base must be 8-byte aligned (584 = 8 x 73).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer        */
  CSA2_ERR_UNSUPPORTED = -2, /* a method constant outside what the library builds */
  CSA2_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required         */
  CSA2_ERR_HIP = -4,         /* the HIP runtime reported an error at launch        */
  CSA2_ERR_SCRATCH = -5      /* larger than the fixed scratch array of a _noalloc call */
};

#define CSA2_ABI_VERSION 5

int csa2_abi_version(void);
const char *csa2_status_string(int status);

/*
 * csa2_rope_table -- HOST function: cos/sin table of the compressed-entry RoPE.
 *   For each position p = pos[j] and pair i = 0..31:
 *     out[j*64 + i] = (float)cos(p * theta^(-2i/64)), out[j*64 + 32 + i] = (float)sin(...)
 *   evaluated in double.  [ZB] §1.2 model table (compress_rope_theta = 160000),
 *   [ZB] §3.3.2 (RoPE acts on the rope tail only).
 *   pos: host [n]; out: host [n, 64].  Errors: CSA2_ERR_INVALID_ARG for NULL / n < 0.
 */
int csa2_rope_table(const int64_t *pos, int64_t n, double theta, float *out);

/*
 * csa2_compress_pack -- compressor + RoPE + FP4 pack + indexer-K projection + MXFP4.
 *   [DF] §4.2 compressor equation: entry j pools the m latents m*j .. m*j+m-1 with
 *   per-channel non-negative weights, c_j = sum_i a_i x_{mj+i}, a_i = w_i / sum(w)
 *   (m = 1: c_j = x_j, the per-token projection of [ZB] §3.3.2);
 *   [ZB] §2.4.4: RoPE on channels 448..511 (adjacent pairs (448+2i, 449+2i)) before
 *   quantisation, same FP4 format for NoPE and RoPE channels;
 *   [ZB] §2.3.1: indexer K is a projection of the main-KV entry: k = W_idx c~ over the
 *   512 rotated fp32 channels (one ascending fma chain per output);
 *   [DF] §4.4: main KV E2M1 + E4M3 per 16, indexer K MXFP4 (E2M1 + E8M0 per 32).
 *   Quantisation rules: E4M3 scale = nearest-even E4M3 of fp32(amax/6), saturating at
 *   448; element = E2M1 grid point nearest to |e|/S (exact, ties to the even code,
 *   saturating at 6), sign bit only on non-zero codes; E8M0 code = floor(log2 amax) - 2
 *   + 127 clamped to [0, 254] (0 when amax = 0).  The output bytes are bit-exact.
 *
 *   latent_bf16 [n_entries*m, 512]; pool_w fp32 (not read when m = 1; weights must be >= 0
 *   with a positive sum per channel, which is not checked): per_token_w = 0 -> static
 *   per-channel weights [m, 512] shared by every entry; per_token_w = 1 -> one weight row per
 *   latent token, [n_entries*m, 512], row m*j + i weighting latent m*j + i (per-token gates:
 *   [DF] §4.2 notes the pooling weights may be projected from the input; same formula);
 *   rope_cs fp32 [n_entries, 64] (cos[32], sin[32] at each entry's position, e.g. from
 *   csa2_rope_table); w_idx_bf16 [128, 512];
 *   kv_out [n_entries, 288] and idx_out (an indexer-K cache in the tile layout, room for
 *   entries 0 .. n_entries - 1: ceil(n_entries / 32) tiles) receive the packed entries.
 *   n_entries = 0 is a no-op.  Errors: INVALID_ARG (NULL, n < 0, misaligned outputs),
 *   UNSUPPORTED (m not 1 or 2); INVALID_ARG also for per_token_w not 0 or 1.
 */
int csa2_compress_pack(const uint16_t *latent_bf16, int64_t n_entries, int m,
                       const float *pool_w, int per_token_w, const float *rope_cs,
                       const uint16_t *w_idx_bf16, uint8_t *kv_out, uint8_t *idx_out, void *stream);

/*
 * csa2_compress_append -- csa2_compress_pack writing entry i to cache entry dst_rows[i]
 *   (main-KV row dst_rows[i]; indexer-K entry dst_rows[i] of the tile layout).
 *   [DF] §4.3: a Full layer writes its own main KV and indexer K; a decoding token at
 *   position p completes an entry of a ratio-m cache when p + 1 is a multiple of m, and
 *   the batch's new entries land at each sequence's next row, which need not be adjacent.
 *   Same arguments and results as csa2_compress_pack, with kv_out / idx_out replaced by
 *   the caches (16-byte aligned bases) and dst_rows: device int64 [n_entries] (8-byte
 *   aligned), the row of each entry; a negative row drops that entry.
 *   Errors: as csa2_compress_pack, and INVALID_ARG for a NULL dst_rows.
 */
int csa2_compress_append(const uint16_t *latent_bf16, int64_t n_entries, int m, const float *pool_w,
                         int per_token_w, const float *rope_cs, const uint16_t *w_idx_bf16,
                         const int64_t *dst_rows, uint8_t *kv_cache, uint8_t *idx_cache, void *stream);

/*
 * csa2_index_score -- lightning-indexer scores over the MXFP4 indexer-K cache.
 *   [ZB] §3.3.2 (indexer query q^I and per-head weights produce the Top-K set),
 *   [ZB] §2.3.4 / [DF] §4.7 (the Full layer scores every causally visible entry; a
 *   Reindex layer scores only its candidate pool):
 *     s(t, j) = sum_{h<32} head_w[t,h] * max(0, q_idx[t,h,:] . k^_j)
 *   with k^_j the exact dequantisation of entry j, bf16 products, fp32 accumulation.
 *
 *   q_idx_bf16 [n_q, 32, 128]; head_w fp32 [n_q, 32]; idx_cache: the indexer-K cache in
 *   the tile layout; q_base int64 [n_q]: cache entry of entry 0 of query t's sequence (a
 *   sequence need not start a tile; entries of other sequences in a shared tile are not
 *   read);
 *   q_nvis int32 [n_q]: visible entries of query t (entries 0 .. nvis-1);
 *   pool_blocks: NULL  -> Full mode: scores[t, j] for j < nvis, -inf for nvis <= j < width;
 *                [n_q, M] int32 block ids (-1 = empty) -> candidate mode: scores[t, 8s+o]
 *                is the score of entry 8*pool[s]+o, -inf when empty or j >= nvis;
 *                width must then equal 8*M.
 *   scores fp32 [n_q, width] (every element is written);
 *   block_max: NULL or fp32 [n_q, ceil(width/8)] (Full mode only): max of each block of
 *   8 scores, -inf padding ([ZB] §2.3.4 pad-and-amax).
 *   Errors: INVALID_ARG (NULL required pointer, n_q < 0, width < 0, width != 8*M in
 *   candidate mode, misaligned idx_cache), UNSUPPORTED (M > 2048).
 */
int csa2_index_score(const uint16_t *q_idx_bf16, const float *head_w, const uint8_t *idx_cache,
                     const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                     int32_t M, int32_t n_q, int32_t width, float *scores, float *block_max,
                     void *stream);

/*
 * csa2_quantize_q_mxfp4 -- packs indexer-query head vectors into MXFP4 records.
 *   [ZB] §2.4.4: DeepSeek-V4 trains the indexer Q and K for FP4; the format is OCP MXFP4,
 *   the indexer-K format above: each 128-channel head vector becomes 68 bytes (64 bytes
 *   of E2M1 codes, channel 2b in the low nibble of byte b; 4 E8M0 scales, one per 32
 *   channels) by the same rules as the indexer-K packer of csa2_compress_pack (E8M0 code
 *   floor(log2 amax) - 2 + 127 clamped to [0, 254], 0 for an all-zero group, 254 for a
 *   group holding an infinity; nearest-even E2M1 of x / X saturating at 6; NaN -> code 0).
 *   q_bf16 [n_vec, 128] (16-byte aligned); out [n_vec, 68] (4-byte aligned).  Bit-exact.
 *   For the indexer query n_vec = n_q * 32 and out is [n_q, 32, 68].
 *   Errors: INVALID_ARG (NULL, n_vec < 0, misalignment).
 */
int csa2_quantize_q_mxfp4(const uint16_t *q_bf16, int64_t n_vec, uint8_t *out, void *stream);

/*
 * csa2_index_score_fp4q -- csa2_index_score with the indexer query in MXFP4.
 *   [ZB] §2.4.4 (FP4 indexer Q and K): s(t, j) = sum_h head_w[t,h] max(0, q^_{t,h} . k^_j)
 *   with q^_{t,h} the dequantised 68-byte query record of head h (csa2_quantize_q_mxfp4)
 *   and k^_j as in csa2_index_score; products are exact, sums fp32.  The contraction runs
 *   on gfx950's block-scaled FP4 matrix instructions.
 *   q_fp4 [n_q, 32, 68] (4-byte aligned); every other argument, the modes, outputs and
 *   errors are those of csa2_index_score.
 */
int csa2_index_score_fp4q(const uint8_t *q_fp4, const float *head_w, const uint8_t *idx_cache,
                          const int64_t *q_base, const int32_t *q_nvis, const int32_t *pool_blocks,
                          int32_t M, int32_t n_q, int32_t width, float *scores, float *block_max,
                          void *stream);

/*
 * csa2_append_index_score -- a decode step's append and indexer scores in one launch:
 *   the result of csa2_compress_append of each query's newest entry followed by
 *   csa2_index_score in Full mode.
 *   [DF] §4.3 (a decoding token completes the newest entry of its sequence, and the Full
 *   layer then scores every visible entry, the newest included), [DF] §4.2 / §4.4 and
 *   [ZB] §2.3.1 / §2.4.4 (the entry, as in csa2_compress_pack), [ZB] §3.3.2 / §2.3.4 (the
 *   scores and block maxima, as in csa2_index_score).  Only the scores of the tile of 32
 *   slots holding the newest entry depend on the append; one workgroup per query packs the
 *   entry and then scores that tile, while the others score every other tile.
 *
 *   Query t appends one entry: latent_bf16 rows [t*m, t*m + m) (bf16 [n_q*m, 512],
 *   16-byte aligned), pool_w fp32 [m, 512] (per_token_w = 0) or [n_q*m, 512] with rows
 *   [t*m, t*m + m) weighting query t's latents (per_token_w = 1; neither is read when m = 1),
 *   rope_cs fp32 [n_q, 64]
 *   (the entry's cos[32], sin[32]), w_idx_bf16 [128, 512] (16-byte aligned), written to
 *   entry q_base[t] + q_nvis[t] - 1 of kv_cache [rows, 288] and of idx_cache (tile layout)
 *   (16-byte aligned bases); q_nvis[t] counts the new entry.  Queries must append to
 *   distinct rows.  A query with q_nvis[t] <= 0 appends nothing and gets an all -inf row.
 *   q_idx_bf16, head_w, q_base, q_nvis, width, scores and block_max are those of
 *   csa2_index_score in Full mode (no pool), with the same results bit for bit; the
 *   cache bytes are those of csa2_compress_append.  scores may be NULL when block_max is
 *   given: the block maxima alone are written, and csa2_block_topk_rescore selects from them
 *   by re-scoring the few entries it needs (no score row crosses HBM; at the 1M-context
 *   batch-4 decode this saves 0.9 us of the scan and costs about 2 us of selection).
 *   Errors: INVALID_ARG (NULL required pointer, n_q < 0, width <= 0 with n_q > 0,
 *   misalignment, per_token_w not 0 or 1), UNSUPPORTED (m not 1 or 2, n_q > 65535,
 *   width > 2^23).
 */
int csa2_append_index_score(const uint16_t *latent_bf16, int m, const float *pool_w, int per_token_w,
                            const float *rope_cs,
                            const uint16_t *w_idx_bf16, uint8_t *kv_cache, uint8_t *idx_cache,
                            const uint16_t *q_idx_bf16, const float *head_w, const int64_t *q_base,
                            const int32_t *q_nvis, int32_t n_q, int32_t width, float *scores,
                            float *block_max, void *stream);

/*
 * csa2_append_index_score_sel -- csa2_append_index_score (bf16 query) that also takes the
 *   first pass of the selection that follows it ([ZB] §2.3.4 / [DF] §4.7, csa2_block_topk in
 *   Full mode): the count of every query's older blocks (all blocks of its row but the one
 *   holding entry min(q_nvis[t], width) - 1) by the top 12 bits of their maximum's ranking
 *   key, added into the histogram region of a csa2_block_topk workspace, so that
 *   csa2_block_topk_prebuilt on the scores and maxima this call writes skips that pass.
 *   sel_workspace: the workspace of that selection call (csa2_block_topk_workspace(n_q,
 *   width, M, K) bytes, at least n_q * 16 KiB, 4-byte aligned) with its histogram region
 *   zero on entry, as every csa2_block_topk call leaves it; block_max is required (scores
 *   may be NULL, as above).  Every other argument, result and error as
 *   csa2_append_index_score; WORKSPACE when sel_ws_bytes < n_q * 16 KiB.
 */
int csa2_append_index_score_sel(const uint16_t *latent_bf16, int m, const float *pool_w, int per_token_w,
                                const float *rope_cs, const uint16_t *w_idx_bf16, uint8_t *kv_cache,
                                uint8_t *idx_cache, const uint16_t *q_idx_bf16, const float *head_w,
                                const int64_t *q_base, const int32_t *q_nvis, int32_t n_q, int32_t width,
                                float *scores, float *block_max, void *sel_workspace, size_t sel_ws_bytes,
                                void *stream);

/*
 * csa2_append_index_score_fp4q -- csa2_append_index_score with the indexer query in MXFP4
 *   (q_fp4 [n_q, 32, 68], 4-byte aligned, from csa2_quantize_q_mxfp4): the scores of
 *   csa2_index_score_fp4q.  Every other argument, result and error as above, except that
 *   scores is required.
 */
int csa2_append_index_score_fp4q(const uint16_t *latent_bf16, int m, const float *pool_w, int per_token_w,
                                 const float *rope_cs, const uint16_t *w_idx_bf16, uint8_t *kv_cache,
                                 uint8_t *idx_cache, const uint8_t *q_fp4, const float *head_w,
                                 const int64_t *q_base, const int32_t *q_nvis, int32_t n_q, int32_t width,
                                 float *scores, float *block_max, void *stream);

/*
 * csa2_append_index_score_packq -- csa2_append_index_score_fp4q with the indexer query
 *   packed inside the launch: the result of csa2_quantize_q_mxfp4 of q_idx_bf16 followed by
 *   csa2_append_index_score_fp4q, bit for bit ([ZB] §2.4.4, the FP4 indexer query).  Each
 *   workgroup packs its query's 32 head vectors into its own LDS; the packed records are
 *   not written out.  Arguments, results and errors are those of csa2_append_index_score
 *   (q_idx_bf16 [n_q, 32, 128], 16-byte aligned).
 */
int csa2_append_index_score_packq(const uint16_t *latent_bf16, int m, const float *pool_w, int per_token_w,
                                  const float *rope_cs,
                                  const uint16_t *w_idx_bf16, uint8_t *kv_cache, uint8_t *idx_cache,
                                  const uint16_t *q_idx_bf16, const float *head_w, const int64_t *q_base,
                                  const int32_t *q_nvis, int32_t n_q, int32_t width, float *scores,
                                  float *block_max, void *stream);

/*
 * csa2_block_topk -- hierarchical selection: block max -> top-M block pool -> Top-K.
 *   [ZB] §2.3.4 and [DF] §4.7: g_r = max over block r (b = `block` positions, -inf
 *   padding); the block holding the newest visible position takes +inf; the M blocks
 *   with the largest g_r form the pool P_t (|P_t| <= 8M); a layer's Top-K is taken
 *   inside the pool.  Ties go to the lower block / entry index; NaN ranks as -inf.
 *   Full mode (pool_blocks == NULL): scores [n_q, width] from csa2_index_score Full
 *   mode; block_max may be NULL (recomputed) or the array index_score wrote.  The
 *   visible count is min(q_nvis[t], width).  pool_out: NULL or [n_q, M] selected block
 *   ids ascending, -1 padded.  The Top-K inside the pool equals the Top-K of the whole
 *   row (an entry outside the pool is outranked by the maxima of the M-1 older blocks
 *   above its block), which is how it is computed.
 *   Candidate mode (pool_blocks != NULL, [n_q, M]): scores [n_q, width = 8M] laid out as
 *   csa2_index_score candidate mode; pool_out must be NULL.
 *   topk_out [n_q, K]: selected entry ids (relative to the sequence) ascending, -1 pad.
 *   workspace: device scratch of at least csa2_block_topk_workspace(n_q, width, M, K)
 *   bytes, 4-byte aligned.  Its histogram region, the first n_q * 16 KiB, must be all zero
 *   before the call (allocate the buffer zero-filled); every call that completes leaves that
 *   region zero again, so one buffer can be reused by consecutive calls on the same stream
 *   with the same or a smaller n_q (a larger n_q needs its larger region zeroed again).
 *   Calls that overlap in time must not share a workspace.
 *   Errors: INVALID_ARG, UNSUPPORTED (block != 8, M > 2048, K > 512, K < 1, M < 1, rows
 *   longer than 2^20 blocks, Full mode with a Top-K and M - 1 < K: the Top-K is computed as
 *   the row's global Top-K, which equals the Top-K inside the pool only when the maxima of
 *   the M - 1 older pool blocks outrank every entry outside it), WORKSPACE (workspace
 *   missing or too small).
 */
size_t csa2_block_topk_workspace(int32_t n_q, int32_t width, int32_t M, int32_t K);
/*   Pool-only mode (topk_out == NULL, Full mode): the pool alone, built from the caller's
 *   block scores in block_max ([n_q, ceil(width/8)], required) by the same rules (top M-1
 *   older blocks plus the forced newest block); scores may be NULL; K must still be in
 *   range.  HISA's coarse filter uses it with the scores of its block means. */
int csa2_block_topk(const float *scores, const float *block_max, int32_t n_q, int32_t width,
                    const int32_t *q_nvis, const int32_t *pool_blocks, int32_t block,
                    int32_t M, int32_t K, int32_t *pool_out, int32_t *topk_out,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * csa2_block_topk_prebuilt -- csa2_block_topk in Full mode (pool_blocks NULL, block_max
 *   required) whose workspace's histogram region already holds the counts of its first pass,
 *   added by csa2_append_index_score_sel for these block maxima and visible counts: the call
 *   skips that pass.  Results bit for bit those of csa2_block_topk; it leaves the histogram
 *   region zero, as csa2_block_topk does.  Arguments and errors as csa2_block_topk.
 */
int csa2_block_topk_prebuilt(const float *scores, const float *block_max, int32_t n_q, int32_t width,
                             const int32_t *q_nvis, int32_t block, int32_t M, int32_t K, int32_t *pool_out,
                             int32_t *topk_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * csa2_block_topk_rescore -- csa2_block_topk in Full mode without a score row: the
 *   selection of [ZB] §2.3.4 / [DF] §4.7 over the scores s(t, j) of [ZB] §3.3.2, from the
 *   block maxima that csa2_append_index_score (scores = NULL) or csa2_index_score wrote.
 *   The pool needs only the maxima; the Top-K needs the scores of the entries of the
 *   candidate blocks (those whose maximum reaches the histogram bin of the K-th largest
 *   older-block maximum, and the newest block), and these few are computed again from
 *   the indexer cache with the scan's own tile arithmetic, bit for bit the scores
 *   csa2_index_score would have written.  Results: those of csa2_block_topk given that
 *   score row, bit for bit.
 *   block_max fp32 [n_q, ceil(width/8)] (4-byte aligned); q_nvis, width as csa2_block_topk;
 *   q_idx_bf16 [n_q, 32, 128] (16-byte aligned), head_w fp32 [n_q, 32], idx_cache (tile
 *   layout, 16-byte aligned) and q_base [n_q]: the scan's inputs (query t's entry j is
 *   cache entry q_base[t] + j); M, K, pool_out (NULL: no pool), topk_out (required) as
 *   csa2_block_topk.  workspace: csa2_block_topk_rescore_workspace(n_q, width, M, K) bytes,
 *   4-byte aligned, histogram region zero before the first call and left zero by every
 *   call, as csa2_block_topk's (a 1M-context batch of 4 needs 21 MB: each K2 workgroup's
 *   list segment holds every entry of its slice, so no list overflows).
 *   Errors: INVALID_ARG (NULL required pointer, misalignment), UNSUPPORTED (M, K out of
 *   range or M - 1 < K, width > 2^23, n_q > 65535), WORKSPACE.
 */
size_t csa2_block_topk_rescore_workspace(int32_t n_q, int32_t width, int32_t M, int32_t K);
int csa2_block_topk_rescore(const float *block_max, int32_t n_q, int32_t width, const int32_t *q_nvis,
                            const uint16_t *q_idx_bf16, const float *head_w, const uint8_t *idx_cache,
                            const int64_t *q_base, int32_t M, int32_t K, int32_t *pool_out, int32_t *topk_out,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * csa2_block_topk_noalloc -- csa2_block_topk that allocates nothing and takes no workspace,
 *   for callers that cannot allocate device memory: code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc.  The workspace is a fixed device array
 *   of CSA2_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the process
 *   ends); each call first clears its histogram region with a kernel (no memset), so the
 *   call may be captured.  Every call on one GPU shares that GPU's array: calls that overlap
 *   in time on one GPU (other streams, other host threads) race and must not be issued.
 *   Arguments, modes, results and errors are those of csa2_block_topk without workspace and
 *   ws_bytes, plus CSA2_ERR_SCRATCH when csa2_block_topk_workspace(n_q, width, M, K)
 *   exceeds CSA2_NOALLOC_SCRATCH_BYTES (e.g. 4 rows of 2^20 entries fit; 4096 prefill rows
 *   of 34816 do not), and CSA2_ERR_HIP if the array's device address cannot be obtained.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa2_block_topk_noalloc(const float *scores, const float *block_max, int32_t n_q, int32_t width,
                            const int32_t *q_nvis, const int32_t *pool_blocks, int32_t block, int32_t M,
                            int32_t K, int32_t *pool_out, int32_t *topk_out, void *stream);

/*
 * csa2_block_mean_pack -- HISA's block-mean indexer keys.
 *   [ZB] §2.3.4 (the HISA paragraphs): the prefix is cut into blocks of consecutive
 *   entries; every block keeps the mean of its indexer keys as an auxiliary for the search,
 *   updated for the newest block only while decoding; the block means are scored with the
 *   same indexer query and head weights and the best blocks expanded for token-level
 *   scoring.  Record b of sequence s, for the entries e = 8b .. min(8b + 8, n_s) - 1 at cache
 *   entries seq_base[s] + e: the fp32 sum of their exact dequantised keys in ascending order,
 *   divided once (IEEE) by their count, packed in the indexer-K format (68 B, MXFP4 rules
 *   of csa2_compress_pack).  Bit-exact.
 *   idx_cache: the indexer-K cache (tile layout, 4-byte aligned); seq_base int64 [n_seq],
 *   seq_n int32 [n_seq]
 *   (entries of sequence s); first_block: NULL (0) or int32 [n_seq]; the call writes blocks
 *   first_block[s] .. first_block[s] + n_blocks - 1 that hold at least one entry, to
 *   entries mean_base[s] + b of mean_cache (int64 [n_seq]; mean_cache in the tile layout,
 *   4-byte aligned).  A decode
 *   step passes first_block = (n_s - 1) / 8 and n_blocks = 1.  Scoring the block means is
 *   csa2_index_score over mean_cache with q_nvis = ceil(n / 8); the pool is csa2_block_topk's
 *   pool-only mode on those scores; the final Top-K is candidate mode inside it.
 *   Errors: INVALID_ARG (NULL, negative counts, misalignment), UNSUPPORTED (n_seq > 65535).
 */
int csa2_block_mean_pack(const uint8_t *idx_cache, const int64_t *seq_base, const int32_t *seq_n,
                         const int32_t *first_block, int32_t n_seq, int32_t n_blocks,
                         uint8_t *mean_cache, const int64_t *mean_base, void *stream);

/*
 * csa2_append_mean_index_score -- HISA's decode step in one launch: the result of
 *   csa2_compress_append of each query's newest entry, then csa2_block_mean_pack of the
 *   block holding it, then csa2_index_score (Full mode) over the block means.
 *   [ZB] §2.3.4 (the HISA paragraphs: block-mean keys, the newest block's mean updated while
 *   decoding, the block means scored with the indexer query and head weights), [DF] §4.3
 *   (a decoding token completes the newest entry of its sequence).  Only the newest block's
 *   record, and so only the scores of the tile of 32 block means holding it, depend on the
 *   append: one workgroup per query packs the entry, re-packs that block's record (its
 *   older entries from idx_cache, the new one as just packed) and scores that tile, while
 *   the others score every other tile of block means.
 *
 *   The appended entry (latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache,
 *   idx_cache, q_base, q_nvis) is that of csa2_append_index_score: entry q_base[t] + q_nvis[t] - 1,
 *   with q_nvis[t] counting it.  Block b of query t covers its entries 8b .. 8b + 7 (cache
 *   entries q_base[t] + 8b ..); its record is entry mean_base[t] + b of mean_cache (int64
 *   [n_q]; mean_cache in the tile layout, 16-byte aligned), and the call rewrites that of block
 *   (q_nvis[t] - 1) / 8 by the rules of csa2_block_mean_pack.  The scores are those of
 *   csa2_index_score over mean_cache with q_base = mean_base and ceil(q_nvis[t] / 8)
 *   visible rows: scores fp32 [n_q, width] and block_max (NULL, or fp32 [n_q,
 *   ceil(width / 8)]), bit for bit.  A query with q_nvis[t] <= 0 writes nothing and gets an
 *   all -inf row.  Queries must append to distinct rows and own distinct mean rows.
 *   Errors: those of csa2_append_index_score, and INVALID_ARG for a NULL or misaligned
 *   mean_cache or a NULL mean_base.
 */
int csa2_append_mean_index_score(const uint16_t *latent_bf16, int m, const float *pool_w, int per_token_w,
                                 const float *rope_cs,
                                 const uint16_t *w_idx_bf16, uint8_t *kv_cache, uint8_t *idx_cache,
                                 uint8_t *mean_cache, const int64_t *mean_base, const uint16_t *q_idx_bf16,
                                 const float *head_w, const int64_t *q_base, const int32_t *q_nvis, int32_t n_q,
                                 int32_t width, float *scores, float *block_max, void *stream);

/*
 * csa2_append_mean_index_score_fp4q -- csa2_append_mean_index_score with the indexer query
 *   in MXFP4 (q_fp4 [n_q, 32, 68], 4-byte aligned): the scores of csa2_index_score_fp4q.
 *   Every other argument, result and error as above.
 */
int csa2_append_mean_index_score_fp4q(const uint16_t *latent_bf16, int m, const float *pool_w,
                                      int per_token_w, const float *rope_cs, const uint16_t *w_idx_bf16, uint8_t *kv_cache,
                                      uint8_t *idx_cache, uint8_t *mean_cache, const int64_t *mean_base,
                                      const uint8_t *q_fp4, const float *head_w, const int64_t *q_base,
                                      const int32_t *q_nvis, int32_t n_q, int32_t width, float *scores,
                                      float *block_max, void *stream);

/*
 * csa2_sparse_attn -- sparse latent attention over the selected FP4 entries joined with
 *   the sliding window.  [ZB] §3.3.2.1: key = value = c (the 512-channel entry); one
 *   softmax per head over the selected entries and the window rows ([ZB] §3.3.2, joint
 *   sparse attention with the SWA KV):
 *     o_h = sum_k p_k key_k,  p = softmax(scale * q_h . key_k)
 *   q_bf16 [n_q, 64, 512] (RoPE already applied); kv_cache flat [rows, 288];
 *   q_base int64 [n_q]; topk int32 [n_q, K] (entry ids relative to q_base, -1 = unused);
 *   swa_bf16 [rows, 512]; swa_start int64 [n_q]: first window row of query t;
 *   swa_len int32 [n_q]: window rows of query t (clamped to [0, 128]);
 *   scale: logit scale (1/sqrt(512) is the library's documented default reading);
 *   out fp32 [n_q, 64, 512]; lse: NULL or fp32 [n_q, 64], natural-log partition
 *   function (max logit + log sum exp); a query with no keys gets out = 0, lse = -inf.
 *   Numerics: every key value is exact in bf16 (E2M1 x E4M3, FP8 window values, bf16 rows)
 *   and q is used as given, so the logits' products are exact for inputs of any finite
 *   magnitude, summed in fp32; the probabilities enter the value sum as two bf16 parts
 *   (about 2^-17 relative), accumulated in fp32.
 *   workspace: csa2_sparse_attn_workspace(n_q, K) bytes, 16-byte aligned, caller-owned,
 *   contents on entry ignored (may be NULL when that size is 0).  Small batches split each
 *   query's keys over several workgroups whose partial sums land here before a merge; large
 *   batches need none.  Pointers q_bf16, kv_cache, swa_bf16 and out are 16-byte aligned.
 *   Errors: INVALID_ARG, UNSUPPORTED (K > 512), WORKSPACE.
 */
size_t csa2_sparse_attn_workspace(int32_t n_q, int32_t K);
int csa2_sparse_attn(const uint16_t *q_bf16, const uint8_t *kv_cache, const int64_t *q_base,
                     const int32_t *topk, int32_t K, const uint16_t *swa_bf16,
                     const int64_t *swa_start, const int32_t *swa_len, float scale, float *out,
                     float *lse, int32_t n_q, void *workspace, size_t ws_bytes, void *stream);

/*
 * csa2_swa_pack_fp8 -- packs bf16 window rows into FP8 window rows (format above).
 *   [ZB] §2.4.4: the sliding-window KV stays FP8 while the compressed entries go FP4.
 *   rows_bf16 [n, 512] (16-byte aligned); dst_rows: NULL (row r goes to out row r) or
 *   int64 [n], the out row of row r (negative: row r is skipped), so a decode step can
 *   append its new tokens at their ring slots; out: FP8 rows, 8-byte aligned, large
 *   enough for every destination row.  Bit-exact: the codes do not depend on rounding
 *   order.  Errors: INVALID_ARG (null pointer, n < 0, misalignment).
 */
int csa2_swa_pack_fp8(const uint16_t *rows_bf16, int64_t n, const int64_t *dst_rows, uint8_t *out,
                      void *stream);

/*
 * csa2_sparse_attn_swa_fp8 -- csa2_sparse_attn with the window read from FP8 window rows.
 *   Same computation and arguments as csa2_sparse_attn, the window rows being the
 *   dequantised FP8 rows (value = E4M3 code x 2^(scale code - 127); RoPE channels as
 *   stored).  swa8: FP8 window rows (8-byte aligned).  swa_ring: 0 = window row r of query
 *   t is swa_start[t] + r; R >= 128 = the buffer is a sequence of rings of R rows (one per
 *   sequence) and the window wraps inside the ring that holds swa_start[t]:
 *     row = s + (swa_start[t] - s + r) mod R,  s = swa_start[t] - swa_start[t] mod R.
 *   The FP8 window values decode exactly into bf16 (4 significant bits times a power of two).
 *   Errors: INVALID_ARG (also 0 < swa_ring < 128), UNSUPPORTED (K > 512), WORKSPACE.
 */
int csa2_sparse_attn_swa_fp8(const uint16_t *q_bf16, const uint8_t *kv_cache, const int64_t *q_base,
                             const int32_t *topk, int32_t K, const uint8_t *swa8, int64_t swa_ring,
                             const int64_t *swa_start, const int32_t *swa_len, float scale,
                             float *out, float *lse, int32_t n_q, void *workspace, size_t ws_bytes,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
