// append_index.hip -- a decode step's append and its indexer scores in one launch (gfx950).
//
// A decoding step appends each sequence's newest entry (pooling, RoPE and both FP4 packs:
// [DF] "CSA2 与每 token 890 字节" §4.2 and §4.4, [ZB] "把 KV Cache 压缩推到极致" §2.3.1 and
// §2.4.4) and then scores every visible entry for the step's query ([ZB] §3.3.2, §2.3.4; [DF]
// §4.7).  Only the scores of the tile of 32 slots holding the new entry depend on it, so one
// launch does both:
//   - one workgroup per query t compresses the newest entry of t's sequence into row
//     q_base[t] + q_nvis[t] - 1 (compress_entry_lds / compress_entry_wg of compress_few.hpp),
//     then scores that tile, taking the new entry's indexer row from its own LDS
//     (index_tiles.hpp, kNewestSlots);
//   - the other workgroups score every other tile of t's row and read none of that tile's
//     entries (kOlderSlots).
// The bf16-query launch uses workgroups of 12 waves that fill a CU each
// (append_index_wide_kernel); the MXFP4-query and HISA launches use 4-wave workgroups, the
// append workgroup being x = 0 of row t.
// No workgroup reads what another writes, so there is no cross-workgroup synchronisation
// (a device-scope fence here costs a write-back of the L2 while the scan streams).  The
// bytes and scores are those of csa2_compress_append followed by csa2_index_score: the
// append's latency chain (the 512-step projection) runs beside the scan instead of before it.
//
// HISA's decode step ([ZB] §2.3.4, the HISA paragraphs) scores block means instead of
// entries, and the only mean the new entry changes is that of its own block.  Its launch
// has the same shape: workgroup 0 of query t appends the entry, re-packs the mean record
// of the newest block (the block's older entries from the cache, the new one from LDS,
// block_mean.hpp) and scores the tile of block means that holds it, taking that record
// from LDS; the other workgroups score every other tile of block means.
#include "block_mean.hpp"
#include "compress_few.hpp"
#include "index_tiles.hpp"

namespace csa2 {
namespace {
using namespace idx;

constexpr int kAppendWgs = 1;  // append workgroups per query

// The MXFP4-query launch (the bf16 one is append_index_wide_kernel below).
template <bool kFp4Q, bool kScores = true>
__global__ __launch_bounds__(kThreads) void append_index_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ idx_cache,
    const void* __restrict__ q_in, const float* __restrict__ head_w, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, int32_t width, float* __restrict__ scores, float* __restrict__ block_max,
    int64_t w_stride) {
  const int t = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (blockIdx.x >= kAppendWgs) {
    score_tiles<false, kFp4Q, kOlderSlots, false, kScores>(q_in, head_w, idx_cache, q_base, q_nvis, nullptr, 0, width,
                                                           scores, block_max, t,
                                                           (int32_t)(blockIdx.x - kAppendWgs) * kWaves + wave,
                                                           (int32_t)(gridDim.x - kAppendWgs) * kWaves);
    return;
  }
  __shared__ EntryShared sh;
  const int32_t nvis = q_nvis[t];
  const int64_t row = nvis > 0 ? q_base[t] + nvis - 1 : -1;  // nothing visible: nothing appended
  compress_entry_wg(latent + (int64_t)t * m * kD, m, pool_w + t * w_stride, rope_cs + (int64_t)t * kDRope, w_idx, row, kv_cache,
                    idx_cache, sh);
  score_tiles<false, kFp4Q, kNewestSlots, false, kScores>(q_in, head_w, idx_cache, q_base, q_nvis, nullptr, 0, width,
                                                          scores, block_max, t, wave, kWaves, sh.idx_row);
}

// The bf16-query launch in workgroups of 12 waves, which fill a CU each (3 waves per SIMD):
// the waves sharing a SIMD then belong to one workgroup, dispatched together, so none of them
// is favoured for being older (with three 4-wave workgroups per CU the last-dispatched third
// of the scan finished about 6 us after the first on the 1M-context batch-4 step), and each
// append workgroup has a CU to itself and its W_idx rows in LDS (compress_entry_lds).
// Workgroups 0 .. n_q - 1 append query t = blockIdx.x's entry and score the tile holding it
// (first wave); workgroup n_q + s scans the groups of 4 tiles j, j + per_q, ... of query
// s % n_q (j = s / n_q), its waves claiming the tiles one at a time: the 3 waves sharing a SIMD
// are still issued oldest first, and with equal static shares the youngest third finished
// about 6 us after the oldest.
// kHist: the launch also counts every query's older block maxima into hist (kSelBins bins per
// query, as the selection's first pass: csa2_append_index_score_sel): a scan workgroup counts
// its tiles' blocks in LDS and adds its non-zero bins at its end, the append workgroup adds the
// older blocks of the tile it scores.
constexpr int kWideWaves = 12;
constexpr int kWideThreads = 64 * kWideWaves;

template <bool kScores, bool kHist = false>
__global__ __launch_bounds__(kWideThreads) void append_index_wide_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ idx_cache,
    const void* __restrict__ q_in, const float* __restrict__ head_w, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, int32_t n_q, int32_t width, float* __restrict__ scores,
    float* __restrict__ block_max, int64_t w_stride, int32_t per_q, uint32_t* __restrict__ hist) {
  const int L = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (L >= n_q) {  // groups of 4 tiles j, j + per_q, ... of query t, claimed a tile at a time
    const int s = L - n_q, t = s % n_q, j = s / n_q;
    __shared__ uint32_t claim;
    if constexpr (kHist) {
      __shared__ uint32_t lh[kSelBins];
      for (int b = threadIdx.x; b < kSelBins; b += kWideThreads) lh[b] = 0u;
      if (threadIdx.x == 0) claim = 0u;
      __syncthreads();
      score_tiles<false, false, kOlderSlots, false, kScores, true>(q_in, head_w, idx_cache, q_base, q_nvis, nullptr,
                                                                   0, width, scores, block_max, t, j, per_q, nullptr,
                                                                   nullptr, &claim, lh);
      __syncthreads();
      // the query's workgroups end together: each starts its pass over the bins at its own
      // offset, so their adds to one bin do not all arrive at once
      uint32_t* gh = hist + (int64_t)t * kSelBins;
      for (int i = threadIdx.x; i < kSelBins; i += kWideThreads) {
        const int b = (i + 64 * j) & (kSelBins - 1);
        if (lh[b]) atomicAdd(&gh[b], lh[b]);
      }
    } else {
      if (threadIdx.x == 0) claim = 0u;
      __syncthreads();
      score_tiles<false, false, kOlderSlots, false, kScores, true>(q_in, head_w, idx_cache, q_base, q_nvis, nullptr,
                                                                   0, width, scores, block_max, t, j, per_q, nullptr,
                                                                   nullptr, &claim);
    }
    return;
  }
  const int t = L;
  __shared__ EntryShared sh;
  __shared__ WRows wl;
  const int32_t nvis = q_nvis[t];
  const int64_t row = nvis > 0 ? q_base[t] + nvis - 1 : -1;  // nothing visible: nothing appended
  compress_entry_lds<kWideWaves>(latent + (int64_t)t * m * kD, m, pool_w + t * w_stride, rope_cs + (int64_t)t * kDRope,
                                 w_idx, row, kv_cache, idx_cache, sh, wl);
  if (wave != 0) return;  // the newest tile is one tile: one wave scores it
  score_tiles<false, false, kNewestSlots, false, kScores>(q_in, head_w, idx_cache, q_base, q_nvis, nullptr, 0, width,
                                                          scores, block_max, t, 0, 1, sh.idx_row, nullptr, nullptr,
                                                          nullptr, kHist ? hist + (int64_t)t * kSelBins : nullptr);
}

// One of the 512 tasks (head, group of 32 channels, quarter) of packing the query of t to
// MXFP4 into LDS by the rules of csa2_quantize_q_mxfp4 (mxfp4_pack8), 4 consecutive lanes per
// group.
__device__ __forceinline__ void pack_query_task(const uint16_t* __restrict__ q, uint8_t* rec, int task) {
  const int v = task >> 4, grp = (task >> 2) & 3, sub = task & 3;
  uint32_t code;
  const uint32_t word = mxfp4_pack8(*reinterpret_cast<const uint4*>(q + v * kIdxDim + 32 * grp + 8 * sub), code);
  *reinterpret_cast<uint32_t*>(rec + v * kIdxBytes + 16 * grp + 4 * sub) = word;
  if (sub == 0) rec[v * kIdxBytes + 64 + grp] = (uint8_t)code;
}

// The MXFP4-query step with the bf16 query packed inside the launch (which saves the packer's
// launch), in whole-CU workgroups of 12 waves as append_index_wide_kernel: every workgroup
// packs the query into LDS (the first 512 threads, one task each, by the rules of
// csa2_quantize_q_mxfp4), n_q append workgroups, then per_q claimed-tile scan workgroups per
// query (32.6 -> 29.3 us per launch on the 1M-context batch-4 step against 4-wave workgroups
// at 4 per CU; 16-wave workgroups, 4 waves per SIMD, spilled 7 registers and ran no faster).
template <int kWavesWg>
__global__ __launch_bounds__(64 * kWavesWg) void append_index_packq_wide_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ idx_cache,
    const uint16_t* __restrict__ q_bf16, const float* __restrict__ head_w, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, int32_t n_q, int32_t width, float* __restrict__ scores,
    float* __restrict__ block_max, int64_t w_stride, int32_t per_q) {
  const int L = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int t = L < n_q ? L : (L - n_q) % n_q;
  __shared__ __attribute__((aligned(16))) uint8_t q_rec[kIdxHeads * kIdxBytes];
  __shared__ uint32_t claim;
  if (threadIdx.x < kIdxHeads * 16) pack_query_task(q_bf16 + (int64_t)t * kIdxHeads * kIdxDim, q_rec, threadIdx.x);
  if (threadIdx.x == 0) claim = 0u;
  __syncthreads();
  if (L >= n_q) {
    score_tiles<false, true, kOlderSlots, false, true, true>(q_bf16, head_w, idx_cache, q_base, q_nvis, nullptr, 0,
                                                             width, scores, block_max, t, (L - n_q) / n_q, per_q,
                                                             nullptr, q_rec, &claim);
    return;
  }
  __shared__ EntryShared sh;
  __shared__ WRows wl;
  const int32_t nvis = q_nvis[t];
  const int64_t row = nvis > 0 ? q_base[t] + nvis - 1 : -1;  // nothing visible: nothing appended
  compress_entry_lds<kWavesWg>(latent + (int64_t)t * m * kD, m, pool_w + t * w_stride,
                                  rope_cs + (int64_t)t * kDRope, w_idx, row, kv_cache, idx_cache, sh, wl);
  if (wave != 0) return;
  score_tiles<false, true, kNewestSlots>(q_bf16, head_w, idx_cache, q_base, q_nvis, nullptr, 0, width, scores,
                                         block_max, t, 0, 1, sh.idx_row, q_rec);
}

struct MeanEntryShared {
  EntryShared e;
  __attribute__((aligned(16))) uint8_t mean_row[kIdxBytes + 12];  // the newest block's record (68 B)
};

// mean_cache rows mean_base[t] .. hold query t's block means (block b = entries 8b .. 8b + 7
// of its sequence); the scores are those of the ceil(q_nvis[t] / 8) visible block means
template <bool kFp4Q>
__global__ __launch_bounds__(kThreads) void append_mean_index_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ idx_cache,
    uint8_t* __restrict__ mean_cache, const int64_t* __restrict__ mean_base, const void* __restrict__ q_in,
    const float* __restrict__ head_w, const int64_t* __restrict__ q_base, const int32_t* __restrict__ q_nvis,
    int32_t width, float* __restrict__ scores, float* __restrict__ block_max, int64_t w_stride) {
  const int t = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (blockIdx.x >= kAppendWgs) {
    score_tiles<false, kFp4Q, kOlderSlots, true>(q_in, head_w, mean_cache, mean_base, q_nvis, nullptr, 0, width,
                                                 scores, block_max, t,
                                                 (int32_t)(blockIdx.x - kAppendWgs) * kWaves + wave,
                                                 (int32_t)(gridDim.x - kAppendWgs) * kWaves);
    return;
  }
  __shared__ MeanEntryShared sh;
  const int32_t nvis = q_nvis[t];
  const int64_t row = nvis > 0 ? q_base[t] + nvis - 1 : -1;  // nothing visible: nothing appended
  compress_entry_wg(latent + (int64_t)t * m * kD, m, pool_w + t * w_stride, rope_cs + (int64_t)t * kDRope, w_idx, row, kv_cache,
                    idx_cache, sh.e);
  if (nvis > 0 && threadIdx.x < 16) {  // lane 4g + sub: channels 32g + 8sub .. + 7
    const int g = threadIdx.x >> 2, sub = threadIdx.x & 3;
    const int32_t b = (nvis - 1) / kBlock;  // the newest block
    const int cnt = nvis - b * kBlock;
    uint32_t code;
    const uint32_t word = block_mean_word(idx_cache, q_base[t] + (int64_t)b * kBlock, cnt, sh.e.idx_row, g, sub, code);
    idx_store_word(mean_cache, mean_base[t] + b, g, sub, word, code);
    *reinterpret_cast<uint32_t*>(&sh.mean_row[16 * g + 4 * sub]) = word;
    if (sub == 0) sh.mean_row[64 + g] = (uint8_t)code;
  }
  __syncthreads();
  score_tiles<false, kFp4Q, kNewestSlots, true>(q_in, head_w, mean_cache, mean_base, q_nvis, nullptr, 0, width,
                                                scores, block_max, t, wave, kWaves, sh.mean_row);
}

// HISA's bf16-query decode launch in whole-CU workgroups, as append_index_wide_kernel: n_q
// append workgroups (compress_entry_lds, then the first wave re-packs the newest block's mean
// record and scores the tile of block means holding it), then per_q scan workgroups per query
// over groups of 4 tiles of block means, their waves claiming the tiles.
__global__ __launch_bounds__(kWideThreads) void append_mean_index_wide_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ idx_cache,
    uint8_t* __restrict__ mean_cache, const int64_t* __restrict__ mean_base, const void* __restrict__ q_in,
    const float* __restrict__ head_w, const int64_t* __restrict__ q_base, const int32_t* __restrict__ q_nvis,
    int32_t n_q, int32_t width, float* __restrict__ scores, float* __restrict__ block_max, int64_t w_stride,
    int32_t per_q) {
  const int L = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (L >= n_q) {
    __shared__ uint32_t claim;
    if (threadIdx.x == 0) claim = 0u;
    __syncthreads();
    const int s = L - n_q, t = s % n_q, j = s / n_q;
    score_tiles<false, false, kOlderSlots, true, true, true>(q_in, head_w, mean_cache, mean_base, q_nvis, nullptr, 0,
                                                             width, scores, block_max, t, j, per_q, nullptr, nullptr,
                                                             &claim);
    return;
  }
  const int t = L;
  __shared__ MeanEntryShared sh;
  __shared__ WRows wl;
  const int32_t nvis = q_nvis[t];
  const int64_t row = nvis > 0 ? q_base[t] + nvis - 1 : -1;  // nothing visible: nothing appended
  compress_entry_lds<kWideWaves>(latent + (int64_t)t * m * kD, m, pool_w + t * w_stride, rope_cs + (int64_t)t * kDRope,
                                 w_idx, row, kv_cache, idx_cache, sh.e, wl);
  if (wave != 0) return;
  if (nvis > 0 && threadIdx.x < 16) {  // lane 4g + sub: channels 32g + 8sub .. + 7
    const int g = threadIdx.x >> 2, sub = threadIdx.x & 3;
    const int32_t b = (nvis - 1) / kBlock;  // the newest block
    const int cnt = nvis - b * kBlock;
    uint32_t code;
    const uint32_t word = block_mean_word(idx_cache, q_base[t] + (int64_t)b * kBlock, cnt, sh.e.idx_row, g, sub, code);
    idx_store_word(mean_cache, mean_base[t] + b, g, sub, word, code);
    *reinterpret_cast<uint32_t*>(&sh.mean_row[16 * g + 4 * sub]) = word;
    if (sub == 0) sh.mean_row[64 + g] = (uint8_t)code;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the record is in LDS for this wave's reads
  __builtin_amdgcn_wave_barrier();
  score_tiles<false, false, kNewestSlots, true>(q_in, head_w, mean_cache, mean_base, q_nvis, nullptr, 0, width, scores,
                                                block_max, t, 0, 1, sh.mean_row);
}

// workgroups of each kernel of this file that fit on the device at once (per device)
std::atomic<int> resident_entry[kMaxDevices], resident_entry_max[kMaxDevices], resident_fp4q[kMaxDevices],
    resident_packq[kMaxDevices], resident_mean[kMaxDevices], resident_mean_fp4q[kMaxDevices],
    resident_sel[kMaxDevices], resident_sel_max[kMaxDevices];

// scan workgroups per query of append_index_wide_kernel: the resident workgroups left after the
// n_q append workgroups, shared evenly (at least one, at most one per 3 groups of 4 tiles)
int32_t wide_per_q(int resident, int32_t n_q, int32_t width) {
  const int32_t ntiles = (width + kTile - 1) / kTile;
  int64_t per_q = (resident - (int64_t)n_q) / n_q;
  const int64_t max_q = (ntiles + kWideWaves - 1) / kWideWaves;
  if (per_q > max_q) per_q = max_q;
  if (per_q < 1) per_q = 1;
  return (int32_t)per_q;
}

// workgroups along x: the append workgroup, then the scan's share of one round of resident
// workgroups (at least one, at most what the row's tiles can use)
int64_t grid_x(int resident, int32_t n_q, int32_t width) {
  const int32_t ntiles = (width + kTile - 1) / kTile;
  int64_t scan_x = resident / n_q - kAppendWgs;
  const int64_t max_x = (ntiles + kWaves - 1) / kWaves;
  if (scan_x > max_x) scan_x = max_x;
  if (scan_x < 1) scan_x = 1;
  return kAppendWgs + scan_x;
}

// floats from one query's pooling-weight rows to the next: 0 for the static [m, 512] weights,
// m * 512 for per-token weights [n_q * m, 512]
int64_t weight_stride(int m, int per_token_w) { return (per_token_w && m > 1) ? (int64_t)m * kD : 0; }

// the checks both fused calls share
template <bool kFp4Q>
int check_args(const uint16_t* latent, int m, const float* pool_w, int per_token_w, const float* rope_cs,
               const uint16_t* w_idx, uint8_t* kv_cache, uint8_t* idx_cache, const void* q, const float* head_w,
               const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
               float* block_max, bool maxima_only_ok = false) {
  if (n_q < 0 || width < 0 || (per_token_w != 0 && per_token_w != 1)) return CSA2_ERR_INVALID_ARG;
  if (m != 1 && m != 2) return CSA2_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (width == 0) return CSA2_ERR_INVALID_ARG;  // every query appends into a visible slot
  if (!latent || !rope_cs || !w_idx || !kv_cache || !idx_cache || !q || !head_w || !q_base || !q_nvis)
    return CSA2_ERR_INVALID_ARG;
  if (!scores && !(maxima_only_ok && block_max)) return CSA2_ERR_INVALID_ARG;  // NULL scores: maxima only
  if (m == 2 && !pool_w) return CSA2_ERR_INVALID_ARG;
  if (n_q > 65535 || width > kMaxIndexWidth) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(w_idx) |
       reinterpret_cast<uintptr_t>(kv_cache) | reinterpret_cast<uintptr_t>(idx_cache)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(q) & (kFp4Q ? 3 : 15)) return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(rope_cs) | reinterpret_cast<uintptr_t>(pool_w) |
       reinterpret_cast<uintptr_t>(head_w) | reinterpret_cast<uintptr_t>(scores) |
       reinterpret_cast<uintptr_t>(block_max)) & 3)
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

template <bool kFp4Q>
int append_index_entry(const uint16_t* latent, int m, const float* pool_w, int per_token_w, const float* rope_cs,
                       const uint16_t* w_idx, uint8_t* kv_cache, uint8_t* idx_cache, const void* q,
                       const float* head_w, const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                       float* scores, float* block_max, void* stream) {
  const int rc = check_args<kFp4Q>(latent, m, pool_w, per_token_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base, q_nvis,
                                  n_q, width, scores, block_max, !kFp4Q);
  if (rc != CSA2_OK || n_q == 0) return rc;
  if constexpr (!kFp4Q) {  // bf16 query: whole-CU workgroups (with scores NULL, block maxima only)
    const int32_t per_q =
        scores ? wide_per_q(resident_workgroups(append_index_wide_kernel<true>, kWideThreads, resident_entry), n_q, width)
               : wide_per_q(resident_workgroups(append_index_wide_kernel<false>, kWideThreads, resident_entry_max), n_q,
                            width);
    const int64_t grid = (int64_t)n_q * (1 + per_q);
    if (scores)
      hipLaunchKernelGGL(append_index_wide_kernel<true>, dim3((unsigned)grid), dim3(kWideThreads), 0, (hipStream_t)stream,
                         latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base, q_nvis, n_q, width,
                         scores, block_max, weight_stride(m, per_token_w), per_q, nullptr);
    else
      hipLaunchKernelGGL(append_index_wide_kernel<false>, dim3((unsigned)grid), dim3(kWideThreads), 0,
                         (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                         q_nvis, n_q, width, scores, block_max, weight_stride(m, per_token_w), per_q, nullptr);
    return check_launch();
  } else {
    const int64_t gx = grid_x(resident_workgroups(append_index_kernel<true>, kThreads, resident_fp4q), n_q, width);
    hipLaunchKernelGGL(append_index_kernel<true>, dim3((unsigned)gx, (unsigned)n_q), dim3(kThreads), 0,
                       (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                       q_nvis, width, scores, block_max, weight_stride(m, per_token_w));
    return check_launch();
  }
}

int append_index_sel_entry(const uint16_t* latent, int m, const float* pool_w, int per_token_w, const float* rope_cs,
                           const uint16_t* w_idx, uint8_t* kv_cache, uint8_t* idx_cache, const uint16_t* q,
                           const float* head_w, const int64_t* q_base, const int32_t* q_nvis, int32_t n_q,
                           int32_t width, float* scores, float* block_max, void* sel_ws, size_t sel_ws_bytes,
                           void* stream) {
  const int rc = check_args<false>(latent, m, pool_w, per_token_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                                   q_nvis, n_q, width, scores, block_max, true);
  if (rc != CSA2_OK || n_q == 0) return rc;
  if (!block_max) return CSA2_ERR_INVALID_ARG;  // the histogram counts the block maxima written
  if (!sel_ws || (reinterpret_cast<uintptr_t>(sel_ws) & 3)) return CSA2_ERR_INVALID_ARG;
  if (sel_ws_bytes < (size_t)n_q * kSelBins * sizeof(uint32_t)) return CSA2_ERR_WORKSPACE;
  uint32_t* hist = static_cast<uint32_t*>(sel_ws);  // the selection workspace starts with the histogram rows
  if (scores) {
    const int32_t per_q =
        wide_per_q(resident_workgroups(append_index_wide_kernel<true, true>, kWideThreads, resident_sel), n_q, width);
    const int64_t grid = (int64_t)n_q * (1 + per_q);
    hipLaunchKernelGGL((append_index_wide_kernel<true, true>), dim3((unsigned)grid), dim3(kWideThreads), 0,
                       (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                       q_nvis, n_q, width, scores, block_max, weight_stride(m, per_token_w), per_q, hist);
  } else {
    const int32_t per_q = wide_per_q(
        resident_workgroups(append_index_wide_kernel<false, true>, kWideThreads, resident_sel_max), n_q, width);
    const int64_t grid = (int64_t)n_q * (1 + per_q);
    hipLaunchKernelGGL((append_index_wide_kernel<false, true>), dim3((unsigned)grid), dim3(kWideThreads), 0,
                       (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                       q_nvis, n_q, width, scores, block_max, weight_stride(m, per_token_w), per_q, hist);
  }
  return check_launch();
}

int append_index_packq_entry(const uint16_t* latent, int m, const float* pool_w, int per_token_w, const float* rope_cs,
                             const uint16_t* w_idx, uint8_t* kv_cache, uint8_t* idx_cache, const uint16_t* q,
                             const float* head_w, const int64_t* q_base, const int32_t* q_nvis, int32_t n_q,
                             int32_t width, float* scores, float* block_max, void* stream) {
  const int rc = check_args<false>(latent, m, pool_w, per_token_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base, q_nvis,
                                   n_q, width, scores, block_max);
  if (rc != CSA2_OK || n_q == 0) return rc;
  const int32_t per_q =
      wide_per_q(resident_workgroups(append_index_packq_wide_kernel<kWideWaves>, 64 * kWideWaves, resident_packq), n_q,
                 width);
  const int64_t grid = (int64_t)n_q * (1 + per_q);
  hipLaunchKernelGGL(append_index_packq_wide_kernel<kWideWaves>, dim3((unsigned)grid), dim3(64 * kWideWaves), 0,
                     (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base,
                     q_nvis, n_q, width, scores, block_max, weight_stride(m, per_token_w), per_q);
  return check_launch();
}

template <bool kFp4Q>
int append_mean_index_entry(const uint16_t* latent, int m, const float* pool_w, int per_token_w, const float* rope_cs,
                            const uint16_t* w_idx, uint8_t* kv_cache, uint8_t* idx_cache, uint8_t* mean_cache,
                            const int64_t* mean_base, const void* q, const float* head_w, const int64_t* q_base,
                            const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores, float* block_max,
                            void* stream) {
  const int rc = check_args<kFp4Q>(latent, m, pool_w, per_token_w, rope_cs, w_idx, kv_cache, idx_cache, q, head_w, q_base, q_nvis,
                                  n_q, width, scores, block_max);
  if (rc != CSA2_OK || n_q == 0) return rc;
  if (!mean_cache || !mean_base || (reinterpret_cast<uintptr_t>(mean_cache) & 15)) return CSA2_ERR_INVALID_ARG;
  if constexpr (!kFp4Q) {  // bf16 query: whole-CU workgroups over the block means
    const int32_t per_q =
        wide_per_q(resident_workgroups(append_mean_index_wide_kernel, kWideThreads, resident_mean), n_q, width);
    const int64_t grid = (int64_t)n_q * (1 + per_q);
    hipLaunchKernelGGL(append_mean_index_wide_kernel, dim3((unsigned)grid), dim3(kWideThreads), 0, (hipStream_t)stream,
                       latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, mean_cache, mean_base, q, head_w,
                       q_base, q_nvis, n_q, width, scores, block_max, weight_stride(m, per_token_w), per_q);
    return check_launch();
  } else {
    const int64_t gx =
        grid_x(resident_workgroups(append_mean_index_kernel<true>, kThreads, resident_mean_fp4q), n_q, width);
    hipLaunchKernelGGL(append_mean_index_kernel<true>, dim3((unsigned)gx, (unsigned)n_q), dim3(kThreads), 0,
                       (hipStream_t)stream, latent, m, pool_w, rope_cs, w_idx, kv_cache, idx_cache, mean_cache,
                       mean_base, q, head_w, q_base, q_nvis, width, scores, block_max, weight_stride(m, per_token_w));
    return check_launch();
  }
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_append_index_score(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w, const float* rope_cs,
                                       const uint16_t* w_idx_bf16, uint8_t* kv_cache, uint8_t* idx_cache,
                                       const uint16_t* q_idx_bf16, const float* head_w, const int64_t* q_base,
                                       const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                                       float* block_max, void* stream) {
  return csa2::append_index_entry<false>(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache, q_idx_bf16,
                                         head_w, q_base, q_nvis, n_q, width, scores, block_max, stream);
}

extern "C" int csa2_append_index_score_sel(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w,
                                           const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_cache,
                                           uint8_t* idx_cache, const uint16_t* q_idx_bf16, const float* head_w,
                                           const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                                           float* scores, float* block_max, void* sel_workspace, size_t sel_ws_bytes,
                                           void* stream) {
  return csa2::append_index_sel_entry(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache,
                                      q_idx_bf16, head_w, q_base, q_nvis, n_q, width, scores, block_max, sel_workspace,
                                      sel_ws_bytes, stream);
}

extern "C" int csa2_append_index_score_fp4q(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w,
                                            const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_cache,
                                            uint8_t* idx_cache, const uint8_t* q_fp4, const float* head_w,
                                            const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                                            float* scores, float* block_max, void* stream) {
  return csa2::append_index_entry<true>(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache, q_fp4,
                                        head_w, q_base, q_nvis, n_q, width, scores, block_max, stream);
}

extern "C" int csa2_append_index_score_packq(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w,
                                             const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_cache,
                                             uint8_t* idx_cache, const uint16_t* q_idx_bf16, const float* head_w,
                                             const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                                             float* scores, float* block_max, void* stream) {
  return csa2::append_index_packq_entry(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache, q_idx_bf16,
                                        head_w, q_base, q_nvis, n_q, width, scores, block_max, stream);
}

extern "C" int csa2_append_mean_index_score(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w,
                                            const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_cache,
                                            uint8_t* idx_cache, uint8_t* mean_cache, const int64_t* mean_base,
                                            const uint16_t* q_idx_bf16, const float* head_w, const int64_t* q_base,
                                            const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                                            float* block_max, void* stream) {
  return csa2::append_mean_index_entry<false>(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache,
                                              mean_cache, mean_base, q_idx_bf16, head_w, q_base, q_nvis, n_q, width,
                                              scores, block_max, stream);
}

extern "C" int csa2_append_mean_index_score_fp4q(const uint16_t* latent_bf16, int m, const float* pool_w, int per_token_w,
                                                 const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_cache,
                                                 uint8_t* idx_cache, uint8_t* mean_cache, const int64_t* mean_base,
                                                 const uint8_t* q_fp4, const float* head_w, const int64_t* q_base,
                                                 const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                                                 float* block_max, void* stream) {
  return csa2::append_mean_index_entry<true>(latent_bf16, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache,
                                             mean_cache, mean_base, q_fp4, head_w, q_base, q_nvis, n_q, width, scores,
                                             block_max, stream);
}
