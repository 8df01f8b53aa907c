// hisa.hip -- block-mean indexer keys for HISA's coarse filter (gfx950).
//
// [ZB] "把 KV Cache 压缩推到极致" §2.3.4 (the HISA paragraphs): the prefix is cut into
// blocks of consecutive entries and each block keeps the mean of its indexer keys as a
// search auxiliary (the token keys stay).  The first stage scores the block means with the
// same indexer query and head weights, the best blocks are expanded into candidate entries,
// and the second stage scores those entries for the final Top-K.  Both stages are the
// existing indexer calls: the block means are stored in the indexer-K format (68-byte MXFP4
// records), so csa2_index_score scores them like entries, csa2_block_topk's pool-only mode
// keeps the best blocks, and candidate mode re-scores and selects inside them.
//
// The mean of a block is the fp32 sum of its entries' exact dequantised keys in ascending
// position order, divided once by the entry count (what a decoding block's running sum and
// count give), then packed by the indexer-K rules.  A decode step re-packs only the block
// that holds the newest entry; completed blocks keep their records.
#include "block_mean.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kRecPerWg = kThreads / 16;  // 16 threads per block record: 4 groups x 4 lanes x 8 channels

__global__ __launch_bounds__(kThreads) void block_mean_pack_kernel(
    const uint8_t* __restrict__ idx_cache, const int64_t* __restrict__ seq_base, const int32_t* __restrict__ seq_n,
    const int32_t* __restrict__ first_block, int32_t n_blocks, uint8_t* __restrict__ mean_cache,
    const int64_t* __restrict__ mean_base) {
  const int s = blockIdx.y;
  const int r = threadIdx.x >> 4, g = (threadIdx.x >> 2) & 3, sub = threadIdx.x & 3;
  const int32_t i = blockIdx.x * kRecPerWg + r;
  const int32_t n = seq_n[s];
  const int32_t b = (first_block ? first_block[s] : 0) + i;
  // the 16 lanes of a record share b: they leave together
  if (i >= n_blocks || b < 0 || (int64_t)b * kBlock >= n) return;
  const int cnt = min(kBlock, n - b * kBlock);
  uint32_t code;
  const uint32_t word = block_mean_word(idx_cache, seq_base[s] + (int64_t)b * kBlock, cnt, nullptr, g, sub, code);
  idx_store_word(mean_cache, mean_base[s] + b, g, sub, word, code);
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_block_mean_pack(const uint8_t* idx_cache, const int64_t* seq_base, const int32_t* seq_n,
                                    const int32_t* first_block, int32_t n_seq, int32_t n_blocks,
                                    uint8_t* mean_cache, const int64_t* mean_base, void* stream) {
  using namespace csa2;
  if (n_seq < 0 || n_blocks < 0) return CSA2_ERR_INVALID_ARG;
  if (n_seq == 0 || n_blocks == 0) return CSA2_OK;
  if (!idx_cache || !seq_base || !seq_n || !mean_cache || !mean_base) return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(idx_cache) | reinterpret_cast<uintptr_t>(mean_cache)) & 3)
    return CSA2_ERR_INVALID_ARG;
  if (n_seq > 65535) return CSA2_ERR_UNSUPPORTED;
  const int64_t gx = ((int64_t)n_blocks + kRecPerWg - 1) / kRecPerWg;
  hipLaunchKernelGGL(block_mean_pack_kernel, dim3((unsigned)gx, (unsigned)n_seq), dim3(kThreads), 0,
                     (hipStream_t)stream, idx_cache, seq_base, seq_n, first_block, n_blocks, mean_cache, mean_base);
  return check_launch();
}
