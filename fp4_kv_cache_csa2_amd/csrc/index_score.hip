// index_score.hip -- csa2_index_score and csa2_index_score_fp4q: lightning-indexer scores
// s(t, j) = sum_h w[t,h] * max(0, q[t,h,:] . k^_j) over the MXFP4 indexer-K cache (gfx950).
//
// [ZB] "把 KV Cache 压缩推到极致" §3.3.2 and §2.3.4, [DF] "CSA2 与每 token 890 字节" §4.7.
// Few queries (decode, Reindex pools) run the wave-per-query tile loop of index_tiles.hpp
// over a grid of one round of resident workgroups; batches of many Full-mode queries
// (prefill chunks) take the shared-tile kernels of index_score_mq.hip / index_fp4q.hip.
#include "index_tiles.hpp"

namespace csa2 {
namespace {
using namespace idx;

template <bool kPool, bool kFp4Q>
__global__ __launch_bounds__(kThreads) void index_score_kernel(
    const void* __restrict__ q_in, const float* __restrict__ head_w,
    const uint8_t* __restrict__ idx_cache, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M,
    int32_t width, float* __restrict__ scores, float* __restrict__ block_max) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  score_tiles<kPool, kFp4Q, kAllSlots>(q_in, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, width, scores,
                                       block_max, blockIdx.y, (int32_t)blockIdx.x * kWaves + wave,
                                       (int32_t)gridDim.x * kWaves);
}

}  // namespace
}  // namespace csa2

namespace {
// workgroups of index_score_kernel that fit on the device at once (per device)
std::atomic<int> resident_index[csa2::kMaxDevices];

// argument checks and launch shared by the bf16-query and MXFP4-query entry points
template <bool kFp4Q>
int index_score_entry(const void* q, const float* head_w, const uint8_t* idx_cache, const int64_t* q_base,
                      const int32_t* q_nvis, const int32_t* pool_blocks, int32_t M, int32_t n_q, int32_t width,
                      float* scores, float* block_max, void* stream) {
  using namespace csa2;
  if (n_q < 0 || width < 0) return CSA2_ERR_INVALID_ARG;
  if (n_q == 0 || width == 0) return CSA2_OK;
  if (!q || !head_w || !idx_cache || !q_base || !q_nvis || !scores) return CSA2_ERR_INVALID_ARG;
  if (pool_blocks) {
    if (M < 1) return CSA2_ERR_INVALID_ARG;
    if (M > kMaxPool) return CSA2_ERR_UNSUPPORTED;
    if ((int64_t)width != 8LL * M) return CSA2_ERR_INVALID_ARG;
    if (block_max) return CSA2_ERR_INVALID_ARG;
  }
  if (n_q > 65535 || width > kMaxIndexWidth) return CSA2_ERR_UNSUPPORTED;
  // bf16 queries are read as 16-byte pieces; MXFP4 query records (68 B) as dwords
  if ((reinterpret_cast<uintptr_t>(q) & (kFp4Q ? 3 : 15)) | (reinterpret_cast<uintptr_t>(idx_cache) & 15))
    return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(head_w) | reinterpret_cast<uintptr_t>(scores) |
       reinterpret_cast<uintptr_t>(block_max)) & 3)
    return CSA2_ERR_INVALID_ARG;
  const int32_t ntiles = (width + kTile - 1) / kTile;
  if (pool_blocks == nullptr && n_q >= kMqMinQueries) {  // many queries: shared K tiles
    if constexpr (kFp4Q)
      return launch_index_score_mq_fp4q(static_cast<const uint8_t*>(q), head_w, idx_cache, q_base, q_nvis, n_q,
                                        width, scores, block_max, stream);
    else
      return launch_index_score_mq(static_cast<const uint16_t*>(q), head_w, idx_cache, q_base, q_nvis, n_q, width,
                                   scores, block_max, stream);
  }
  // one full round of resident workgroups; each wave strides over its query's tiles
  int64_t grid_x = (resident_workgroups(index_score_kernel<false, false>, kThreads, resident_index) + n_q - 1) / n_q;
  const int64_t max_x = (ntiles + kWaves - 1) / kWaves;
  if (grid_x > max_x) grid_x = max_x;
  if (grid_x < 1) grid_x = 1;
  if (pool_blocks != nullptr)
    hipLaunchKernelGGL((index_score_kernel<true, kFp4Q>), dim3((unsigned)grid_x, n_q), dim3(kThreads), 0,
                       (hipStream_t)stream, q, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, width, scores,
                       block_max);
  else
    hipLaunchKernelGGL((index_score_kernel<false, kFp4Q>), dim3((unsigned)grid_x, n_q), dim3(kThreads), 0,
                       (hipStream_t)stream, q, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, width, scores,
                       block_max);
  return check_launch();
}
}  // namespace

extern "C" int csa2_index_score(const uint16_t* q_idx_bf16, const float* head_w,
                                const uint8_t* idx_cache, const int64_t* q_base,
                                const int32_t* q_nvis, const int32_t* pool_blocks, int32_t M,
                                int32_t n_q, int32_t width, float* scores, float* block_max,
                                void* stream) {
  return index_score_entry<false>(q_idx_bf16, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, n_q, width, scores,
                                  block_max, stream);
}

extern "C" int csa2_index_score_fp4q(const uint8_t* q_fp4, const float* head_w, const uint8_t* idx_cache,
                                     const int64_t* q_base, const int32_t* q_nvis, const int32_t* pool_blocks,
                                     int32_t M, int32_t n_q, int32_t width, float* scores, float* block_max,
                                     void* stream) {
  return index_score_entry<true>(q_fp4, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, n_q, width, scores,
                                 block_max, stream);
}
