// index_score.hip -- lightning-indexer scoring over the MXFP4 indexer-K cache (gfx950).
//
// Computes s(t, j) = sum_h w[t,h] * max(0, q[t,h,:] . k^_j) ([ZB] "把 KV Cache 压缩推到极致"
// §3.3.2: indexer query and per-head weights produce the Top-K set; §2.3.4 / [DF]
// "CSA2 与每 token 890 字节" §4.7: a Full layer scores every visible entry and reduces
// blocks of 8 by max, a Reindex layer scores only its candidate pool).
//
// Design.  One wavefront owns one query and streams tiles of 32 entries.  The 32 heads
// x 128 dims contraction runs on v_mfma_f32_32x32x16_bf16 with the heads as the M
// dimension: the query sits in registers as eight A fragments for the whole scan, and
// each tile's B fragments are built in registers straight from the packed bytes: every
// lane loads 32 contiguous payload bytes of one entry (half of its 64) plus the 4-byte
// scale word, and v_cvt_scalef32_pk_bf16_fp4 turns two E2M1 nibbles and their E8M0
// power-of-two scale into two exact bf16 values.  The K dimension is permuted so that
// lane group g and step s hold dims 64g + 8s .. 64g + 8s + 7 for both operands, which
// leaves the dot products unchanged and makes each lane's bytes contiguous.  ReLU, the
// head weights and the head sum run on the accumulator registers; a 32-lane swap
// finishes the sum.  HBM traffic per entry is its 68 bytes plus 4.5 bytes of output.  The
// waves of the grid walk a query's tiles in grid-stride order, so the whole grid streams
// one front of the row at a time.
#include "index_common.hpp"

namespace csa2 {
namespace {
using namespace idx;

#ifndef CSA2_INDEX_DEPTH
#define CSA2_INDEX_DEPTH 4
#endif
constexpr int kDepth = CSA2_INDEX_DEPTH;  // tiles in flight per wave

__global__ __launch_bounds__(kThreads) void index_score_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ head_w,
    const uint8_t* __restrict__ idx_cache, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M,
    int32_t width, float* __restrict__ scores, float* __restrict__ block_max) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 31, g = lane >> 5;
  const int32_t nvis = q_nvis[t];
  const int64_t base = q_base[t];
  const int32_t ntiles = (width + kTile - 1) / kTile;
  // grid-stride tile order: at any moment the grid streams one front of the row
  const int32_t first = (int32_t)blockIdx.x * kWaves + wave;
  const int32_t tstride = (int32_t)gridDim.x * kWaves;
  const int32_t nt = first < ntiles ? (ntiles - first + tstride - 1) / tstride : 0;  // this wave's tiles
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  float* srow = scores + (int64_t)t * width;

  if (nvis <= 0) {  // nothing visible: the row is all -inf
    for (int32_t k = 0; k < nt; k++) {
      const int32_t p = (first + k * tstride) * kTile + n;
      if (g == 0 && p < width) srow[p] = -__builtin_inff();
      if (block_max != nullptr && g == 0 && (n & 7) == 0 && p < width)
        block_max[(int64_t)t * nbw + (p >> 3)] = -__builtin_inff();
    }
    return;
  }

  // query: head n, dims 64g .. 64g + 63 as eight bf16x8 A fragments
  bf16x8 a[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + ((int64_t)t * kIdxHeads + n) * kIdxDim + 64 * g);
#pragma unroll
    for (int s = 0; s < 8; s++) a[s] = __builtin_bit_cast(bf16x8, qp[s]);
  }
  // head weight of each accumulator row held by this lane: row = 8(r/4) + 4g + r%4
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; r++) wr[r] = head_w[(int64_t)t * kIdxHeads + 8 * (r >> 2) + 4 * g + (r & 3)];

  const uint8_t* last_row = idx_cache + (base + nvis - 1) * kIdxBytes;
  // the cache row of this lane's entry in tile k; invalid slots read the last visible row
  auto row_of = [&](int32_t k, bool& valid) -> const uint8_t* {
    const int32_t p = (first + k * tstride) * kTile + n;
    int64_t j;
    if (pool_blocks == nullptr) {
      j = p;
      valid = p < nvis;
    } else {
      const int32_t slot = p >> 3;
      const int32_t b = slot < M ? pool_blocks[(int64_t)t * M + slot] : -1;
      j = (int64_t)b * kBlock + (p & 7);
      valid = b >= 0 && j < nvis;
    }
    return valid ? idx_cache + (base + j) * kIdxBytes : last_row;
  };
  auto load = [&](int32_t k, RawTile& r, bool& valid) {
    const uint8_t* row = row_of(k, valid);
    r.lo = *reinterpret_cast<const u32x4_a4*>(row + 32 * g);
    r.hi = *reinterpret_cast<const u32x4_a4*>(row + 32 * g + 16);
    r.sc = *reinterpret_cast<const uint32_t*>(row + 64);
  };
  auto process = [&](const RawTile& cur, bool valid, int32_t k) {
    const float x0 = e8m0_scale((cur.sc >> (16 * g)) & 255u);
    const float x1 = e8m0_scale((cur.sc >> (16 * g + 8)) & 255u);
    const uint32_t words[8] = {cur.lo[0], cur.lo[1], cur.lo[2], cur.lo[3], cur.hi[0], cur.hi[1], cur.hi[2], cur.hi[3]};
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const bf16x8 b = cvt_fp4x8(words[s], s < 4 ? x0 : x1);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b, acc, 0, 0, 0);
    }
    // ReLU, head weight and the sum over this lane's 16 heads as four short chains
    float part[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      part[c] = wr[4 * c] * __builtin_fmaxf(acc[4 * c], 0.0f);
#pragma unroll
      for (int r = 1; r < 4; r++) part[c] = __builtin_fmaf(wr[4 * c + r], __builtin_fmaxf(acc[4 * c + r], 0.0f), part[c]);
    }
    const float sc = valid ? sum_halves((part[0] + part[1]) + (part[2] + part[3])) : -__builtin_inff();
    const int32_t p = (first + k * tstride) * kTile + n;
    if (g == 0 && p < width) srow[p] = sc;
    if (block_max != nullptr) {
      const float bm = max8_lanes(sc);
      if (g == 0 && (n & 7) == 0 && p < width) block_max[(int64_t)t * nbw + (p >> 3)] = bm;
    }
  };

  // software pipeline: kDepth tiles of this wave are in flight while one is processed
  RawTile pipe[kDepth];
  bool pv[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; u++)
    if (u < nt) load(u, pipe[u], pv[u]);
  for (int32_t k0 = 0; k0 < nt; k0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      const int32_t k = k0 + u;
      if (k < nt) {
        const RawTile cur = pipe[u];
        const bool cv = pv[u];
        if (k + kDepth < nt) load(k + kDepth, pipe[u], pv[u]);
        process(cur, cv, k);
      }
    }
  }
}

}  // namespace
}  // namespace csa2

namespace {
// workgroups of index_score_kernel that fit on the device at once (queried per device)
int resident_workgroups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, csa2::index_score_kernel, csa2::kThreads, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 2;
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}
}  // namespace

extern "C" int csa2_index_score(const uint16_t* q_idx_bf16, const float* head_w,
                                const uint8_t* idx_cache, const int64_t* q_base,
                                const int32_t* q_nvis, const int32_t* pool_blocks, int32_t M,
                                int32_t n_q, int32_t width, float* scores, float* block_max,
                                void* stream) {
  using namespace csa2;
  if (n_q < 0 || width < 0) return CSA2_ERR_INVALID_ARG;
  if (n_q == 0 || width == 0) return CSA2_OK;
  if (!q_idx_bf16 || !head_w || !idx_cache || !q_base || !q_nvis || !scores) return CSA2_ERR_INVALID_ARG;
  if (pool_blocks) {
    if (M < 1) return CSA2_ERR_INVALID_ARG;
    if (M > kMaxPool) return CSA2_ERR_UNSUPPORTED;
    if ((int64_t)width != 8LL * M) return CSA2_ERR_INVALID_ARG;
    if (block_max) return CSA2_ERR_INVALID_ARG;
  }
  if (n_q > 65535) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_idx_bf16) | reinterpret_cast<uintptr_t>(idx_cache)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(head_w) | reinterpret_cast<uintptr_t>(scores) |
       reinterpret_cast<uintptr_t>(block_max)) & 3)
    return CSA2_ERR_INVALID_ARG;
  const int32_t ntiles = (width + kTile - 1) / kTile;
  if (pool_blocks == nullptr && n_q >= kMqMinQueries)  // many queries: shared K-tile decode
    return launch_index_score_mq(q_idx_bf16, head_w, idx_cache, q_base, q_nvis, n_q, width, scores, block_max,
                                 stream);
  // one full round of resident workgroups; each wave strides over its query's tiles
  int64_t grid_x = (resident_workgroups() + n_q - 1) / n_q;
  const int64_t max_x = (ntiles + kWaves - 1) / kWaves;
  if (grid_x > max_x) grid_x = max_x;
  if (grid_x < 1) grid_x = 1;
  hipLaunchKernelGGL(index_score_kernel, dim3((unsigned)grid_x, n_q), dim3(kThreads), 0, (hipStream_t)stream,
                     q_idx_bf16, head_w, idx_cache, q_base, q_nvis, pool_blocks, M, width, scores, block_max);
  return check_launch();
}
