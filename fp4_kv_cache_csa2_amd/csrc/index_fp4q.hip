// index_fp4q.hip -- the lightning indexer with an MXFP4 query (gfx950).
//
// [ZB] "把 KV Cache 压缩推到极致" §2.4.4: DeepSeek-V4 already trains both the indexer Q and
// the indexer K for FP4.  The query's head vectors are packed in the indexer-K format (OCP
// MXFP4: 128 E2M1 codes, one E8M0 scale per 32 channels, 68 bytes) and the score is the
// usual s(t, j) = sum_h w_h max(0, q^_h . k^_j) with q^_h the dequantised head vector.
//
// With both operands in MXFP4 the contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4,
// which takes the stored codes and E8M0 scales as they are: a 32-entry tile of one query
// is two instructions (four times the bf16 rate) and the K bytes need no conversion.  What
// remains on the vector ALU is the epilogue (ReLU, head weight, head sum: two operations
// per head and entry), which is what bounds these kernels.
//
// This file holds the query packer and the many-query (prefill) kernel; the one-query
// (decode) kernel is index_score_kernel<., true> in index_score.hip.
#include "index_common.hpp"

namespace csa2 {
namespace {
using namespace idx;

// ---------------------------------------------------------------------------------------
// Query packer: 4 threads per (head vector, group of 32 channels), 8 channels each.  The
// group's amax comes from two shuffles inside the 4 lanes; codes by the exact encoders
// shared with the indexer-K packer, so the bytes equal the indexer-K rule bit for bit.
constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kPackThreads) void quantize_q_mxfp4_kernel(const uint16_t* __restrict__ q,
                                                                        int64_t n_vec, uint8_t* __restrict__ out) {
  const int64_t gi = (int64_t)blockIdx.x * (kPackThreads / 4) + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const int64_t v = gi >> 2;
  const int g = (int)(gi & 3);
  if (v >= n_vec) return;  // the 4 lanes of a group share v: all leave or none
  uint32_t code;
  const uint32_t word = mxfp4_pack8(*reinterpret_cast<const uint4*>(q + v * kIdxDim + 32 * g + 8 * sub), code);
  uint8_t* dst = out + v * kIdxBytes;
  *reinterpret_cast<uint32_t*>(dst + 16 * g + 4 * sub) = word;
  if (sub == 0) dst[64 + g] = (uint8_t)code;
}

// ---------------------------------------------------------------------------------------
// Many queries over one sequence (a prefill chunk) with MXFP4 queries.  Each wave holds
// kFqQPW queries (two 16-byte A fragments and a scale word each) and walks the workgroup's
// tiles; every tile's B fragments (two 16-byte loads and the scale word per lane, L2-hot:
// the whole chunk's K is a few MB) feed 2 x kFqQPW MFMAs.  No LDS staging and no barriers.
// Head weights sit in LDS.  A workgroup whose queries belong to different sequences scores
// each query from its own rows.
constexpr int kFqQPW = 4;                 // queries per wave
constexpr int kFqQB = kFqQPW * kWaves;    // queries per workgroup
constexpr int kFqTiles = 32;              // tiles of 32 entries per workgroup
constexpr int kFqDepth = 3;               // tiles in flight per wave
constexpr int kRawBuf = 0x00020000;       // buffer descriptor word 3: raw 32-bit dwords

template <bool kBmax>
__global__ __launch_bounds__(kThreads) void index_score_mq_fp4q_kernel(
    const uint8_t* __restrict__ q_fp4, const float* __restrict__ head_w, const uint8_t* __restrict__ idx_cache,
    const int64_t* __restrict__ q_base, const int32_t* __restrict__ q_nvis, int32_t n_q, int32_t width,
    float* __restrict__ scores, float* __restrict__ block_max) {
  __shared__ int64_t s_base[kFqQB];
  __shared__ int32_t s_nvis[kFqQB];
  __shared__ __attribute__((aligned(16))) float s_w[kFqQB][kIdxHeads];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int qb0 = blockIdx.y * kFqQB;
  const int32_t ntiles = (width + kTile - 1) / kTile;
  const int32_t tile0 = blockIdx.x * kFqTiles;
  const int32_t tile1 = min(tile0 + kFqTiles, ntiles);
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  if (threadIdx.x < kFqQB) {
    const int t = qb0 + threadIdx.x;
    s_base[threadIdx.x] = t < n_q ? q_base[t] : -1;
    s_nvis[threadIdx.x] = t < n_q ? max(min(q_nvis[t], width), 0) : 0;  // entries past width are never scored
  }
  for (int i = threadIdx.x; i < kFqQB * kIdxHeads; i += kThreads) {
    const int j = i / kIdxHeads, h = i % kIdxHeads;
    const int t = qb0 + j;
    s_w[j][h] = t < n_q ? head_w[(int64_t)t * kIdxHeads + h] : 0.0f;
  }
  __syncthreads();
  const int64_t base0 = s_base[0];
  int32_t max_nvis = 0;
  bool shared = true;
  for (int j = 0; j < kFqQB; j++) {
    if (qb0 + j >= n_q) break;
    max_nvis = max(max_nvis, s_nvis[j]);
    shared = shared && s_base[j] == base0;
  }
  // this wave's queries: A fragments, scale words, visible counts and output rows as
  // buffer resources (empty for a padding slot, so its stores are dropped)
  constexpr int32_t kOut = 1 << 30;  // a byte offset past every buffer's end
  fp4x32 qa[kFqQPW][2];
  uint32_t qsc[kFqQPW];
  int32_t nv[kFqQPW];
  __amdgpu_buffer_rsrc_t rs_s[kFqQPW], rs_b[kFqQPW];
#pragma unroll
  for (int j = 0; j < kFqQPW; j++) {
    const int t = qb0 + wave * kFqQPW + j;
    const bool real = t < n_q;
    const int tt = real ? t : qb0;  // a padding slot reads a real query and writes nothing
    nv[j] = real ? s_nvis[wave * kFqQPW + j] : 0;
    load_fp4_query(q_fp4 + ((int64_t)tt * kIdxHeads + n) * kIdxBytes, g, qa[j], qsc[j]);
    rs_s[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)tt * width, (short)0, real ? width * 4 : 0, kRawBuf);
    rs_b[j] = __builtin_amdgcn_make_buffer_rsrc(kBmax ? (void*)(block_max + (int64_t)tt * nbw) : (void*)scores,
                                                (short)0, (kBmax && real) ? nbw * 4 : 0, kRawBuf);
  }
  // scores of one query for one tile from its accumulators: ReLU, head weights (accumulator
  // row 4c + r of this lane is head 8c + 4g + r), head sum, causal mask, block maximum; one
  // lane stores each value, the others aim past the end of the buffer
  auto finish = [&](int j, const f32x16& acc, int32_t k) {
    const float* wj = &s_w[wave * kFqQPW + j][4 * g];
    float part[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const float4 w4 = *reinterpret_cast<const float4*>(wj + 8 * c);
      part[c] = w4.x * relu(acc[4 * c]);
      part[c] = __builtin_fmaf(w4.y, relu(acc[4 * c + 1]), part[c]);
      part[c] = __builtin_fmaf(w4.z, relu(acc[4 * c + 2]), part[c]);
      part[c] = __builtin_fmaf(w4.w, relu(acc[4 * c + 3]), part[c]);
    }
    const int32_t p = k * kTile + n;
    const float sum = sum_halves((part[0] + part[1]) + (part[2] + part[3]));
    const float sc = masked_score(sum, p < nv[j]);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_s[j], g ? kOut : 4 * p, 0, 0);
    if constexpr (kBmax)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(max8_lanes(sc)), rs_b[j],
                                            (g | (n & 7)) ? kOut : 4 * (p >> 3), 0, 0);
  };

  if (shared && max_nvis > 0) {
    // the tiles of the sequence's entries that some query of the block sees, as a buffer
    // resource; entries past the visible ones (the ragged last tile, the pipeline's
    // overrun) read past its end, which returns zeros
    int32_t rel0;
    const __amdgpu_buffer_rsrc_t rs = idx_rsrc(idx_cache, base0, max_nvis, rel0);
    const int32_t tend = max(min(tile1, (max_nvis + kTile - 1) / kTile), tile0);
    const int32_t nt = tend - tile0;
    auto load = [&](int32_t k, RawTile& r) {
      const int32_t p = k * kTile + n;
      load_entry_share<0>(rs, p < max_nvis ? rel0 + p : -1, g, r);  // L2-hot: every query block reads it
      r.sc >>= 8 * g;
    };
    auto process = [&](const RawTile& cur, int32_t k) {
      f32x16 acc[kFqQPW];
#pragma unroll
      for (int j = 0; j < kFqQPW; j++) acc[j] = mfma_fp4_tile(qa[j], qsc[j], cur.lo, cur.hi, cur.sc, f32x16{});
#pragma unroll
      for (int j = 0; j < kFqQPW; j++) finish(j, acc[j], k);
    };
    // full groups of kFqDepth tiles stream through the loop with no branches; the last
    // partial group is finished after it
    RawTile pipe[kFqDepth];
#pragma unroll
    for (int u = 0; u < kFqDepth; u++) {
      load(tile0 + u, pipe[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int32_t k0 = 0;
    for (; k0 + kFqDepth <= nt; k0 += kFqDepth) {
#pragma unroll
      for (int u = 0; u < kFqDepth; u++) {
        process(pipe[u], tile0 + k0 + u);
        load(tile0 + k0 + u + kFqDepth, pipe[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kFqDepth - 1; u++)
      if (k0 + u < nt) process(pipe[u], tile0 + k0 + u);
    // tiles past every query's visible range
    for (int32_t k = tend; k < tile1; k++) {
#pragma unroll
      for (int j = 0; j < kFqQPW; j++) finish(j, f32x16{}, k);
    }
    return;
  }
  // mixed sequences (or nothing visible): each query from its own rows, one tile at a time
#pragma unroll
  for (int j = 0; j < kFqQPW; j++) {
    const int64_t base = s_base[wave * kFqQPW + j];
    int32_t rel0;
    const __amdgpu_buffer_rsrc_t rs = idx_rsrc(idx_cache, nv[j] > 0 ? base : 0, nv[j], rel0);
    for (int32_t k = tile0; k < tile1; k++) {
      f32x16 acc = {};
      if (k * kTile < nv[j]) {
        const int32_t p = k * kTile + n;
        RawTile r;
        load_entry_share<0>(rs, p < nv[j] ? rel0 + p : -1, g, r);
        acc = mfma_fp4_tile(qa[j], qsc[j], r.lo, r.hi, r.sc >> (8 * g), acc);
      }
      finish(j, acc, k);
    }
  }
}

}  // namespace

int launch_index_score_mq_fp4q(const uint8_t* q_fp4, const float* head_w, const uint8_t* idx_cache,
                               const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                               float* scores, float* block_max, void* stream) {
  const int32_t ntiles = (width + kTile - 1) / kTile;
  const int64_t gx = (ntiles + kFqTiles - 1) / kFqTiles, gy = (n_q + kFqQB - 1) / kFqQB;
  if (gx > 0x7FFFFFFF || gy > 65535) return CSA2_ERR_UNSUPPORTED;
  if (block_max != nullptr)
    hipLaunchKernelGGL(index_score_mq_fp4q_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       (hipStream_t)stream, q_fp4, head_w, idx_cache, q_base, q_nvis, n_q, width, scores, block_max);
  else
    hipLaunchKernelGGL(index_score_mq_fp4q_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       (hipStream_t)stream, q_fp4, head_w, idx_cache, q_base, q_nvis, n_q, width, scores, block_max);
  return check_launch();
}

}  // namespace csa2

// [ZB] §2.4.4 (FP4 indexer query, OCP MXFP4): packs bf16 head vectors into 68-byte records.
extern "C" int csa2_quantize_q_mxfp4(const uint16_t* q_bf16, int64_t n_vec, uint8_t* out, void* stream) {
  using namespace csa2;
  if (n_vec < 0) return CSA2_ERR_INVALID_ARG;
  if (n_vec == 0) return CSA2_OK;
  if (!q_bf16 || !out) return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q_bf16) & 15) | (reinterpret_cast<uintptr_t>(out) & 3)) return CSA2_ERR_INVALID_ARG;
  const int64_t blocks = (n_vec * 4 + kPackThreads / 4 - 1) / (kPackThreads / 4);
  if (blocks > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(quantize_q_mxfp4_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, (hipStream_t)stream,
                     q_bf16, n_vec, out);
  return check_launch();
}
