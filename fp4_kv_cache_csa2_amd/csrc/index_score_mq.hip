// index_score_mq.hip -- lightning-indexer scoring for many queries over one sequence
// (a prefill chunk) on gfx950.
//
// Same score as the single-query kernel ([ZB] "把 KV Cache 压缩推到极致" §3.3.2: s = sum_h
// w_h max(0, q_h . k^_j); [DF] "CSA2 与每 token 890 字节" §4.1 causal visibility), organised
// for the MFMA-bound case where every query reads the same K rows.
#include "index_common.hpp"

namespace csa2 {
namespace {
using namespace idx;

// ---------------------------------------------------------------------------------------
// Many queries over one sequence (a prefill chunk).  Every query of a workgroup reads the
// same K rows, so each tile of 32 entries is decoded once, into LDS as the bf16 B fragments
// of the eight MFMA steps, and every wave runs its two queries against it: one fragment read
// feeds two MFMAs and the FP4 conversion is shared by the eight queries of the workgroup.
// Tiles are double-buffered in LDS and their raw bytes prefetched kMqDepth tiles ahead.  A
// workgroup whose queries belong to different sequences scores each query from its own rows
// instead (the single-query path, one wave per query).
constexpr int kMqQPW = 2;                      // queries per wave
constexpr int kMqQB = kMqQPW * kWaves;         // queries per workgroup
constexpr int kMqTiles = 32;                   // tiles of 32 entries per workgroup
constexpr int kMqDepth = 3;                    // raw tiles in flight per wave

constexpr int kRawBuf = 0x00020000;  // buffer descriptor word 3: raw 32-bit dwords

template <bool kBmax>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void index_score_mq_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ head_w,
    const uint8_t* __restrict__ idx_cache, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, int32_t n_q, int32_t width, float* __restrict__ scores,
    float* __restrict__ block_max) {
  __shared__ __attribute__((aligned(16))) bf16x8 s_b[2][8][64];  // [buffer][MFMA step][lane]
  __shared__ int64_t s_base[kMqQB];
  __shared__ int32_t s_nvis[kMqQB];
  __shared__ __attribute__((aligned(16))) float s_w[kMqQB][kIdxHeads];  // head weights
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int qb0 = blockIdx.y * kMqQB;
  const int32_t ntiles = (width + kTile - 1) / kTile;
  const int32_t tile0 = blockIdx.x * kMqTiles;
  const int32_t tile1 = min(tile0 + kMqTiles, ntiles);
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  if (threadIdx.x < kMqQB) {
    const int t = qb0 + threadIdx.x;
    s_base[threadIdx.x] = t < n_q ? q_base[t] : -1;
    s_nvis[threadIdx.x] = t < n_q ? q_nvis[t] : 0;
  }
  {
    const int j = threadIdx.x >> 5, h = threadIdx.x & 31;  // 256 threads = 8 queries x 32 heads
    const int t = qb0 + j;
    s_w[j][h] = t < n_q ? head_w[(int64_t)t * kIdxHeads + h] : 0.0f;
  }
  __syncthreads();
  const int64_t base0 = s_base[0];
  int32_t max_nvis = 0;
  bool shared = true;
  for (int j = 0; j < kMqQB; j++) {
    if (qb0 + j >= n_q) break;
    max_nvis = max(max_nvis, s_nvis[j]);
    shared = shared && s_base[j] == base0;
  }
  // this wave's queries: A fragments (head n, the scan's channel split: dims 32g + 8s for
  // s < 4, 64 + 32g + 8(s - 4) after), visible counts and output rows as buffer resources
  // (empty for a padding slot, so its stores are dropped)
  constexpr int32_t kOut = 1 << 30;  // a byte offset past every buffer's end
  bf16x8 a[kMqQPW][8];
  int32_t nv[kMqQPW];
  int tq[kMqQPW];
  __amdgpu_buffer_rsrc_t rs_s[kMqQPW], rs_b[kMqQPW];
#pragma unroll
  for (int j = 0; j < kMqQPW; j++) {
    const int t = qb0 + wave * kMqQPW + j;
    tq[j] = t;
    const bool real = t < n_q;
    const int tt = real ? t : qb0;  // a padding slot reads a real query and writes nothing
    nv[j] = real ? s_nvis[wave * kMqQPW + j] : 0;
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + ((int64_t)tt * kIdxHeads + n) * kIdxDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 8; s++) a[j][s] = __builtin_bit_cast(bf16x8, qp[s < 4 ? s : s + 4]);
    rs_s[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)tt * width, (short)0, real ? width * 4 : 0, kRawBuf);
    rs_b[j] = __builtin_amdgcn_make_buffer_rsrc(kBmax ? (void*)(block_max + (int64_t)tt * nbw) : (void*)scores,
                                                (short)0, (kBmax && real) ? nbw * 4 : 0, kRawBuf);
  }
  // scores of one query for one tile from its accumulators: ReLU, head weights (accumulator
  // row 4c + r of this lane is head 8c + 4g + r), head sum, causal mask, block maximum; one
  // lane stores each value, the others aim past the end of the buffer (no branches)
  auto finish = [&](int j, const f32x16& acc, int32_t k) {
    const float* wj = &s_w[wave * kMqQPW + j][4 * g];
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
    const float sc = masked_score(sum_halves((part[0] + part[1]) + (part[2] + part[3])), p < nv[j]);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_s[j], g ? kOut : 4 * p, 0, 0);
    if constexpr (kBmax)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(max8_lanes(sc)), rs_b[j],
                                            (g | (n & 7)) ? kOut : 4 * (p >> 3), 0, 0);
  };

  if (shared && max_nvis > 0) {
    // wave w decodes MFMA steps 2w and 2w+1 of every tile: lane (n, g) takes bytes
    // 8(w % 2) .. + 7 of plane g + 2(w / 2) of entry n (16 channels) and that group's E8M0 byte
    const int plane = g + 2 * (wave >> 1);
    struct Raw { uint2 w; uint32_t sc; };
    auto load = [&](int32_t k, Raw& r) {
      const int32_t p = k * kTile + n;
      const int64_t j = base0 + (p < max_nvis ? p : max_nvis - 1);  // past the visible rows: the last one
      r.w = *reinterpret_cast<const uint2*>(idx_cache + idx_plane_off(j, plane) + 8 * (wave & 1));
      r.sc = idx_cache[idx_scale_off(j) + plane];
    };
    auto stage = [&](const Raw& r, int buf) {
      const float x = e8m0_scale(r.sc);
      s_b[buf][2 * wave][lane] = cvt_fp4x8(r.w.x, x);
      s_b[buf][2 * wave + 1][lane] = cvt_fp4x8(r.w.y, x);
    };
    // tiles that some query of the block can see
    const int32_t tend = min(tile1, (max_nvis + kTile - 1) / kTile);
    // (loads past the visible rows read the last one, so they need no guard)
    Raw pipe[kMqDepth];
#pragma unroll
    for (int u = 0; u < kMqDepth; u++) load(tile0 + u, pipe[u]);
    if (tile0 < tend) {
      stage(pipe[0], 0);
      load(tile0 + kMqDepth, pipe[0]);
    }
    __syncthreads();
    for (int32_t k0 = tile0; k0 < tend; k0 += kMqDepth) {
#pragma unroll
      for (int u = 0; u < kMqDepth; u++) {
        const int32_t k = k0 + u;
        if (k < tend) {
          const int buf = (k - tile0) & 1;
          // stage the next tile into the other buffer, then refill its pipeline slot
          if (k + 1 < tend) {
            const int un = (u + 1) % kMqDepth;
            stage(pipe[un], buf ^ 1);
            load(k + 1 + kMqDepth, pipe[un]);
          }
          f32x16 acc0 = {}, acc1 = {};
#pragma unroll
          for (int s = 0; s < 8; s++) {
            const bf16x8 b = s_b[buf][s][lane];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], b, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], b, acc1, 0, 0, 0);
          }
          finish(0, acc0, k);
          finish(1, acc1, k);
          __syncthreads();  // buffer buf is free again; buf ^ 1 is complete
        }
      }
    }
    // tiles past every query's visible range
    for (int32_t k = max(tend, tile0); k < tile1; k++) {
#pragma unroll
      for (int j = 0; j < kMqQPW; j++) {
        const f32x16 z = {};
        finish(j, z, k);
      }
    }
    return;
  }
  // mixed sequences (or nothing visible): each query from its own rows, one tile at a time
  for (int j = 0; j < kMqQPW; j++) {
    const int t = tq[j];
    if (t >= n_q) continue;
    const int64_t base = s_base[wave * kMqQPW + j];
    for (int32_t k = tile0; k < tile1; k++) {
      const int32_t p = k * kTile + n;
      f32x16 acc = {};
      if (nv[j] > 0 && k * kTile < nv[j]) {
        const int64_t e = base + (p < nv[j] ? p : nv[j] - 1);  // past the visible rows: the last one
        const uint4 lo = *reinterpret_cast<const uint4*>(idx_cache + idx_plane_off(e, g));
        const uint4 hi = *reinterpret_cast<const uint4*>(idx_cache + idx_plane_off(e, 2 + g));
        const uint32_t scw = *reinterpret_cast<const uint32_t*>(idx_cache + idx_scale_off(e));
        const float x0 = e8m0_scale((scw >> (8 * g)) & 255u);
        const float x1 = e8m0_scale((scw >> (8 * g + 16)) & 255u);
        const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int s = 0; s < 8; s++)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][s], cvt_fp4x8(words[s], s < 4 ? x0 : x1), acc, 0, 0, 0);
      }
      finish(j, acc, k);
    }
  }
}

}  // namespace

int launch_index_score_mq(const uint16_t* q_idx_bf16, const float* head_w, const uint8_t* idx_cache,
                          const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                          float* block_max, void* stream) {
  const int32_t ntiles = (width + kTile - 1) / kTile;
  const int64_t gx = (ntiles + kMqTiles - 1) / kMqTiles, gy = (n_q + kMqQB - 1) / kMqQB;
  if (gx > 0x7FFFFFFF || gy > 65535) return CSA2_ERR_UNSUPPORTED;
  if (block_max != nullptr)
    hipLaunchKernelGGL(index_score_mq_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       (hipStream_t)stream, q_idx_bf16, head_w, idx_cache, q_base, q_nvis, n_q, width, scores,
                       block_max);
  else
    hipLaunchKernelGGL(index_score_mq_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       (hipStream_t)stream, q_idx_bf16, head_w, idx_cache, q_base, q_nvis, n_q, width, scores,
                       block_max);
  return check_launch();
}

}  // namespace csa2
