// index_tiles.hpp -- the tile loop of lightning-indexer scoring over the MXFP4 indexer-K
// cache, shared by the scoring kernels (gfx950).
//
// Computes s(t, j) = sum_h w[t,h] * max(0, q[t,h,:] . k^_j) ([ZB] "把 KV Cache 压缩推到极致"
// §3.3.2: indexer query and per-head weights produce the Top-K set; §2.3.4 / [DF]
// "CSA2 与每 token 890 字节" §4.7: a Full layer scores every visible entry and reduces
// blocks of 8 by max, a Reindex layer scores only its candidate pool).
//
// Design.  One wavefront owns one query and streams tiles of 32 entries.  The 32 heads
// x 128 dims contraction runs on v_mfma_f32_32x32x16_bf16 with the heads as the M
// dimension: the query sits in registers as eight A fragments for the whole scan, and
// each tile's B fragments are built in registers straight from the packed bytes: lane
// (n, g) loads planes g and 2 + g of entry n (32 payload bytes) plus its scale word, and
// v_cvt_scalef32_pk_bf16_fp4 turns two E2M1 nibbles and their E8M0 power-of-two scale
// into two exact bf16 values.  The K dimension is split the same way for both operands
// (lane group g and step s hold dims 32g + 8s .. + 7 for s < 4 and 64 + 32g + 8(s - 4) ..
// + 7 after), which leaves the dot products unchanged.  In the tile layout a wave's three
// loads of a tile are two contiguous 1 KB runs and one 128-byte run, each line fetched
// once, so the decode stream goes out non-temporal.  ReLU, the head weights and the head
// sum run on the accumulator registers; a 32-lane swap finishes the sum.  HBM traffic per
// entry is its 68 bytes plus 4.5 bytes of output.  The waves of the grid walk a query's
// tiles in grid-stride order, so the whole grid streams one front of the row at a time.
//
// Streaming.  All cache reads and score writes go through buffer resources whose sizes
// bound the row: loads past the end return zeros and stores past the end are dropped.
// That keeps the tile loop free of branches, so the compiler's memory-counter waits
// leave the younger tiles in flight, and lets duplicate lanes drop their stores by
// aiming past the end.  Measured on the 1M-context batch-4 decode, the stores are the
// costly part beyond the read stream (9.4 MB written against 143 MB read costs about
// as much as the MFMA and VALU work).
#pragma once
#include "index_common.hpp"

namespace csa2 {
namespace idx {

#ifndef CSA2_INDEX_DEPTH
#define CSA2_INDEX_DEPTH 3
#endif
constexpr int kDepth = CSA2_INDEX_DEPTH;  // tiles in flight per wave
constexpr int kRawBuf = 0x00020000;        // buffer descriptor word 3: raw 32-bit dwords

// Which slots of each row a call writes.  kOlderSlots and kNewestSlots split a Full-mode
// row at the tile of 32 slots that holds the newest visible entry (slot min(nvis, width)
// - 1, so the tile holds the newest block of 8 whole): kOlderSlots visits every other tile
// and reads none of that tile's entries, so an append may write the newest entry while it
// runs; kNewestSlots visits that tile alone and takes the entry at slot nvis - 1 from
// fresh_row, the 68-byte row its caller has just packed.  Together they write exactly what
// kAllSlots writes, with the same arithmetic per slot.
enum : int { kAllSlots = 0, kOlderSlots = 1, kNewestSlots = 2 };

// ---- the per-tile arithmetic of the bf16 query, in pieces that the selection's
// re-scoring of single entries calls too (the same operations in the same order give the
// same bits): lane (n, g) of a wave works on entry n of a 32-entry tile, dims 64g .. 64g + 63.

// the query fragments of lane (n, g) (head n, dims 32g + 8s .. + 7 for steps s < 4 and
// 64 + 32g + 8(s - 4) .. + 7 after: eight bf16x8 A fragments) and the head weights of the
// accumulator rows it holds (row 8(r/4) + 4g + r%4)
__device__ __forceinline__ void load_query_bf16(const uint16_t* __restrict__ q, const float* __restrict__ head_w,
                                                int t, int n, int g, bf16x8 (&a)[8], float (&wr)[16]) {
  const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)t * kIdxHeads + n) * kIdxDim + 32 * g);
#pragma unroll
  for (int s = 0; s < 8; s++) a[s] = __builtin_bit_cast(bf16x8, qp[s < 4 ? s : s + 4]);
  typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  const f32x4_a4* wp = reinterpret_cast<const f32x4_a4*>(head_w + (int64_t)t * kIdxHeads);
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const f32x4_a4 v = wp[2 * c + g];  // rows 8c + 4g .. 8c + 4g + 3
#pragma unroll
    for (int r = 0; r < 4; r++) wr[4 * c + r] = v[r];
  }
}

// q . k for the tile on v_mfma_f32_32x32x16_bf16: the entry's FP4 codes become exact bf16
// B fragments with their E8M0 scale (v_cvt_scalef32_pk_bf16_fp4)
__device__ __forceinline__ f32x16 mfma_bf16_tile(const bf16x8 (&a)[8], const RawTile& cur, int g) {
  f32x16 acc = {};
  const float x0 = e8m0_scale((cur.sc >> (8 * g)) & 255u);       // group g
  const float x1 = e8m0_scale((cur.sc >> (8 * g + 16)) & 255u);  // group 2 + g
  const uint32_t words[8] = {cur.lo[0], cur.lo[1], cur.lo[2], cur.lo[3], cur.hi[0], cur.hi[1], cur.hi[2], cur.hi[3]};
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const bf16x8 b = cvt_fp4x8(words[s], s < 4 ? x0 : x1);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b, acc, 0, 0, 0);
  }
  return acc;
}

// ReLU, head weight and the sum over the 32 heads of the tile's accumulators (four short
// chains over this lane's 16 heads, then the other lane half's): both halves of the wave
// end with entry n's score, or -inf for an invalid slot
__device__ __forceinline__ float head_sum(const f32x16& acc, const float (&wr)[16], bool valid) {
  float part[4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    part[c] = wr[4 * c] * relu(acc[4 * c]);
#pragma unroll
    for (int r = 1; r < 4; r++) part[c] = __builtin_fmaf(wr[4 * c + r], relu(acc[4 * c + r]), part[c]);
  }
  return masked_score(sum_halves((part[0] + part[1]) + (part[2] + part[3])), valid);
}

// kPool: Reindex layers score their candidate pool (entry j of slot p is block
// pool_blocks[p / 8] * 8 + p % 8); Full layers score entries 0 .. width-1 directly.
// kFp4Q: the indexer query arrives in MXFP4 (each head vector a 68-byte record like an
// indexer-K entry, [ZB] §2.4.4: the indexer Q and K are both trained for FP4), and the
// contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands' E2M1 codes and
// E8M0 scales fed to the instruction as stored: two MFMAs per tile, no conversions.
// kMeans: the rows scored are HISA's block means (one per 8 entries); q_nvis counts
// entries and the row's visible means are ceil(q_nvis[t] / 8).
// The wave is tile `first` of the grid-stride order with stride `tstride` (wave-uniform).
// kScores = false leaves the score row unwritten (block maxima only; scores may be NULL).
// lhist (kClaim, LDS) / ghist (kNewestSlots, global): when given, each older block maximum
// written (every block of the row but the one holding entry min(nvis, width) - 1) is also
// counted in bin order_key(max) >> kSelBinShift, as the selection's first pass counts it.
// kClaim: `first` and `tstride` describe the workgroup's tiles in groups of 4 consecutive
// tiles (groups first, first + tstride, ...), and its waves claim c = 0, 1, ... from the LDS
// counter *claim (zero before the first claim): claim c is tile 4 (first + (c / 4) tstride) +
// c % 4.  A wave that the SIMD serves more often scans more tiles (waves sharing a SIMD are
// issued oldest first), and the 4 block maxima of a group (one 16-byte store each) fill a
// 64-byte line from one workgroup, so one L2 writes the line back whole.
template <bool kPool, bool kFp4Q, int kPart, bool kMeans = false, bool kScores = true, bool kClaim = false>
__device__ __forceinline__ void score_tiles(
    const void* __restrict__ q_in, const float* __restrict__ head_w,
    const uint8_t* __restrict__ idx_cache, const int64_t* __restrict__ q_base,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M,
    int32_t width, float* __restrict__ scores, float* __restrict__ block_max, int t, int32_t first,
    int32_t tstride, const uint8_t* fresh_row = nullptr, const uint8_t* q_rec = nullptr,
    uint32_t* claim = nullptr, uint32_t* lhist = nullptr, uint32_t* ghist = nullptr) {
  static_assert(!kPool || kPart == kAllSlots, "a candidate pool is scored whole");
  static_assert(!kClaim || (!kPool && kPart != kNewestSlots), "claimed tiles: a Full row's older tiles");
  // tiles in flight per wave: the newest-tile part visits one tile
  constexpr int kPipe = kPart == kNewestSlots ? 1 : kDepth;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;
  const int32_t nvis_in = q_nvis[t];
  const int32_t nvis = kMeans ? (nvis_in > 0 ? (nvis_in - 1) / kBlock + 1 : 0) : nvis_in;
  const int64_t base = q_base[t];
  const int32_t ntiles = (width + kTile - 1) / kTile;
  // the tile of 32 slots that holds the newest visible entry, or -1 when nothing is visible
  const int32_t t_new = nvis > 0 ? (min(nvis, width) - 1) / kTile : -1;
  // the tiles this call visits, walked in grid-stride order: every tile (kOlderSlots passes
  // over t_new without reading or writing it), or t_new alone (all wave-uniform)
  const int32_t n_list = kPart == kNewestSlots ? (t_new >= 0 ? 1 : 0) : ntiles;
  // grid-stride tile order: at any moment the grid streams one front of the row
  const int32_t nt = first < n_list ? (n_list - first + tstride - 1) / tstride : 0;  // this wave's tiles
  auto tile_of = [&](int32_t k) -> int32_t {
    if constexpr (kPart == kNewestSlots) return t_new;
    else return first + k * tstride;
  };
  // kOlderSlots: tile k of this wave is the newest tile, which the call leaves alone
  auto dead = [&](int32_t k) -> bool {
    if constexpr (kPart == kOlderSlots) return first + k * tstride == t_new;
    else return false;
  };
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  float* srow = scores + (int64_t)t * width;

  // kClaim: tile of the workgroup's claim c (increasing with c)
  auto claim_tile_of = [&](int32_t c) -> int32_t { return 4 * (first + (c >> 2) * tstride) + (c & 3); };
  if (nvis <= 0) {  // nothing visible: the row is all -inf (claimed tiles: the waves split the list statically)
    const int32_t k_begin = kClaim ? (int32_t)(threadIdx.x >> 6) : 0;
    const int32_t k_step = kClaim ? (int32_t)(blockDim.x >> 6) : 1;
    for (int32_t k = k_begin; kClaim ? claim_tile_of(k) < n_list : k < nt; k += k_step) {
      const int32_t p = (kClaim ? claim_tile_of(k) : tile_of(k)) * kTile + n;  // (nothing visible: no newest tile)
      if (kScores && g == 0 && p < width) srow[p] = -__builtin_inff();
      if (block_max != nullptr && g == 0 && (n & 7) == 0 && p < width)
        block_max[(int64_t)t * nbw + (p >> 3)] = -__builtin_inff();
    }
    return;
  }

  // the query (head n, dims 64g .. 64g + 63: eight bf16x8 A fragments, or for an MXFP4
  // query two 32-code fragments and the head's scale word) and the head weight of each
  // accumulator row this lane holds (row 8(r/4) + 4g + r%4), loaded ahead of the first
  // cache tiles (below)
  bf16x8 a[8];
  fp4x32 qa[2];
  uint32_t qsc = 0;
  float wr[16];

  // Buffer resources bound the tiles of the sequence's visible entries, the score row and
  // the block-max row (empty when block_max is NULL): loads past the end return zeros and
  // stores past the end are dropped,
  // so the streaming loop below needs no branches (and the compiler's memory-counter
  // waits stay exact).  Offsets are 32-bit: the host limits width to 2^23 entries.
  const int32_t nv = min(nvis, kMaxIndexWidth);  // rows past 2^23 are never addressed
  int32_t rel0;  // the sequence's first entry, counted from the resource's first tile
  const __amdgpu_buffer_rsrc_t rs_cache = idx_rsrc(idx_cache, base, nv, rel0);
  const __amdgpu_buffer_rsrc_t rs_score = __builtin_amdgcn_make_buffer_rsrc(srow, (short)0, width * 4, kRawBuf);
  const __amdgpu_buffer_rsrc_t rs_bmax = __builtin_amdgcn_make_buffer_rsrc(
      block_max != nullptr ? (void*)(block_max + (int64_t)t * nbw) : (void*)srow, (short)0,
      block_max != nullptr ? nbw * 4 : 0, kRawBuf);
  const __amdgpu_buffer_rsrc_t rs_pool = __builtin_amdgcn_make_buffer_rsrc(
      kPool ? (void*)(pool_blocks + (int64_t)t * M) : (void*)srow, (short)0, kPool ? M * 4 : 0, kRawBuf);
  constexpr int32_t kOut = 1 << 30;  // a byte offset past every buffer's end

  // this lane's entry of tile k, counted from the resource's first tile (-1 when the slot is
  // empty: its loads read past the end and return zeros)
  auto row_off = [&](int32_t k, bool& valid) -> int32_t {
    const int32_t p = tile_of(k) * kTile + n;
    int32_t j;
    if constexpr (kPool) {
      const int32_t b = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs_pool, 4 * (p >> 3), 0, 0);
      const int64_t jj = (int64_t)b * kBlock + (p & 7);
      valid = (p >> 3) < M && b >= 0 && jj < nv;
      j = (int32_t)jj;
    } else {
      j = p;
      valid = p < nv && !dead(k);
    }
    return valid ? rel0 + j : -1;
  };
  // a Full row streams every tile once (non-temporal loads); a candidate pool gathers blocks
  // whose tiles may share scale lines
  constexpr int kAux = kPool ? 0 : kLoadStream;
  // A Full row's tiles (not a pool, not the single newest tile) put lane (n, g)'s bytes at the
  // same place in every tile, so each load and store takes a per-lane offset fixed for the
  // whole scan plus one wave-uniform offset per tile (the buffer instructions' scalar
  // offset): the address arithmetic stays off the vector ALU.
  constexpr bool kFast = !kPool && kPart != kNewestSlots;
  const int32_t e_lane = rel0 + n;  // entry slot n of tile 0, from the resource's first tile (< 63)
  const int32_t vo_plane = (e_lane >> 5) * kIdxTileBytes + kIdxPlaneBytes * g + 16 * (e_lane & 31);
  const int32_t vo_scale = (e_lane >> 5) * kIdxTileBytes + kIdxScaleOff + 4 * (e_lane & 31);
  const int32_t vo_score = g ? kOut : 4 * n;                   // one lane per score,
  const int32_t vo_bmax = (g | (n & 7)) ? kOut : 4 * (n >> 3);  // one per block maximum
  // a Full row's older tile T (wave-uniform; T < 0: no tile, its loads return zeros)
  auto load_tile = [&](int32_t T, RawTile& r) {
    const int32_t left = (T < 0 || (kPart == kOlderSlots && T == t_new)) ? 0 : nv - T * kTile;  // visible slots
    r.valid = n < left;
    const int32_t soff = T < 0 ? 0 : T * kIdxTileBytes;
    const int32_t vp = r.valid ? vo_plane : kOut, vs = r.valid ? vo_scale : kOut;
    r.lo = __builtin_bit_cast(u32x4_a4, __builtin_amdgcn_raw_buffer_load_b128(rs_cache, vp, soff, kAux));
    r.hi = __builtin_bit_cast(u32x4_a4,
                              __builtin_amdgcn_raw_buffer_load_b128(rs_cache, vp, soff + 2 * kIdxPlaneBytes, kAux));
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(rs_cache, vs, soff, kAux);
  };
  auto load = [&](int32_t k, RawTile& r) {
    if constexpr (kFast) {
      const int32_t T = tile_of(k);                        // wave-uniform
      const int32_t left = dead(k) ? 0 : nv - T * kTile;  // visible slots of the tile (may be <= 0)
      r.valid = n < left;
      const int32_t soff = T * kIdxTileBytes;
      const int32_t vp = r.valid ? vo_plane : kOut, vs = r.valid ? vo_scale : kOut;
      r.lo = __builtin_bit_cast(u32x4_a4, __builtin_amdgcn_raw_buffer_load_b128(rs_cache, vp, soff, kAux));
      r.hi = __builtin_bit_cast(u32x4_a4,
                                __builtin_amdgcn_raw_buffer_load_b128(rs_cache, vp, soff + 2 * kIdxPlaneBytes, kAux));
      r.sc = __builtin_amdgcn_raw_buffer_load_b32(rs_cache, vs, soff, kAux);
      return;
    }
    int32_t e = row_off(k, r.valid);
    // kNewestSlots: the entry at slot nvis - 1 was packed by this workgroup, which holds its
    // record in fresh_row; it is taken from there and not read back from the cache
    bool fresh = false;
    if constexpr (kPart == kNewestSlots) {
      fresh = tile_of(k) * kTile + n == nvis - 1;
      if (fresh) e = -1;
    }
    load_entry_share<kAux>(rs_cache, e, g, r);
    if constexpr (kPart == kNewestSlots) {
      if (fresh) load_record_share(fresh_row, g, r);
    }
  };
  // the scores of a Full row's older tile T >= 0 (the newest tile's stores are dropped)
  auto process_tile = [&](const RawTile& cur, int32_t T) {
    f32x16 acc;
    if constexpr (kFp4Q) {
      acc = mfma_fp4_tile(qa, qsc, cur.lo, cur.hi, cur.sc >> (8 * g), f32x16{});
    } else {
      acc = mfma_bf16_tile(a, cur, g);
    }
    const float sc = head_sum(acc, wr, cur.valid);
    const bool drop = kPart == kOlderSlots && T == t_new;  // wave-uniform
    if constexpr (kScores)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_score, vo_score, drop ? kOut : T * (4 * kTile), 0);
    const float bmx = max8_lanes(sc);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bmx), rs_bmax, vo_bmax, drop ? kOut : T * (4 * kTile / kBlock),
                                          0);
    // every visible block of an older tile is an older block (the newest is in tile t_new)
    if (lhist != nullptr && !drop && (g | (n & 7)) == 0 && T * kTile + n < nv)
      __hip_atomic_fetch_add(&lhist[order_key(bmx) >> kSelBinShift], 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto process = [&](const RawTile& cur, int32_t k) {
    f32x16 acc;
    if constexpr (kFp4Q) {
      acc = mfma_fp4_tile(qa, qsc, cur.lo, cur.hi, cur.sc >> (8 * g), f32x16{});
    } else {
      acc = mfma_bf16_tile(a, cur, g);
    }
    const float sc = head_sum(acc, wr, cur.valid);
    // both lane halves hold the entry's score and all 8 lanes of a block its maximum; one
    // lane writes each value and the others aim past the buffer's end, so their stores
    // are dropped without a branch (as are slots past the row's end)
    const bool drop = dead(k);  // wave-uniform
    if constexpr (kFast) {
      const int32_t T = tile_of(k);
      if constexpr (kScores)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_score, vo_score, drop ? kOut : T * (4 * kTile), 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(max8_lanes(sc)), rs_bmax, vo_bmax,
                                            drop ? kOut : T * (4 * kTile / kBlock), 0);
      return;
    }
    const int32_t p = tile_of(k) * kTile + n;
    if constexpr (kScores)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs_score, (g || drop) ? kOut : 4 * p, 0, 0);
    const float bmx = max8_lanes(sc);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bmx), rs_bmax, ((g | (n & 7)) || drop) ? kOut : 4 * (p >> 3),
                                          0, 0);
    if constexpr (kPart == kNewestSlots) {  // the newest tile's older blocks
      const int32_t nw = min(nvis, width);
      if (ghist != nullptr && (g | (n & 7)) == 0 && p < nw && (p >> 3) < (nw - 1) >> 3)
        atomicAdd(&ghist[order_key(bmx) >> kSelBinShift], 1u);
    }
  };

  // The query and head weights are loaded first, then the first kPipe tiles, and a wait
  // for all but the tiles' loads completes the query before the loop.  The compiler then
  // knows the query registers are ready inside the loop; otherwise it re-checks them on
  // every pass with a wait that drains this wave's tiles in flight (loads complete in order).
  {
    if constexpr (kFp4Q) {
      // q_rec: the query's 32 records, already packed by the caller (in LDS)
      load_fp4_query(q_rec != nullptr ? q_rec + n * kIdxBytes
                                      : static_cast<const uint8_t*>(q_in) + ((int64_t)t * kIdxHeads + n) * kIdxBytes,
                     g, qa, qsc);
      typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
      const f32x4_a4* wp = reinterpret_cast<const f32x4_a4*>(head_w + (int64_t)t * kIdxHeads);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const f32x4_a4 v = wp[2 * c + g];  // rows 8c + 4g .. 8c + 4g + 3
#pragma unroll
        for (int r = 0; r < 4; r++) wr[4 * c + r] = v[r];
      }
    } else {
      load_query_bf16(static_cast<const uint16_t*>(q_in), head_w, t, n, g, a, wr);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // software pipeline: kPipe - 1 tiles of this wave are in flight while one is processed.
  // Full groups of kPipe tiles stream through the loop; loads past the wave's last tile
  // return zeros and are never processed; the last partial group is finished after it.
  // (the scheduling barriers keep the tiles' loads in tile order, so each tile's wait
  // counts only older loads)
  RawTile pipe[kPipe];
  if constexpr (kClaim) {
    // a wave's claims only grow, and so do their tiles: its first claim past the row's end
    // ends its loop
    auto claim_tile = [&]() -> int32_t {
      uint32_t c = 0;
      if (lane == 0) c = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      c = __builtin_amdgcn_readfirstlane(c);
      const int32_t T = c < (uint32_t)n_list ? claim_tile_of((int32_t)c) : n_list;  // c < n_list: no overflow
      return T < n_list ? T : -1;
    };
    int32_t T[kPipe];
#pragma unroll
    for (int u = 0; u < kPipe; u++) {
      T[u] = claim_tile();
      load_tile(T[u], pipe[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPipe * 3));
    for (;;) {
#pragma unroll
      for (int u = 0; u < kPipe; u++) {
        if (T[u] < 0) return;  // wave-uniform: every later claim is past the end too
        process_tile(pipe[u], T[u]);
        __builtin_amdgcn_s_setprio(2);
        T[u] = claim_tile();
        load_tile(T[u], pipe[u]);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (kFp4Q) __builtin_amdgcn_sched_barrier(0);  // tiles' loads in tile order
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPipe; u++) {
    load(u, pipe[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Full mode issues three loads per tile; a pool tile's block-id load precedes its three
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPipe * (kPool ? 4 : 3)));
  int32_t k0 = 0;
  for (; k0 + kPipe <= nt; k0 += kPipe) {
#pragma unroll
    for (int u = 0; u < kPipe; u++) {
      process(pipe[u], k0 + u);
      // the next tile's loads issue at raised wave priority, so they leave ahead of the other
      // waves' compute on this SIMD (33.1 -> 32.8 us on the 1M-context batch-4 scan)
      __builtin_amdgcn_s_setprio(2);
      load(k0 + u + kPipe, pipe[u]);  // reuses this tile's registers, so none are copied
      __builtin_amdgcn_s_setprio(0);
      // the MXFP4-query body leaves the scheduler room to interleave different tiles' loads,
      // which would make each tile's wait cover younger tiles too: keep them in tile order
      if constexpr (kFp4Q) __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < kPipe - 1; u++)
    if (k0 + u < nt) process(pipe[u], k0 + u);
}

}  // namespace idx
}  // namespace csa2
