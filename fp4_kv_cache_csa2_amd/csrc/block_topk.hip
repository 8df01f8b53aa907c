// block_topk.hip -- hierarchical sparse selection for gfx950: block max -> top-M block
// pool -> Top-K inside the pool.
//
// Follows [ZB] "把 KV Cache 压缩推到极致" §2.3.4 (pad with -inf, max over blocks of 8, the
// newest visible block forced to +inf, the selected blocks expanded and truncated to the
// visible width) and [DF] "CSA2 与每 token 890 字节" §4.7 (g_r, TopM over blocks, pool =
// union of the selected blocks, |P_t| <= 2048 x 8).  Ties go to the lower index.
//
// Design.  One 1024-thread workgroup per query.  Scores become order-preserving uint32
// keys (NaN -> -inf).  A k-largest selection is an exact 4-pass MSB radix select (8-bit
// digits, LDS histogram) that yields the threshold key tau and how many keys equal to
// tau are still needed, followed by an order-preserving compaction: every wave owns a
// contiguous segment, counts its survivors with ballots, the wave offsets are scanned
// once, and the second pass writes the survivors in ascending index order.  Keys of up
// to 16384 candidates live in LDS; longer block-key rows are read from global memory
// (L2-resident, written by the indexer kernel just before).
#include "csa2_device.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 16384;

struct SelShared {
  uint32_t keys[kLdsKeys];   // LDS-resident keys (blocks or candidates)
  int32_t pool[kMaxPool];    // selected block ids, ascending
  int32_t sel[kMaxTopK];     // selected candidate indices, ascending
  uint32_t hist[256];
  int32_t wave_a[kWaves];
  int32_t wave_b[kWaves];
  uint32_t prefix;
  int32_t remain;
  int32_t eq_total;
  int32_t count;
};

// Threshold of the k largest keys among keys[0..n): returns tau; need_eq = number of
// keys equal to tau that belong to the selection (lowest indices first); eq_total = how
// many keys equal tau.  Requires 1 <= k <= n.
__device__ void radix_threshold(const uint32_t* keys, int n, int k, SelShared& sh, uint32_t& tau,
                                int& need_eq, int& eq_total) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.prefix = 0;
    sh.remain = k;
  }
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending); exclusive prefix over lanes
      const int l = tid;
      uint32_t c[4];
      uint32_t local = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        c[q] = sh.hist[255 - 4 * l - q];
        local += c[q];
      }
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (l >= o) incl += y;
      }
      uint32_t above = incl - local;
      const uint32_t rem = (uint32_t)sh.remain;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if (above < rem && rem <= above + c[q]) {
          const uint32_t d = 255u - 4u * l - q;
          sh.prefix = prefix | (d << shift);
          sh.remain = (int)(rem - above);
          sh.eq_total = (int)c[q];
        }
        above += c[q];
      }
    }
    __syncthreads();
    mask |= 255u << shift;
  }
  tau = sh.prefix;
  need_eq = sh.remain;
  eq_total = sh.eq_total;
  __syncthreads();
}

// Ordered compaction: writes the indices i (ascending) with key > tau, or key == tau
// among the first need_eq such keys, never a zero key.  out_ids may be LDS or global.
// Returns the number written (also in sh.count).
__device__ int compact_selected(const uint32_t* keys, int n, uint32_t tau, int need_eq, int eq_total,
                                SelShared& sh, int32_t* out_ids) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (n + kWaves - 1) / kWaves;
  const int lo = wave * seg, hi = min(n, lo + seg);
  const bool all_eq = (need_eq >= eq_total);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // pass A: per-wave counts of keys > tau and keys == tau
  int gt = 0, eq = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi ? keys[i] : 0u;
    const bool ok = i < hi && key != 0u;
    gt += __popcll(__ballot(ok && key > tau));
    eq += __popcll(__ballot(ok && key == tau));
  }
  if (lane == 0) {
    sh.wave_a[wave] = gt;
    sh.wave_b[wave] = eq;
  }
  __syncthreads();
  // exclusive offsets of this wave among equal keys and among survivors
  int eq_acc = 0, sel_acc = 0, eq_off = 0, sel_off = 0;
  for (int w = 0; w < kWaves; w++) {
    if (w == wave) {
      eq_off = eq_acc;
      sel_off = sel_acc;
    }
    const int e_w = sh.wave_b[w];
    const int take_eq = all_eq ? e_w : max(0, min(e_w, need_eq - eq_acc));
    eq_acc += e_w;
    sel_acc += sh.wave_a[w] + take_eq;
  }
  const int total = sel_acc;
  __syncthreads();
  // pass B: write survivors in index order
  int run_eq = eq_off, run_sel = sel_off;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi ? keys[i] : 0u;
    const bool ok = i < hi && key != 0u;
    const bool is_eq = ok && key == tau;
    const uint64_t eqb = __ballot(is_eq);
    const int my_eq = run_eq + __popcll(eqb & lt_mask);
    const bool sel = ok && (key > tau || (is_eq && (all_eq || my_eq < need_eq)));
    const uint64_t selb = __ballot(sel);
    if (sel) out_ids[run_sel + __popcll(selb & lt_mask)] = i;
    run_eq += __popcll(eqb);
    run_sel += __popcll(selb);
  }
  if (tid == 0) sh.count = total;
  __syncthreads();
  return total;
}

// k largest of keys[0..n) (zero keys excluded), ascending indices into out_ids.
__device__ int select_topk(const uint32_t* keys, int n, int k, SelShared& sh, int32_t* out_ids) {
  if (n <= 0) return 0;
  const int kk = min(k, n);
  uint32_t tau;
  int need_eq, eq_total;
  radix_threshold(keys, n, kk, sh, tau, need_eq, eq_total);
  if (tau == 0u) {  // fewer non-zero keys than k: take every non-zero key
    need_eq = 0;
    eq_total = 1;
  }
  return compact_selected(keys, n, tau, need_eq, eq_total, sh, out_ids);
}

__global__ __launch_bounds__(kThreads) void block_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ block_max, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M,
    int32_t K, int32_t* __restrict__ pool_out, int32_t* __restrict__ topk_out,
    uint32_t* __restrict__ ws_keys) {
  __shared__ SelShared sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = scores + (int64_t)t * width;
  int32_t* tk = topk_out + (int64_t)t * K;
  int32_t npool;

  if (pool_blocks == nullptr) {
    const int32_t n = min(q_nvis[t], width);
    const int32_t nb = n > 0 ? (n + kBlock - 1) / kBlock : 0;
    const int32_t nbw = (width + kBlock - 1) / kBlock;
    // block keys: max over the visible positions of each block, newest block forced to +inf
    uint32_t* bkeys = nb <= kLdsKeys ? sh.keys : ws_keys + (int64_t)t * nbw;
    for (int r = tid; r < nb; r += kThreads) {
      uint32_t key;
      if (r == nb - 1) {
        key = 0xFFFFFFFFu;
      } else if (block_max != nullptr) {
        key = order_key(block_max[(int64_t)t * nbw + r]);
      } else {
        float mx = -__builtin_inff();
        for (int o = 0; o < kBlock; o++) {
          const float v = row[r * kBlock + o];
          mx = (v > mx) ? v : mx;  // NaN never wins, so it ranks as -inf
        }
        key = order_key(mx);
      }
      bkeys[r] = key;
    }
    __syncthreads();
    if (nb <= M) {
      for (int r = tid; r < nb; r += kThreads) sh.pool[r] = r;
      npool = nb;
      __syncthreads();
    } else {
      npool = select_topk(bkeys, nb, M, sh, sh.pool);
    }
    if (pool_out != nullptr) {
      int32_t* po = pool_out + (int64_t)t * M;
      for (int s = tid; s < M; s += kThreads) po[s] = s < npool ? sh.pool[s] : -1;
    }
    // candidates: the visible positions of the pool blocks, in ascending entry order
    const int nc = npool * kBlock;
    for (int c = tid; c < nc; c += kThreads) {
      const int32_t j = sh.pool[c >> 3] * kBlock + (c & 7);
      sh.keys[c] = j < n ? order_key(row[j]) : 0u;
    }
    __syncthreads();
    const int cnt = select_topk(sh.keys, nc, K, sh, sh.sel);
    // map candidate indices to entry ids; ascending order is preserved
    for (int i = tid; i < K; i += kThreads) {
      const int c = i < cnt ? sh.sel[i] : -1;
      tk[i] = c < 0 ? -1 : sh.pool[c >> 3] * kBlock + (c & 7);
    }
  } else {
    const int32_t nvis = q_nvis[t];
    const int32_t* pb = pool_blocks + (int64_t)t * M;
    const int nc = M * kBlock;
    for (int c = tid; c < nc; c += kThreads) {
      const int32_t b = pb[c >> 3];
      const int64_t j = (int64_t)b * kBlock + (c & 7);
      sh.keys[c] = (b >= 0 && j < nvis) ? order_key(row[c]) : 0u;
    }
    __syncthreads();
    const int cnt = select_topk(sh.keys, nc, K, sh, sh.sel);
    for (int i = tid; i < K; i += kThreads) {
      const int c = i < cnt ? sh.sel[i] : -1;
      tk[i] = c < 0 ? -1 : pb[c >> 3] * kBlock + (c & 7);
    }
  }
}

}  // namespace
}  // namespace csa2

extern "C" size_t csa2_block_topk_workspace(int32_t n_q, int32_t width, int32_t M, int32_t K) {
  (void)M;
  (void)K;
  if (n_q <= 0 || width <= 0) return 0;
  const int64_t nbw = (width + csa2::kBlock - 1) / csa2::kBlock;
  if (nbw <= csa2::kLdsKeys) return 0;
  return (size_t)n_q * (size_t)nbw * sizeof(uint32_t);
}

extern "C" int csa2_block_topk(const float* scores, const float* block_max, int32_t n_q,
                               int32_t width, const int32_t* q_nvis, const int32_t* pool_blocks,
                               int32_t block, int32_t M, int32_t K, int32_t* pool_out,
                               int32_t* topk_out, void* workspace, size_t ws_bytes, void* stream) {
  using namespace csa2;
  if (n_q < 0 || width < 0) return CSA2_ERR_INVALID_ARG;
  if (block != kBlock || M < 1 || M > kMaxPool || K < 1 || K > kMaxTopK) return CSA2_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!scores || !q_nvis || !topk_out) return CSA2_ERR_INVALID_ARG;
  if (pool_blocks && (pool_out || block_max || (int64_t)width != 8LL * M)) return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(block_max) |
       reinterpret_cast<uintptr_t>(topk_out) | reinterpret_cast<uintptr_t>(pool_out)) & 3)
    return CSA2_ERR_INVALID_ARG;
  const size_t need = pool_blocks ? 0 : csa2_block_topk_workspace(n_q, width, M, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  hipLaunchKernelGGL(block_topk_kernel, dim3(n_q), dim3(kThreads), 0, (hipStream_t)stream, scores,
                     block_max, width, q_nvis, pool_blocks, M, K, pool_out, topk_out,
                     (uint32_t*)workspace);
  return check_launch();
}
