// block_topk.hip -- hierarchical sparse selection for gfx950: block max -> top-M block
// pool -> Top-K inside the pool.
//
// Follows [ZB] "把 KV Cache 压缩推到极致" §2.3.4 (pad with -inf, max over blocks of 8, the
// newest visible block forced to +inf, the selected blocks expanded and truncated to the
// visible width) and [DF] "CSA2 与每 token 890 字节" §4.7 (g_r, TopM over blocks, pool =
// union of the selected blocks, |P_t| <= 2048 x 8).  Ties go to the lower index, NaN
// ranks as -inf, outputs are ascending and padded with -1.
//
// Design (three kernels, launched back to back on the caller's stream):
//   K1 hist     many workgroups per query build a 4096-bin histogram of the ranking keys
//               (top 12 bits of an order-preserving uint32 map of the fp32 value) in LDS
//               and add it into a per-query histogram in the workspace.
//   K2 collect  the same grid finds the bin that holds the k-th largest key and writes,
//               in ascending order, the ids of every key in that bin or above into one
//               segment per workgroup: a short ordered list that is a superset of the
//               selection.
//   K3 finalize one 1024-thread workgroup per query runs an exact 4-pass radix select on
//               that list (ties by lower id), appends the forced newest block, writes the
//               pool, and takes the Top-K among the entries of the K+1 highest pool blocks:
//               every global Top-K member's block ranks within the first K+1 blocks, so
//               this is the Top-K of the pool and of the whole row.  K3 returns the
//               histogram to zero.  If the list overflows LDS (massive ties), K3 selects
//               straight from the full key row instead, with the same exact rules.
// The histogram region of the workspace must be zero before the first call; every call
// leaves it zero.
#include "csa2_device.hpp"

namespace csa2 {
namespace {

constexpr int kBins = 4096;        // 12-bit histogram digit
constexpr int kBinShift = 20;
constexpr int kSlice = 1024;       // keys per workgroup in K1 / K2
constexpr int kGThreads = 256;     // K1 / K2 workgroup size
constexpr int kFThreads = 1024;    // K3 workgroup size
constexpr int kFWaves = kFThreads / 64;
constexpr int kListCap = 12288;    // ordered candidate list held in LDS by K3
constexpr int kMaxG = 1024;        // workgroups per query row in K1 / K2 (rows up to 2^20 items)

// ------------------------------------------------------------------ shared helpers

// LDS histogram add; lanes of a wave that share a bin are merged (up to two bins) so a
// concentrated key distribution does not serialise on one LDS address.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin, bool active) {
  const int lane = __lane_id();
  uint64_t todo = __ballot(active);
#pragma unroll
  for (int it = 0; it < 2; it++) {
    if (todo == 0) break;
    const int leader = __ffsll((unsigned long long)todo) - 1;  // wave-uniform
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(active && bin == lb) & todo;
    if (lane == leader) atomicAdd(&h[lb], (uint32_t)__popcll(same));
    todo &= ~same;
  }
  if ((todo >> lane) & 1ull) atomicAdd(&h[bin], 1u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum of v over the threads of a workgroup of NT threads, in thread
// order; total receives the sum over all threads.  s_w holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; w++) {
    const int sw = s_w[w];
    off += (w < wave) ? sw : 0;
    tot += sw;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

struct SelScratch {
  uint32_t hist[2][256];  // double-buffered digit histogram
  int32_t wave_a[kFWaves];
  int32_t wave_b[kFWaves];
  uint32_t prefix;
  int32_t remain;
  int32_t eq_total;
  int32_t take_all;
};

// Exact selection by a 1024-thread workgroup: the k largest non-zero keys of key_at(0..n),
// ties to the lower index, written ascending to out[] (LDS or global).  Returns the count.
template <class F>
__device__ int block_select(F key_at, int n, int k, SelScratch& s, int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= 0 || k <= 0) return 0;
  const int kk = min(k, n);
  // ---- threshold: up to 4 passes of 8-bit digits from the most significant; zero keys
  // (non-candidates) are never counted
  if (tid == 0) {
    s.prefix = 0;
    s.remain = kk;
    s.eq_total = -1;
    s.take_all = 0;
  }
  if (tid < 256) s.hist[0][tid] = 0;
  uint32_t mask = 0;
  int buf = 0;
  for (int shift = 24; shift >= 0; shift -= 8, buf ^= 1) {
    __syncthreads();
    // stop once every key sharing the prefix is needed (or every key is taken)
    if (s.take_all || s.eq_total == s.remain) break;
    const uint32_t prefix = s.prefix;
    if (tid < 256) s.hist[buf ^ 1][tid] = 0;  // the next pass's buffer
    for (int base = 0; base < n; base += kFThreads) {
      const int i = base + tid;
      const uint32_t key = i < n ? key_at(i) : 0u;
      hist_add(s.hist[buf], (key >> shift) & 255u, key != 0u && (key & mask) == prefix);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t c[4], local = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        c[q] = s.hist[buf][255 - 4 * tid - q];
        local += c[q];
      }
      const uint32_t incl = wave_incl_scan(local);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      uint32_t above = incl - local;
      const uint32_t rem = (uint32_t)s.remain;
      if (shift == 24 && total <= rem) {
        if (tid == 0) s.take_all = 1;  // no more candidates than wanted
      } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if (above < rem && rem <= above + c[q]) {
            s.prefix = prefix | ((255u - 4u * tid - q) << shift);
            s.remain = (int)(rem - above);
            s.eq_total = (int)c[q];
          }
          above += c[q];
        }
      }
    }
    mask |= 255u << shift;
  }
  __syncthreads();
  // the selection: keys whose masked prefix is above tau, plus need_eq of those equal to it
  uint32_t tau = s.prefix;
  int need_eq = s.remain, eq_total = s.eq_total;
  if (s.take_all) {
    mask = 0u;
    tau = 0u;
    need_eq = n;
    eq_total = 0;
  }
  const bool all_eq = need_eq >= eq_total;
  // ---- ordered compaction: each wave owns a contiguous segment
  const int seg = (n + kFWaves - 1) / kFWaves;
  const int lo = min(n, wave * seg), hi = min(n, lo + seg);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int gt = 0, eq = 0;
  for (int b = lo; b < hi; b += 64) {
    const int i = b + lane;
    const uint32_t key = i < hi ? key_at(i) : 0u;
    gt += __popcll(__ballot(key != 0u && (key & mask) > tau));
    eq += __popcll(__ballot(key != 0u && (key & mask) == tau));
  }
  if (lane == 0) {
    s.wave_a[wave] = gt;
    s.wave_b[wave] = eq;
  }
  __syncthreads();
  // per-wave offsets among equal keys and among survivors, lanes 0..15 = waves 0..15
  const uint32_t e_l = lane < kFWaves ? (uint32_t)s.wave_b[lane] : 0u;
  const uint32_t e_incl = wave_incl_scan(e_l);
  const uint32_t e_before = e_incl - e_l;
  uint32_t take = e_l;
  if (!all_eq) {
    const int rest = need_eq - (int)e_before;
    take = (uint32_t)max(0, min((int)e_l, rest));
  }
  const uint32_t s_l = lane < kFWaves ? (uint32_t)s.wave_a[lane] + take : 0u;
  const uint32_t s_incl = wave_incl_scan(s_l);
  const int total = __builtin_amdgcn_readlane((int)s_incl, kFWaves - 1);
  const int eq_off = __builtin_amdgcn_readlane((int)e_before, wave);
  const int sel_off = __builtin_amdgcn_readlane((int)(s_incl - s_l), wave);
  int run_eq = eq_off, run_sel = sel_off;
  for (int b = lo; b < hi; b += 64) {
    const int i = b + lane;
    const uint32_t key = i < hi ? key_at(i) : 0u;
    const bool is_eq = key != 0u && (key & mask) == tau;
    const uint64_t eqb = __ballot(is_eq);
    const bool sel = key != 0u && ((key & mask) > tau || (is_eq && (all_eq || run_eq + __popcll(eqb & lt) < need_eq)));
    const uint64_t selb = __ballot(sel);
    if (sel) out[run_sel + __popcll(selb & lt)] = i;
    run_eq += __popcll(eqb);
    run_sel += __popcll(selb);
  }
  __syncthreads();
  return total;
}

// Per-query view of the selection problem shared by the three kernels.
struct Row {
  bool cand;
  const float* scores;  // row base
  const float* bm;      // block maxima row (full mode)
  const int32_t* pool;  // candidate-mode pool row
  int32_t n;            // visible positions
  int32_t nb;           // visible blocks (full mode)
  int32_t M, K;
  // number of ranking items handled by K1 / K2 and how many of them are selected
  __device__ int32_t items() const { return cand ? 8 * M : max(nb - 1, 0); }
  __device__ bool needs_hist() const { return cand ? true : nb > M; }
  __device__ uint32_t item_key(int32_t i) const {  // 0 = not a candidate
    if (cand) {
      const int32_t b = pool[i >> 3];
      const int64_t j = (int64_t)b * kBlock + (i & 7);
      return (b >= 0 && j < n) ? order_key(scores[i]) : 0u;
    }
    return order_key(bm[i]);  // blocks 0 .. nb-2 (the newest block is handled apart)
  }
};

__device__ __forceinline__ Row make_row(int t, bool cand, const float* scores, const float* bm, int32_t width,
                                        const int32_t* q_nvis, const int32_t* pool_blocks, int32_t M, int32_t K) {
  Row r;
  r.cand = cand;
  r.scores = scores + (int64_t)t * width;
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  r.bm = bm ? bm + (int64_t)t * nbw : nullptr;
  r.pool = cand ? pool_blocks + (int64_t)t * M : nullptr;
  r.M = M;
  r.K = K;
  if (cand) {
    r.n = q_nvis[t];
    r.nb = 0;
  } else {
    r.n = max(0, min(q_nvis[t], width));
    r.nb = (r.n + kBlock - 1) / kBlock;
  }
  return r;
}

// ------------------------------------------------------------------ K1: histogram

__global__ __launch_bounds__(kGThreads) void topk_hist_kernel(
    bool cand, const float* __restrict__ scores, const float* __restrict__ block_max, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K,
    uint32_t* __restrict__ ws_hist, float* __restrict__ ws_bm) {
  __shared__ uint32_t h[kBins];
  const int t = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  Row r = make_row(t, cand, scores, block_max ? block_max : ws_bm, width, q_nvis, pool_blocks, M, K);
  const int32_t lo = g * kSlice;
  if (!cand && block_max == nullptr) {
    // block maxima from the scores (NaN never wins a comparison, so it ranks as -inf)
    float* bmw = ws_bm + (int64_t)t * nbw;
    for (int32_t b = lo + tid; b < min(lo + kSlice, r.nb); b += kGThreads) {
      float mx = -__builtin_inff();
      for (int o = 0; o < kBlock; o++) {
        const int32_t j = b * kBlock + o;
        if (j < r.n) {
          const float v = r.scores[j];
          mx = v > mx ? v : mx;
        }
      }
      bmw[b] = mx;
    }
    __syncthreads();
  }
  if (!r.needs_hist()) return;
  const int32_t hi = min(lo + kSlice, r.items());
  if (lo >= hi) return;
  for (int b = tid; b < kBins; b += kGThreads) h[b] = 0;
  __syncthreads();
  for (int32_t base = lo; base < hi; base += kGThreads) {
    const int32_t i = base + tid;
    const uint32_t key = i < hi ? r.item_key(i) : 0u;
    hist_add(h, key >> kBinShift, key != 0u);
  }
  __syncthreads();
  uint32_t* gh = ws_hist + (int64_t)t * kBins;
  for (int b = tid; b < kBins; b += kGThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

// ------------------------------------------------------------------ K2: ordered collection

__global__ __launch_bounds__(kGThreads) void topk_collect_kernel(
    bool cand, const float* __restrict__ scores, const float* __restrict__ bm, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K,
    int32_t G, int32_t row_cap, const uint32_t* __restrict__ ws_hist, int32_t* __restrict__ ws_cnt,
    int32_t* __restrict__ ws_ids) {
  __shared__ int32_t s_wave[kGThreads / 64];
  __shared__ uint32_t s_b1;
  const int t = blockIdx.y, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Row r = make_row(t, cand, scores, bm, width, q_nvis, pool_blocks, M, K);
  int32_t* cnt = ws_cnt + (int64_t)t * G + g;
  if (!r.needs_hist()) {
    if (tid == 0) *cnt = 0;
    return;
  }
  // thread tid owns bins [16 tid, 16 tid + 16); find the bin holding the kk-th largest
  const uint32_t* gh = ws_hist + (int64_t)t * kBins;
  uint32_t hb[16], local = 0;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    hb[q] = gh[16 * tid + q];
    local += hb[q];
  }
  if (tid == 0) s_b1 = 0xFFFFFFFFu;
  int tot_i;
  const int before = block_excl_scan<kGThreads>((int)local, s_wave, tot_i);
  const uint32_t total = (uint32_t)tot_i;
  uint32_t above = total - (uint32_t)before - local;  // keys in bins above this thread's range
  const uint32_t kk = cand ? min((uint32_t)K, total) : (uint32_t)(M - 1);
  if (kk > 0) {
#pragma unroll
    for (int q = 15; q >= 0; q--) {
      if (above < kk && kk <= above + hb[q]) s_b1 = 16u * tid + q;
      above += hb[q];
    }
  }
  __syncthreads();
  const uint32_t b1 = s_b1;
  // ordered collection of this slice: wave w owns a quarter of the slice
  const int32_t lo = g * kSlice, hi = min(lo + kSlice, r.items());
  const int32_t q4 = kSlice / (kGThreads / 64);
  const int32_t wlo = min(hi, lo + wave * q4), whi = min(hi, wlo + q4);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t mine = 0;
  if (b1 != 0xFFFFFFFFu) {
    for (int32_t b = wlo; b < whi; b += 64) {
      const int32_t i = b + lane;
      const uint32_t key = i < whi ? r.item_key(i) : 0u;
      mine += __popcll(__ballot(key != 0u && (key >> kBinShift) >= b1));
    }
  }
  int32_t all;
  int32_t off = block_excl_scan<kGThreads>(lane == 0 ? mine : 0, s_wave, all);
  off = __shfl(off, 0);
  int32_t* seg = ws_ids + (int64_t)t * row_cap + (int64_t)g * kSlice;
  if (b1 != 0xFFFFFFFFu) {
    for (int32_t b = wlo; b < whi; b += 64) {
      const int32_t i = b + lane;
      const uint32_t key = i < whi ? r.item_key(i) : 0u;
      const bool f = key != 0u && (key >> kBinShift) >= b1;
      const uint64_t fb = __ballot(f);
      if (f) seg[off + __popcll(fb & lt)] = i;
      off += __popcll(fb);
    }
  }
  if (tid == 0) *cnt = all;
}

// ------------------------------------------------------------------ K3: exact finalize

struct FinShared {
  int32_t ids[kListCap];       // ordered candidate ids
  uint32_t keys[kListCap];     // their keys
  int32_t pool[kMaxPool];      // pool block ids, ascending
  int32_t sel[kMaxPool];       // selection indices
  int32_t seg_off[kMaxG + 1];
  int32_t scan[kFWaves];
  SelScratch s;
};

__global__ __launch_bounds__(kFThreads) void topk_final_kernel(
    bool cand, const float* __restrict__ scores, const float* __restrict__ bm, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K,
    int32_t G, int32_t row_cap, uint32_t* __restrict__ ws_hist, const int32_t* __restrict__ ws_cnt,
    const int32_t* __restrict__ ws_ids, int32_t* __restrict__ pool_out, int32_t* __restrict__ topk_out) {
  __shared__ FinShared sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  Row r = make_row(t, cand, scores, bm, width, q_nvis, pool_blocks, M, K);
  int32_t* tk = topk_out + (int64_t)t * K;

  // gather the ordered candidate list (the K2 segments, in workgroup order)
  int32_t total = 0;
  if (r.needs_hist()) {
    // segment offsets: a parallel scan of the G per-workgroup counts (G <= 1024)
    const int c = tid < G ? ws_cnt[(int64_t)t * G + tid] : 0;
    int all;
    const int off = block_excl_scan<kFThreads>(c, sh.scan, all);
    if (tid < G) sh.seg_off[tid] = off;
    if (tid == 0) sh.seg_off[G] = all;
    __syncthreads();
    total = sh.seg_off[G];
    if (total <= kListCap) {
      // every element finds its segment by binary search, so all loads are in flight at once
      const int32_t* rowids = ws_ids + (int64_t)t * row_cap;
      for (int e = tid; e < total; e += kFThreads) {
        int lo = 0, hi = G - 1;  // last segment whose offset is <= e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sh.seg_off[mid] <= e) lo = mid; else hi = mid - 1;
        }
        const int32_t id = rowids[(int64_t)lo * kSlice + (e - sh.seg_off[lo])];
        sh.ids[e] = id;
        sh.keys[e] = r.item_key(id);
      }
    }
    __syncthreads();
  }

  if (cand) {
    int cnt;
    if (total <= kListCap) {
      cnt = block_select([&](int i) { return sh.keys[i]; }, total, K, sh.s, sh.sel);
      for (int i = tid; i < cnt; i += kFThreads) sh.sel[i] = sh.ids[sh.sel[i]];
    } else {
      cnt = block_select([&](int i) { return r.item_key(i); }, r.items(), K, sh.s, sh.sel);
    }
    __syncthreads();
    for (int i = tid; i < K; i += kFThreads) {
      const int32_t p = i < cnt ? sh.sel[i] : -1;
      tk[i] = p < 0 ? -1 : r.pool[p >> 3] * kBlock + (p & 7);
    }
  } else {
    // ---- the pool: top M-1 of the older blocks plus the forced newest block
    int32_t npool = 0;
    if (r.nb > 0) {
      if (!r.needs_hist()) {
        for (int i = tid; i < r.nb - 1; i += kFThreads) sh.pool[i] = i;
        npool = r.nb - 1;
      } else if (total <= kListCap) {
        npool = block_select([&](int i) { return sh.keys[i]; }, total, M - 1, sh.s, sh.sel);
        for (int i = tid; i < npool; i += kFThreads) sh.pool[i] = sh.ids[sh.sel[i]];
      } else {
        npool = block_select([&](int i) { return r.item_key(i); }, r.nb - 1, M - 1, sh.s, sh.pool);
      }
      if (tid == 0) sh.pool[npool] = r.nb - 1;
      npool += 1;
      __syncthreads();
    }
    if (pool_out != nullptr) {
      int32_t* po = pool_out + (int64_t)t * M;
      for (int i = tid; i < M; i += kFThreads) po[i] = i < npool ? sh.pool[i] : -1;
    }
    // ---- the K+1 highest pool blocks hold every Top-K entry
    for (int i = tid; i < npool; i += kFThreads) {
      const int32_t b = sh.pool[i];
      sh.keys[i] = (b == r.nb - 1) ? 0xFFFFFFFFu : order_key(r.bm[b]);
    }
    __syncthreads();
    const int nsb = block_select([&](int i) { return sh.keys[i]; }, npool, K + 1, sh.s, sh.sel);
    for (int i = tid; i < nsb; i += kFThreads) sh.ids[i] = sh.pool[sh.sel[i]];  // ascending block ids
    __syncthreads();
    const int nc = nsb * kBlock;
    for (int c = tid; c < nc; c += kFThreads) {
      const int32_t j = sh.ids[c >> 3] * kBlock + (c & 7);
      sh.keys[kMaxPool + c] = j < r.n ? order_key(r.scores[j]) : 0u;
    }
    __syncthreads();
    const int cnt = block_select([&](int i) { return sh.keys[kMaxPool + i]; }, nc, K, sh.s, sh.sel);
    for (int i = tid; i < K; i += kFThreads) {
      const int32_t c = i < cnt ? sh.sel[i] : -1;
      tk[i] = c < 0 ? -1 : sh.ids[c >> 3] * kBlock + (c & 7);
    }
  }
  // return the histogram to zero for the next call
  if (r.needs_hist())
    for (int b = tid; b < kBins; b += kFThreads) ws_hist[(int64_t)t * kBins + b] = 0u;
}

struct Layout {
  int32_t G, row_cap;
  size_t hist, cnt, ids, bm, total;  // byte offsets
};

Layout make_layout(int32_t n_q, int32_t width, int32_t M, bool cand) {
  Layout L;
  const int64_t nbw = (width + kBlock - 1) / kBlock;
  const int64_t items = cand ? 8LL * M : nbw;
  L.G = (int32_t)((items + kSlice - 1) / kSlice);
  if (L.G < 1) L.G = 1;
  L.row_cap = L.G * kSlice;
  L.hist = 0;
  L.cnt = L.hist + (size_t)n_q * kBins * 4;
  L.ids = L.cnt + (size_t)n_q * L.G * 4;
  L.bm = L.ids + (size_t)n_q * L.row_cap * 4;
  L.total = L.bm + (cand ? 0 : (size_t)n_q * nbw * 4);
  return L;
}

}  // namespace
}  // namespace csa2

extern "C" size_t csa2_block_topk_workspace(int32_t n_q, int32_t width, int32_t M, int32_t K) {
  (void)K;
  if (n_q <= 0 || width < 0 || M < 1) return 0;
  // the larger of the Full-mode and candidate-mode layouts, so one buffer serves both
  const csa2::Layout a = csa2::make_layout(n_q, width, M, false);
  const csa2::Layout b = csa2::make_layout(n_q, width, M, true);
  return a.total > b.total ? a.total : b.total;
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
  const bool cand = pool_blocks != nullptr;
  if (cand && (pool_out || block_max || (int64_t)width != 8LL * M)) return CSA2_ERR_INVALID_ARG;
  if (n_q > 65535) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(block_max) |
       reinterpret_cast<uintptr_t>(topk_out) | reinterpret_cast<uintptr_t>(pool_out) |
       reinterpret_cast<uintptr_t>(workspace)) & 3)
    return CSA2_ERR_INVALID_ARG;
  const Layout L = make_layout(n_q, width, M, cand);
  if (L.G > kMaxG) return CSA2_ERR_UNSUPPORTED;  // rows longer than 2^20 blocks
  if (!workspace || ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  uint32_t* ws_hist = (uint32_t*)(ws + L.hist);
  int32_t* ws_cnt = (int32_t*)(ws + L.cnt);
  int32_t* ws_ids = (int32_t*)(ws + L.ids);
  float* ws_bm = cand ? nullptr : (float*)(ws + L.bm);
  const float* bm = block_max ? block_max : ws_bm;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(topk_hist_kernel, dim3(L.G, n_q), dim3(kGThreads), 0, s, cand, scores, block_max,
                     width, q_nvis, pool_blocks, M, K, ws_hist, ws_bm);
  int st = check_launch();
  if (st != CSA2_OK) return st;
  hipLaunchKernelGGL(topk_collect_kernel, dim3(L.G, n_q), dim3(kGThreads), 0, s, cand, scores, bm, width,
                     q_nvis, pool_blocks, M, K, L.G, L.row_cap, ws_hist, ws_cnt, ws_ids);
  st = check_launch();
  if (st != CSA2_OK) return st;
  hipLaunchKernelGGL(topk_final_kernel, dim3(n_q), dim3(kFThreads), 0, s, cand, scores, bm, width, q_nvis,
                     pool_blocks, M, K, L.G, L.row_cap, ws_hist, ws_cnt, ws_ids, pool_out, topk_out);
  return check_launch();
}
