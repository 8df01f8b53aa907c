// block_topk.hip -- hierarchical sparse selection for gfx950: block max -> top-M block
// pool -> Top-K inside the pool.
//
// Follows [ZB] "把 KV Cache 压缩推到极致" §2.3.4 (pad with -inf, max over blocks of 8, the
// newest visible block forced to +inf, the selected blocks expanded and truncated to the
// visible width) and [DF] "CSA2 与每 token 890 字节" §4.7 (g_r, TopM over blocks, pool =
// union of the selected blocks, |P_t| <= 2048 x 8).  Ties go to the lower index, NaN
// ranks as -inf, outputs are ascending and padded with -1.
//
// Design (three kernels, launched back to back on the caller's stream).  The ranking key
// of a value is an order-preserving uint32 map of the fp32 value (NaN as -inf); its top
// 12 bits are its histogram bin.
//   K1 hist     1024-thread workgroups of 8192 keys each build a 4096-bin histogram of
//               the ranking keys (older blocks' maxima in Full mode, pool entries in
//               candidate mode) in LDS and add it into a per-query histogram in the
//               workspace (few, large workgroups: every global add is a slow atomic; a
//               row that one workgroup covers is written with plain stores).
//   K2 collect  workgroups of 1024 items find the bin of the k-th largest key and write, in
//               ascending order, the ids and keys of every item in that bin or above into
//               one segment per workgroup (list A).  In Full mode it also lists the
//               entries of the blocks in or above the bin of the K-th largest older block,
//               and of the newest block, whose keys reach that bin's lower edge (list B).
//               Every global Top-K entry is
//               in list B: the K highest older blocks alone hold K entries at or above
//               that edge.  The Top-K of the pool equals the global Top-K of the row, since
//               any entry outside the pool is outranked by the M-1 block maxima above it.
//   K3 finalize one 1024-thread workgroup per query and role, the roles in parallel: the
//               pool from list A, the Top-K from list B (or from list A in candidate
//               mode).  Each gathers its list into LDS, one wave per run of segments.
//               The list-A roles read K1's histogram (the count above the boundary bin
//               and the bin's own count), return it to zero, and refine only the boundary
//               bin's low 20 bits; the list-B role starts below the common leading bits of
//               its keys.  Keys are held in registers (one barrier per 10-bit radix
//               pass).  If a list overflows LDS (massive ties), K3
//               selects straight from the full row instead, with the same exact rules.
// The histogram region of the workspace must be zero before the first call; every call
// leaves it zero.
#include <mutex>

#include "csa2_device.hpp"
#include "index_tiles.hpp"

namespace csa2 {
namespace {

constexpr int kBins = kSelBins;        // 12-bit histogram digit
constexpr int kBinShift = kSelBinShift;
constexpr int kSlice = 1024;       // keys per workgroup in K2
// K1 workgroups: 4096 keys on 512 threads for a few long rows (8192 on 1024: 0.45 us slower
// per 1M x 4 decode call), 8192 keys on 1024 threads for many rows (4096 on 512: 0.49 ->
// 0.69 ms for 4096 causal prefill rows of up to 34816 entries)
constexpr int kHSlice = 4096, kHThreads = 512;
constexpr int kHSliceWide = 8192, kHThreadsWide = 1024;
constexpr int kHWideRows = 64;     // rows from which K1 takes the wide workgroups
constexpr int kGThreads = 256;     // K1 / K2 workgroup size
constexpr int kFThreads = 1024;    // K3 workgroup size
constexpr int kFWaves = kFThreads / 64;
constexpr int kListCap = 12288;    // ordered candidate list held in LDS by K3
constexpr int kMaxG = 1024;        // workgroups per query row in K1 / K2 (rows up to 2^20 items)
constexpr int kSegB = 1024;        // entries per K2 workgroup in the Top-K list (more: exact fallback)

// ------------------------------------------------------------------ shared helpers

// LDS histogram add.  Plain atomics: lanes that hit one bin serialise at about two cycles
// a lane, which is still cheaper than merging equal bins with ballots and lane reads.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin, bool active) {
  if (active) atomicAdd(&h[bin], 1u);
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

// Maximum and minimum over the 64 lanes of a wave with the same DPP pattern, returned to
// every lane (lane 63 holds the result after the row broadcasts)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return ~wave_max_u32(~x);
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

constexpr int kPer = kListCap / kFThreads;  // list keys per K3 thread, held in registers
constexpr int kBinsPer = kBins / kFThreads; // histogram bins per K3 thread
constexpr int kSegPer = kMaxG / kFThreads;  // K2 segments per K3 thread

constexpr int kLDigit = 10;                 // bits resolved per radix pass of the list selection
constexpr int kLBins = 1 << kLDigit;         // its digit histogram
constexpr int kLPerLane = kLBins / 64;       // bins per lane of the wave that scans it

struct ListScratch {
  uint32_t hist[3][kLBins] __attribute__((aligned(16)));  // digit histograms, rotated so no pass waits to clear one
  int32_t wcnt[2][kFWaves];
  uint32_t red[3][kFWaves];
  int32_t dec[4];  // a pass's decision: digit (-1: take every matching key), remain, eq_total, total
};

// Exact selection over a list of at most kListCap keys by the K3 workgroup.  The list is
// in ascending id order and ties go to the earlier position.  The caller may pass what it
// already knows: every key whose bits under `mask` exceed `prefix` is selected, and
// `remain` more are wanted among the `eq_total` keys equal to `prefix` under `mask`
// (eq_total < 0: not known); `shift` is the number of low bits not yet resolved.  With
// mask == 0 the search starts below the common leading bits of the smallest and largest
// key, so the first digit does not pile every key into one histogram bin.  Zero keys are
// never selected.  Writes the chosen positions ascending to out[], returns their number
// (to every thread), and sets *thr to a lower bound of every selected key (the resolved
// prefix).  Wave w owns the contiguous run [w*seg, (w+1)*seg) of the list, seg a whole
// number of rounds of 64, and holds it in registers, so a radix pass is a burst of LDS
// atomics, a barrier, wave 0's scan of the 1024 digit counts and a second barrier that
// hands its decision to every wave (sixteen waves repeating the scan would queue four deep
// on each SIMD).  Spreading the list over all 16 waves keeps every wave's chain of
// atomics and ballots short: the same selection on the fewest waves that hold the list
// (one wave for the Top-K role's ~700 keys, with no barriers in its passes) measured
// 20.9 against 19.6 us per selection call.
// key_of(i) gives key i from any source (LDS, or global memory read straight into
// registers); n <= kP * 1024.
template <int kP, class KeyFn>
__device__ __forceinline__ int list_select_g(KeyFn key_of, int n, uint32_t prefix, uint32_t mask, int shift,
                                             int remain, int eq_total, ListScratch& s, int32_t* out, uint32_t* thr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  prefix = __builtin_amdgcn_readfirstlane(prefix);
  mask = __builtin_amdgcn_readfirstlane(mask);
  shift = __builtin_amdgcn_readfirstlane(shift);
  remain = __builtin_amdgcn_readfirstlane(remain);
  eq_total = __builtin_amdgcn_readfirstlane(eq_total);
  n = __builtin_amdgcn_readfirstlane(n);
  for (int b = tid; b < kLBins; b += kFThreads) {
    s.hist[0][b] = 0u;
    s.hist[1][b] = 0u;
  }
  if (remain <= 0 || n <= 0) {
    __syncthreads();
    *thr = 0u;
    return 0;
  }
  const int seg = ((n + kFWaves - 1) / kFWaves + 63) & ~63;
  const int lo = min(n, wave * seg);
  const int len = __builtin_amdgcn_readfirstlane(min(n, lo + seg) - lo);  // wave-uniform
  uint32_t kr[kP];
#pragma unroll
  for (int j = 0; j < kP; j++) kr[j] = (64 * j + lane < len) ? key_of(lo + 64 * j + lane) : 0u;
  __syncthreads();  // the histograms are zero before any wave adds to them

  const int total_sel = [&]() -> int {
    if (mask == 0u) {
      // smallest and largest non-zero key, and their count
      uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, cnt = 0u;
#pragma unroll
      for (int j = 0; j < kP; j++) {
        if (64 * j >= len) continue;
        const uint32_t key = kr[j];
        kmin = min(kmin, key != 0u ? key : 0xFFFFFFFFu);
        kmax = max(kmax, key);
        cnt += key != 0u ? 1u : 0u;
      }
      kmin = wave_min_u32(kmin);
      kmax = wave_max_u32(kmax);
      cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), 63);
      if (lane == 0) {
        s.red[0][wave] = kmin;
        s.red[1][wave] = kmax;
        s.red[2][wave] = cnt;
      }
      __syncthreads();
      kmin = 0xFFFFFFFFu;
      kmax = 0u;
      cnt = 0u;
#pragma unroll
      for (int w = 0; w < kFWaves; w++) {
        kmin = min(kmin, s.red[0][w]);
        kmax = max(kmax, s.red[1][w]);
        cnt += s.red[2][w];
      }
      kmin = __builtin_amdgcn_readfirstlane(kmin);
      kmax = __builtin_amdgcn_readfirstlane(kmax);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
      if (cnt == 0u) return 0;  // workgroup-uniform
      const int common = kmin == kmax ? 32 : __builtin_clz(kmin ^ kmax);
      mask = common == 0 ? 0u : (common == 32 ? 0xFFFFFFFFu : ~0u << (32 - common));
      prefix = kmax & mask;
      shift = 32 - common;
      eq_total = (int)cnt;
    }
    for (int p = 0; shift > 0 && (eq_total < 0 || remain < eq_total); p++) {
      const int nshift = max(shift - kLDigit, 0);
      const uint32_t dmask = (1u << (shift - nshift)) - 1u;
      uint32_t* h = s.hist[p % 3];
      for (int b = tid; b < kLBins; b += kFThreads) s.hist[(p + 1) % 3][b] = 0u;  // last read two passes ago
#pragma unroll
      for (int j = 0; j < kP; j++) {
        if (64 * j >= len) continue;  // uniform: the wave's remaining slots are empty
        const uint32_t key = kr[j];
        if (key != 0u && (key & mask) == prefix) atomicAdd(&h[(key >> nshift) & dmask], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns the kLPerLane digits below kLBins - kLPerLane * l (descending), read as
        // 16-byte words: once for their sum, once for the search (fewer live registers)
        const int hi_bin = kLBins - 1 - kLPerLane * lane;
        const uint4* hw = reinterpret_cast<const uint4*>(h + hi_bin + 1 - kLPerLane);
        uint32_t local = 0;
#pragma unroll
        for (int v = 0; v < kLPerLane / 4; v++) {
          const uint4 w4 = hw[v];
          local += (w4.x + w4.y) + (w4.z + w4.w);
        }
        const uint32_t incl = wave_incl_scan(local);
        const int total = __builtin_amdgcn_readlane((int)incl, 63);
        uint32_t above = incl - local;
        int hit = -1, hit_rem = 0, hit_cnt = 0;
        asm volatile("" ::: "memory");  // read the words again below instead of keeping them
#pragma unroll
        for (int v = kLPerLane / 4 - 1; v >= 0; v--) {  // descending digits: word v from its top
          const uint4 w4 = hw[v];
          const uint32_t cw[4] = {w4.w, w4.z, w4.y, w4.x};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            if ((int)above < remain && remain <= (int)(above + cw[e])) {
              hit = hi_bin + 1 - kLPerLane + 4 * v + 3 - e;
              hit_rem = remain - (int)above;
              hit_cnt = (int)cw[e];
            }
            above += cw[e];
          }
        }
        const uint64_t hb = __ballot(hit >= 0);
        const int src = hb == 0ull ? 0 : __ffsll((unsigned long long)hb) - 1;
        // the lane reads run with the whole wave active: under a lane-0 branch the compiler
        // may compute hit and its companions for lane 0 alone
        const int d0 = hb == 0ull ? -1 : __builtin_amdgcn_readlane(hit, src);
        const int d1 = __builtin_amdgcn_readlane(hit_rem, src);
        const int d2 = __builtin_amdgcn_readlane(hit_cnt, src);
        if (lane == 0) {
          s.dec[0] = d0;
          s.dec[1] = d1;
          s.dec[2] = d2;
          s.dec[3] = total;
        }
      }
      __syncthreads();
      const int dd = __builtin_amdgcn_readfirstlane(s.dec[0]);
      if (dd < 0) {  // fewer matching keys than wanted: take them all
        remain = eq_total = __builtin_amdgcn_readfirstlane(s.dec[3]);
        break;
      }
      const uint32_t d = (uint32_t)dd;
      remain = __builtin_amdgcn_readfirstlane(s.dec[1]);
      eq_total = __builtin_amdgcn_readfirstlane(s.dec[2]);
      prefix |= d << nshift;
      mask |= dmask << nshift;
      shift = nshift;
    }
    const bool all_eq = eq_total >= 0 && remain >= eq_total;
    // ordered compaction: counts per wave, then each wave writes its run of the output
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kP; j++) {
      if (64 * j >= len) continue;
      const uint32_t key = kr[j];
      gt += __popcll(__ballot(key != 0u && (key & mask) > prefix));
      eq += __popcll(__ballot(key != 0u && (key & mask) == prefix));
    }
    if (lane == 0) {
      s.wcnt[0][wave] = gt;
      s.wcnt[1][wave] = eq;
    }
    __syncthreads();
    const uint32_t e_l = lane < kFWaves ? (uint32_t)s.wcnt[1][lane] : 0u;
    const uint32_t e_incl = wave_incl_scan(e_l);
    const uint32_t e_before = e_incl - e_l;
    const uint32_t take = all_eq ? e_l : (uint32_t)max(0, min((int)e_l, remain - (int)e_before));
    const uint32_t s_l = lane < kFWaves ? (uint32_t)s.wcnt[0][lane] + take : 0u;
    const uint32_t s_incl = wave_incl_scan(s_l);
    const int tot_sel = __builtin_amdgcn_readlane((int)s_incl, kFWaves - 1);
    int run_eq = __builtin_amdgcn_readlane((int)e_before, wave);
    int run_sel = __builtin_amdgcn_readlane((int)(s_incl - s_l), wave);
#pragma unroll
    for (int j = 0; j < kP; j++) {
      if (64 * j >= len) continue;
      const uint32_t key = kr[j];
      const bool is_eq = key != 0u && (key & mask) == prefix;
      const uint64_t eqb = __ballot(is_eq);
      const bool sel = key != 0u && ((key & mask) > prefix ||
                                     (is_eq && (all_eq || run_eq + __popcll(eqb & lt) < remain)));
      const uint64_t selb = __ballot(sel);
      if (sel) out[run_sel + __popcll(selb & lt)] = lo + 64 * j + lane;
      run_eq += __popcll(eqb);
      run_sel += __popcll(selb);
    }
    return tot_sel;
  }();
  __syncthreads();  // out[] is complete before its readers
  *thr = prefix;
  return total_sel;
}

// list_select_g over keys held in LDS (the finalize's gathered list), instantiated for the
// fewest 64-key rounds per wave that hold the list (n is workgroup-uniform)
__device__ __forceinline__ int list_select(const uint32_t* keys, int n, uint32_t prefix, uint32_t mask, int shift,
                                           int remain, int eq_total, ListScratch& s, int32_t* out, uint32_t* thr) {
  auto key_of = [&](int i) { return keys[i]; };
  if (n <= 1 * kFThreads) return list_select_g<1>(key_of, n, prefix, mask, shift, remain, eq_total, s, out, thr);
  if (n <= 2 * kFThreads) return list_select_g<2>(key_of, n, prefix, mask, shift, remain, eq_total, s, out, thr);
  if (n <= 4 * kFThreads) return list_select_g<4>(key_of, n, prefix, mask, shift, remain, eq_total, s, out, thr);
  return list_select_g<kPer>(key_of, n, prefix, mask, shift, remain, eq_total, s, out, thr);
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
  // ranking items of the histogram: the pool's positions (candidate mode) or the older
  // blocks 0 .. nb-2 (full mode; the newest block is handled apart)
  __device__ int32_t items() const { return cand ? 8 * M : max(nb - 1, 0); }
  // the key of item i for any i (out-of-range items read item 0 and give 0): the loads do
  // not sit behind a branch, so a caller's unrolled loads are all in flight at once
  __device__ __forceinline__ uint32_t item_key_clamped(int32_t i, int32_t hi) const {
    const int32_t ic = i < hi ? i : 0;
    const uint32_t k = item_key(ic);
    return i < hi ? k : 0u;
  }
  __device__ uint32_t item_key(int32_t i) const {  // 0 = not a candidate
    if (cand) {
      const int32_t b = pool[i >> 3];
      const int64_t j = (int64_t)b * kBlock + (i & 7);
      return (b >= 0 && j < n) ? order_key(scores[i]) : 0u;
    }
    return order_key(bm[i]);
  }
  __device__ uint32_t entry_key(int32_t j) const { return j < n ? order_key(scores[j]) : 0u; }
};

__device__ __forceinline__ Row make_row(int t, bool cand, const float* scores, const float* bm, int32_t width,
                                        const int32_t* q_nvis, const int32_t* pool_blocks, int32_t M, int32_t K) {
  Row r;
  r.cand = cand;
  r.scores = scores ? scores + (int64_t)t * width : nullptr;  // NULL in pool-only mode
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

// Workspace views shared by the kernels (byte offsets are fixed by make_layout).
struct Ws {
  uint32_t* hist;    // [n_q][kBins] ranking keys of the items
  int32_t* cnt_a;    // [n_q][G] per-workgroup lengths of list A
  int32_t* cnt_b;    // [n_q][G] per-workgroup lengths of list B
  int32_t* ids_a;    // [n_q][G * kSlice]
  uint32_t* keys_a;
  int32_t* ids_b;    // [n_q][G * seg_b]
  uint32_t* keys_b;
  float* bm;         // [n_q][nbw] block maxima when the caller gives none
  int32_t G;
  int32_t seg_b;     // list-B slots per K2 workgroup: kSegB, or every slot of its slice when re-scoring
};

// Re-scoring mode (Full mode without a score row): list B's entries are scored from the
// indexer cache by the scan's own tile arithmetic (idx::mfma_bf16_tile, idx::head_sum), so
// their keys are the bits the scan would have written.
struct Rescore {
  const uint16_t* q;         // bf16 indexer query [n_q, 32, 128]
  const float* head_w;       // [n_q, 32]
  const uint8_t* idx_cache;  // tile layout; query t's entry j is entry q_base[t] + j
  const int64_t* q_base;
};

// ------------------------------------------------------------------ K1: histogram

template <bool cand, int kSl, int kTh>
__global__ __launch_bounds__(kTh) void topk_hist_kernel(
    const float* __restrict__ scores, const float* __restrict__ block_max, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K, Ws ws) {
  __shared__ uint32_t h[kBins];
  const int t = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int32_t nbw = (width + kBlock - 1) / kBlock;
  Row r = make_row(t, cand, scores, block_max ? block_max : ws.bm, width, q_nvis, pool_blocks, M, K);
  const int32_t lo = g * kSl;
  if (!cand && block_max == nullptr) {
    // block maxima from the scores (NaN never wins a comparison, so it ranks as -inf)
    float* bmw = ws.bm + (int64_t)t * nbw;
    for (int32_t b = lo + tid; b < min(lo + kSl, r.nb); b += kTh) {
      float v[kBlock];
#pragma unroll
      for (int o = 0; o < kBlock; o++) {  // the block's loads in flight together (j < n for o = 0)
        const int32_t j = b * kBlock + o;
        v[o] = r.scores[j < r.n ? j : b * kBlock];
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int o = 0; o < kBlock; o++)
        if (b * kBlock + o < r.n) mx = v[o] > mx ? v[o] : mx;
      bmw[b] = mx;
    }
    __syncthreads();
  }
  const int32_t hi = min(lo + kSl, r.items());
  if (lo >= hi) return;
  for (int b = tid; b < kBins; b += kTh) h[b] = 0;
  __syncthreads();
  constexpr int kPerH = kSl / kTh;
  uint32_t keys[kPerH];
#pragma unroll
  for (int u = 0; u < kPerH; u++) {  // every key load in flight at once
    const int32_t i = lo + u * kTh + tid;
    keys[u] = r.item_key_clamped(i, hi);
  }
#pragma unroll
  for (int u = 0; u < kPerH; u++) hist_add(h, keys[u] >> kBinShift, keys[u] != 0u);
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)t * kBins;
  if (gridDim.x == 1) {  // the only workgroup of its row: plain stores (the region starts zeroed)
    for (int b = tid; b < kBins; b += kTh)
      if (h[b]) gh[b] = h[b];
  } else {
    for (int b = tid; b < kBins; b += kTh)
      if (h[b]) atomicAdd(&gh[b], h[b]);
  }
}

// ------------------------------------------------------------------ K2: ordered collection

// Each workgroup covers kSlice items of one query; wave w holds items lo + 256w .. +255 in
// registers, four per lane.  List A: the items in the bin of the kA-th largest key or
// above (kA = M-1 for the pool, K in candidate mode), in ascending order.  List B (full
// mode): of every block of the slice in or above the bin of the K-th largest older-block
// maximum, and of the newest block, the visible entries whose keys reach that bin's lower
// edge, in ascending order.  The K highest older blocks alone
// hold K entries at or above that edge, so every Top-K entry keeps its key.
constexpr int kItemsPerLane = kSlice / kGThreads;

template <bool cand, bool kRescore = false>
__global__ __launch_bounds__(kGThreads) void topk_collect_kernel(
    bool want_pool, bool want_topk, const float* __restrict__ scores, const float* __restrict__ bm, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K, Ws ws,
    Rescore rsc) {
  __shared__ int32_t s_wave[kGThreads / 64];
  __shared__ int32_t s_cnt[2][kGThreads / 64];
  __shared__ int32_t s_bnd[2];
  __shared__ int32_t s_cb[kSlice];
  const int t = blockIdx.y, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = ws.G;
  Row r = make_row(t, cand, scores, bm, width, q_nvis, pool_blocks, M, K);
  const int32_t lo = g * kSlice;
  const int32_t hi_a = min(lo + kSlice, r.items());             // ranked items of the slice
  const int32_t hi_b = cand ? lo : min(lo + kSlice, r.nb);       // blocks of the slice, newest included
  // the slice's keys and the histogram load together
  uint32_t key[kItemsPerLane];
#pragma unroll
  for (int j = 0; j < kItemsPerLane; j++) {
    const int32_t i = lo + 256 * wave + 64 * j + lane;
    key[j] = r.item_key_clamped(i, hi_a);  // item 0 of the row always exists
  }
  const uint32_t* gh = ws.hist + (int64_t)t * kBins;
  uint32_t hb[16], local = 0;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    hb[q] = gh[16 * tid + q];
    local += hb[q];
  }
  if (tid < 2) s_bnd[tid] = -1;
  int tot_i;
  const int before = block_excl_scan<kGThreads>((int)local, s_wave, tot_i);
  const int total = tot_i;
  // list A is needed when the selection does not take every item
  const int kA = cand ? min(K, total) : ((want_pool && total > M - 1) ? M - 1 : 0);
  const int kB = (!cand && want_topk && total >= K) ? K : 0;  // 0: every older block is a candidate
  {
    uint32_t above = (uint32_t)(total - before) - local;  // keys in bins above this thread's range
#pragma unroll
    for (int q = 15; q >= 0; q--) {
      if (kA > 0 && (int)above < kA && kA <= (int)(above + hb[q])) s_bnd[0] = 16 * tid + q;
      if (kB > 0 && (int)above < kB && kB <= (int)(above + hb[q])) s_bnd[1] = 16 * tid + q;
      above += hb[q];
    }
  }
  __syncthreads();
  const int32_t b1 = s_bnd[0], b2 = s_bnd[1];
  const uint32_t floor_key = b2 >= 0 ? (uint32_t)b2 << kBinShift : 0u;
  // flags and per-wave counts for list A and the candidate blocks
  uint64_t ba[kItemsPerLane], bb[kItemsPerLane];
  int ca = 0, cb = 0;
#pragma unroll
  for (int j = 0; j < kItemsPerLane; j++) {
    const int32_t i = lo + 256 * wave + 64 * j + lane;
    const uint32_t k = key[j];
    ba[j] = __ballot(b1 >= 0 && k != 0u && (int32_t)(k >> kBinShift) >= b1);
    bb[j] = __ballot(i < hi_b && (i == r.nb - 1 || k >= floor_key));
    ca += __popcll(ba[j]);
    cb += __popcll(bb[j]);
  }
  if (lane == 0) {
    s_cnt[0][wave] = ca;
    s_cnt[1][wave] = cb;
  }
  __syncthreads();
  int oa = 0, ob = 0, na = 0, ncb = 0;
#pragma unroll
  for (int w = 0; w < kGThreads / 64; w++) {
    oa += w < wave ? s_cnt[0][w] : 0;
    ob += w < wave ? s_cnt[1][w] : 0;
    na += s_cnt[0][w];
    ncb += s_cnt[1][w];
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* oid = ws.ids_a + ((int64_t)t * G + g) * kSlice;
  uint32_t* okey = ws.keys_a + ((int64_t)t * G + g) * kSlice;
#pragma unroll
  for (int j = 0; j < kItemsPerLane; j++) {
    const int32_t i = lo + 256 * wave + 64 * j + lane;
    if ((ba[j] >> lane) & 1ull) {
      const int pos = oa + __popcll(ba[j] & lt);
      oid[pos] = i;
      okey[pos] = key[j];
    }
    if ((bb[j] >> lane) & 1ull) s_cb[ob + __popcll(bb[j] & lt)] = i;
    oa += __popcll(ba[j]);
    ob += __popcll(bb[j]);
  }
  if (tid == 0) ws.cnt_a[(int64_t)t * G + g] = na;
  if (cand || !want_topk) return;  // pool-only mode needs no list B
  __syncthreads();
  // ---- list B: of every candidate block, the entries whose keys reach the floor, in
  // order.  Slots (8 per block) go in chunks of 1024: wave w takes slots 256w .. 256w+255
  // of the chunk (4 rounds of 64), and the chunk's survivors append after the last ones.
  // Re-scoring computes each round's 64 keys as two 32-entry tiles (lane (n, g) of tile h
  // scores slot 64u + 32h + n; lane L takes slot 64u + L from tile L / 32).
  const int nslots = ncb * kBlock;
  constexpr int kSlotRounds = kSegB / kGThreads;
  const int seg_b = ws.seg_b;
  int32_t* bid = ws.ids_b + ((int64_t)t * G + g) * seg_b;
  uint32_t* bkey = ws.keys_b + ((int64_t)t * G + g) * seg_b;
  __amdgpu_buffer_rsrc_t rs_cache;
  int32_t rel0 = 0;  // the sequence's first entry, counted from the resource's first tile
  if constexpr (kRescore) rs_cache = idx::idx_rsrc(rsc.idx_cache, rsc.q_base[t], r.n, rel0);
  int nbv = 0;
  for (int c0 = 0; c0 < nslots; c0 += kSegB) {
    uint32_t bk[kSlotRounds];
    uint64_t bf[kSlotRounds];
    int cw = 0;
    if constexpr (kRescore) {
      // the query's fragments and head weights (lane (n, g) as in the scan) go out with the
      // candidate rows, only in workgroups that have candidates
      const int n = lane & 31, gg = lane >> 5;
      bf16x8 qa[8];
      float qw[16];
      idx::load_query_bf16(rsc.q, rsc.head_w, t, n, gg, qa, qw);
      idx::RawTile rt[kSlotRounds][2];
#pragma unroll
      for (int u = 0; u < kSlotRounds; u++) {  // every row load of the chunk in flight at once
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int cs = c0 + 256 * wave + 64 * u + 32 * h + n;
          const int32_t j = cs < nslots ? s_cb[cs >> 3] * kBlock + (cs & 7) : 0;
          rt[u][h].valid = cs < nslots && j < r.n;
          idx::load_entry_share<0>(rs_cache, rt[u][h].valid ? rel0 + j : -1, gg, rt[u][h]);
        }
      }
#pragma unroll
      for (int u = 0; u < kSlotRounds; u++) {
        const int base = c0 + 256 * wave + 64 * u;  // wave-uniform
        float sc0 = 0.0f, sc1 = 0.0f;
        if (base < nslots) sc0 = idx::head_sum(idx::mfma_bf16_tile(qa, rt[u][0], gg), qw, rt[u][0].valid);
        if (base + 32 < nslots) sc1 = idx::head_sum(idx::mfma_bf16_tile(qa, rt[u][1], gg), qw, rt[u][1].valid);
        const int c = base + lane;
        const int32_t j = c < nslots ? s_cb[c >> 3] * kBlock + (c & 7) : 0;
        const uint32_t k = (c < nslots && j < r.n) ? order_key(lane < 32 ? sc0 : sc1) : 0u;
        bk[u] = k >= floor_key ? k : 0u;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSlotRounds; u++) {  // every score load of the chunk in flight at once
        const int c = c0 + 256 * wave + 64 * u + lane;
        const int32_t j = c < nslots ? s_cb[c >> 3] * kBlock + (c & 7) : 0;
        const float v = (c < nslots && j < r.n) ? r.scores[j] : 0.0f;
        const uint32_t k = (c < nslots && j < r.n) ? order_key(v) : 0u;
        bk[u] = k >= floor_key ? k : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kSlotRounds; u++) {
      bf[u] = __ballot(bk[u] != 0u);
      cw += __popcll(bf[u]);
    }
    if (lane == 0) s_cnt[0][wave] = cw;
    __syncthreads();
    int ob2 = nbv, tot = 0;
#pragma unroll
    for (int w = 0; w < kGThreads / 64; w++) {
      ob2 += w < wave ? s_cnt[0][w] : 0;
      tot += s_cnt[0][w];
    }
    __syncthreads();  // s_cnt is rewritten by the next chunk
    if (nbv + tot > seg_b) {  // segment overflow (only without re-scoring): the finalize falls back to the full row
      if (tid == 0) ws.cnt_b[(int64_t)t * G + g] = kListCap + 1;
      return;
    }
#pragma unroll
    for (int u = 0; u < kSlotRounds; u++) {
      if ((bf[u] >> lane) & 1ull) {
        const int c = c0 + 256 * wave + 64 * u + lane;
        const int pos = ob2 + __popcll(bf[u] & lt);
        bid[pos] = s_cb[c >> 3] * kBlock + (c & 7);
        bkey[pos] = bk[u];
      }
      ob2 += __popcll(bf[u]);
    }
    nbv += tot;
  }
  if (tid == 0) ws.cnt_b[(int64_t)t * G + g] = nbv;
}

// ------------------------------------------------------------------ K3: exact finalize

// Thread tid owns the kBinsPer bins below kBins-1-kBinsPer*tid (descending) with counts c[]
// and `above` keys in higher bins.  If rank k (1-based, from the top) falls in one of them,
// records that bin, the count above it and its own count at bnd[slot..slot+2].
__device__ __forceinline__ void hist_boundary(const uint32_t* c, uint32_t above, int k, int slot, int32_t* bnd) {
  if (k <= 0) return;
#pragma unroll
  for (int q = 0; q < kBinsPer; q++) {
    if ((int)above < k && k <= (int)(above + c[q])) {
      bnd[slot] = kBins - 1 - kBinsPer * (int)threadIdx.x - q;
      bnd[slot + 1] = (int)above;
      bnd[slot + 2] = (int)c[q];
    }
    above += c[q];
  }
}

struct FinShared {
  int32_t ids[kListCap];       // the gathered list
  uint32_t keys[kListCap];
  int32_t sel[kMaxPool];       // selected positions (every selection takes <= M-1 or K)
  int32_t seg_off[kMaxG + 1];
  int32_t scan[2 * kFWaves];
  int32_t bnd[4];              // boundary bin, count above it, its count, total
  ListScratch ls;
  SelScratch s;
};

// One workgroup per (role, query).  Role 0 builds the pool from list A (Full mode); role
// 1 takes the Top-K from list B (Full mode) or list A (candidate mode).  Each reads the
// matching histogram, returns it to zero, gathers its list (a superset of the selection
// in ascending id order) and refines the boundary bin's low 20 bits over it.
template <bool cand, bool kRescore = false>
__global__ __launch_bounds__(kFThreads) void topk_final_kernel(
    bool want_pool, bool want_topk, const float* __restrict__ scores, const float* __restrict__ bm, int32_t width,
    const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K, Ws ws,
    int32_t* __restrict__ pool_out, int32_t* __restrict__ topk_out) {
  __shared__ FinShared sh;
  const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int role = !want_topk ? 0 : ((cand || !want_pool) ? 1 : (int)blockIdx.x);
  const int G = ws.G;
  Row r = make_row(t, cand, scores, bm, width, q_nvis, pool_blocks, M, K);
  // the list, its histogram and the rank wanted.  Roles on list A use K1's histogram
  const bool use_a = role == 0 || cand;
  uint32_t* gh = ws.hist + (int64_t)t * kBins;
  const int32_t* cnts = (use_a ? ws.cnt_a : ws.cnt_b) + (int64_t)t * G;
  const int64_t seg_stride = use_a ? kSlice : ws.seg_b;
  const int32_t* lids = (use_a ? ws.ids_a : ws.ids_b) + (int64_t)t * G * seg_stride;
  const uint32_t* lkeys = (use_a ? ws.keys_a : ws.keys_b) + (int64_t)t * G * seg_stride;
  const int want = role == 0 ? M - 1 : K;

  // The first round of the list gather (segments wave + 16k) loads its segments' first 128
  // slots now, before their counts and offsets are known, so these loads and the
  // histogram's are in flight together.  Slots past a segment's count hold stale values
  // and are never used; every slot read lies inside the segment's fixed-size region.
  int32_t pre_id[4][2];
  uint32_t pre_key[4][2];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int g = wave + k * kFWaves;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int64_t src = (int64_t)(g < G ? g : 0) * seg_stride + 64 * h + lane;
      pre_id[k][h] = lids[src];
      pre_key[k][h] = lkeys[src];
    }
  }

  // ---- histogram boundary (list A) and segment offsets, in one pass of two scans
  uint32_t c[kBinsPer];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < kBinsPer; q++) {
    const uint32_t hv = gh[kBins - 1 - kBinsPer * tid - q];  // read by both roles, used by list-A roles
    c[q] = use_a ? hv : 0u;
    local += c[q];
  }
  int cs[kSegPer], cl = 0;
#pragma unroll
  for (int q = 0; q < kSegPer; q++) {
    const int g = kSegPer * tid + q;
    const int32_t cv = cnts[g < G ? g : 0];
    cs[q] = g < G ? cv : 0;
    cl += cs[q];
  }
  const uint32_t xa = wave_incl_scan(local), xb = wave_incl_scan((uint32_t)cl);
  if (lane == 63) {
    sh.scan[wave] = (int)xa;
    sh.scan[kFWaves + wave] = (int)xb;
  }
  if (tid < 4) sh.bnd[tid] = -1;
  __syncthreads();
  int offa = 0, offb = 0, tota = 0, totb = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; w++) {
    const int a = sh.scan[w], b = sh.scan[kFWaves + w];
    offa += (w < wave) ? a : 0;
    offb += (w < wave) ? b : 0;
    tota += a;
    totb += b;
  }
  if (use_a) hist_boundary(c, (uint32_t)(offa + (int)xa - (int)local), min(want, tota), 0, sh.bnd);
  int run = offb + (int)xb - cl;
#pragma unroll
  for (int q = 0; q < kSegPer; q++) {
    const int g = kSegPer * tid + q;
    if (g < G) sh.seg_off[g] = run;
    run += cs[q];
  }
  if (tid == 0) sh.seg_off[G] = totb;
  // K1's histogram has been read (or is not needed): return it to zero for the next call
  if (use_a || !want_pool) {
#pragma unroll
    for (int q = 0; q < kBinsPer; q++) gh[kBins - 1 - kBinsPer * tid - q] = 0u;
  }
  __syncthreads();
  const int total = sh.seg_off[G];
  // Full-mode pool with no more older blocks than M-1: every older block is in
  const bool take_all_blocks = role == 0 && tota <= M - 1;
  const bool listed = !take_all_blocks && total <= kListCap;

  int cnt = 0;
  if (take_all_blocks) {
    cnt = max(r.nb - 1, 0);
  } else if (listed) {
    // gather the list: wave w copies segments w, w + 16, ... (one lane per item).  The first
    // round's first 128 slots are already in registers; the rest loads four segments at a
    // time, and segments longer than that loop on
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int g = wave + k * kFWaves;
      const int off = g < G ? sh.seg_off[g] : 0;
      const int n = g < G ? sh.seg_off[g + 1] - off : 0;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (64 * h + lane < n) {
          sh.ids[off + 64 * h + lane] = pre_id[k][h];
          sh.keys[off + 64 * h + lane] = pre_key[k][h];
        }
      }
      for (int e = 128 + lane; e < n; e += 64) {
        sh.ids[off + e] = lids[(int64_t)g * seg_stride + e];
        sh.keys[off + e] = lkeys[(int64_t)g * seg_stride + e];
      }
    }
    for (int g0 = wave + 4 * kFWaves; g0 < G; g0 += 4 * kFWaves) {
      int32_t gid[4], dst[4], cnt4[4], off4[4];
      uint32_t gkey[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int g = g0 + k * kFWaves;
        off4[k] = g < G ? sh.seg_off[g] : 0;
        cnt4[k] = g < G ? sh.seg_off[g + 1] - off4[k] : 0;
        const bool ok = lane < cnt4[k];
        const int64_t src = (int64_t)(g < G ? g : 0) * seg_stride + (ok ? lane : 0);  // slot 0 stands in
        gid[k] = lids[src];
        gkey[k] = lkeys[src];
        dst[k] = ok ? off4[k] + lane : -1;
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        if (dst[k] >= 0) {
          sh.ids[dst[k]] = gid[k];
          sh.keys[dst[k]] = gkey[k];
        }
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int64_t g = g0 + k * kFWaves;
        for (int e = 64 + lane; e < cnt4[k]; e += 64) {
          sh.ids[off4[k] + e] = lids[g * seg_stride + e];
          sh.keys[off4[k] + e] = lkeys[g * seg_stride + e];
        }
      }
    }
    __syncthreads();
    int kk = min(want, tota);
    uint32_t thr;
    if (!use_a) {
      // Top-K of list B: the selection starts below the common leading bits of its keys
      cnt = list_select(sh.keys, total, 0u, 0u, 32, K, -1, sh.ls, sh.sel, &thr);
      for (int i = tid; i < cnt; i += kFThreads) sh.sel[i] = sh.ids[sh.sel[i]];
    } else {
      const int b1 = sh.bnd[0];
      if (b1 >= 0) {
        cnt = list_select(sh.keys, total, (uint32_t)b1 << kBinShift, ~0u << kBinShift, kBinShift, kk - sh.bnd[1],
                          sh.bnd[2], sh.ls, sh.sel, &thr);
        for (int i = tid; i < cnt; i += kFThreads) sh.sel[i] = sh.ids[sh.sel[i]];
      }
    }
  } else if (role == 0) {
    cnt = block_select([&](int i) { return r.item_key(i); }, r.items(), M - 1, sh.s, sh.sel);
  } else if (cand) {
    cnt = block_select([&](int i) { return r.item_key(i); }, r.items(), K, sh.s, sh.sel);
  } else if constexpr (kRescore) {
    // list B is longer than the LDS list (massive ties): select straight from its segments
    // in global memory (list position i lies in the segment whose offset range holds it),
    // then turn the chosen positions into entry ids
    auto seg_of = [&](int i) {
      int lo = 0, hi = G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.seg_off[mid] <= i) lo = mid;
        else hi = mid;
      }
      return lo;
    };
    cnt = block_select(
        [&](int i) {
          const int sg = seg_of(i);
          return lkeys[(int64_t)sg * seg_stride + (i - sh.seg_off[sg])];
        },
        total, K, sh.s, sh.sel);
    __syncthreads();
    for (int i = tid; i < cnt; i += kFThreads) {
      const int p = sh.sel[i], sg = seg_of(p);
      sh.sel[i] = lids[(int64_t)sg * seg_stride + (p - sh.seg_off[sg])];
    }
  } else {
    cnt = block_select([&](int j) { return r.entry_key(j); }, r.n, K, sh.s, sh.sel);
  }
  __syncthreads();

  if (role == 0) {
    // the pool: the selected older blocks plus the forced newest block, ascending
    int32_t* po = pool_out + (int64_t)t * M;
    const int npool = r.nb > 0 ? cnt + 1 : 0;
    for (int i = tid; i < M; i += kFThreads) {
      int32_t v = -1;
      if (i < cnt) v = take_all_blocks ? i : sh.sel[i];
      else if (i == cnt && npool > 0) v = r.nb - 1;
      po[i] = v;
    }
    return;
  }
  int32_t* tk = topk_out + (int64_t)t * K;
  for (int i = tid; i < K; i += kFThreads) {
    const int32_t p = i < cnt ? sh.sel[i] : -1;
    tk[i] = p < 0 ? -1 : (cand ? r.pool[p >> 3] * kBlock + (p & 7) : p);
  }
}

// ------------------------------------------------------------------ one-launch path for short rows

// Rows of at most 4096 ranking items (4 keys per thread) take the whole selection in one
// launch: one 1024-thread workgroup per query and role reads the keys
// straight from the scores (or block maxima) into registers and runs list_select_g.  The
// pool role ranks the older blocks by their maxima (the caller's, or computed here as K1
// does) and appends the newest block; the Top-K role ranks every visible entry in Full mode
// (the global Top-K equals the Top-K inside the pool) or the pool's slots in candidate
// mode.  The results are those of the three-kernel path bit for bit.  (Measured: one
// workgroup holding 16-32 keys per thread is slower than the three launches -- the 32K-entry
// decode step 68.5 against 51.8 us, a 16384-slot candidate pool 19.6 against 17.0 us -- while
// the 2048-entry step gains 5 us.)
constexpr int kSmallPer = 4;
constexpr int kSmallMax = kSmallPer * kFThreads;  // 4096 keys

struct SmallShared {
  int32_t sel[kMaxPool];
  ListScratch ls;
};

template <bool cand>
__global__ __launch_bounds__(kFThreads) void topk_small_kernel(
    bool want_pool, bool want_topk, const float* __restrict__ scores, const float* __restrict__ block_max,
    int32_t width, const int32_t* __restrict__ q_nvis, const int32_t* __restrict__ pool_blocks, int32_t M, int32_t K,
    int32_t* __restrict__ pool_out, int32_t* __restrict__ topk_out) {
  __shared__ SmallShared sh;
  const int t = blockIdx.y, tid = threadIdx.x;
  const int role = !want_topk ? 0 : ((cand || !want_pool) ? 1 : (int)blockIdx.x);
  const Row r = make_row(t, cand, scores, block_max, width, q_nvis, pool_blocks, M, K);
  uint32_t thr;
  if constexpr (!cand) {  // (candidate mode has no pool role)
  if (role == 0) {
    // the pool: the top M-1 older blocks (every one when there are no more), ascending, then
    // the newest block
    const int nold = max(r.nb - 1, 0);
    const bool take_all = nold <= M - 1;
    int cnt = nold;
    if (!take_all) {
      if (block_max != nullptr) {
        cnt = list_select_g<kSmallPer>([&](int b) { return order_key(r.bm[b]); }, nold, 0u, 0u, 32, M - 1, -1, sh.ls,
                                       sh.sel, &thr);
      } else {  // the block's maximum from its entries (NaN never wins, as in K1)
        cnt = list_select_g<kSmallPer>(
            [&](int b) {
              float v[kBlock];
#pragma unroll
              for (int o = 0; o < kBlock; o++) v[o] = r.scores[b * kBlock + o];  // older blocks are whole
              float mx = -__builtin_inff();
#pragma unroll
              for (int o = 0; o < kBlock; o++) mx = v[o] > mx ? v[o] : mx;
              return order_key(mx);
            },
            nold, 0u, 0u, 32, M - 1, -1, sh.ls, sh.sel, &thr);
      }
    }
    int32_t* po = pool_out + (int64_t)t * M;
    const int npool = r.nb > 0 ? cnt + 1 : 0;
    for (int i = tid; i < M; i += kFThreads) {
      int32_t v = -1;
      if (i < cnt) v = take_all ? i : sh.sel[i];
      else if (i == cnt && npool > 0) v = r.nb - 1;
      po[i] = v;
    }
    return;
  }
  }
  int cnt;
  if constexpr (cand) {
    cnt = list_select_g<kSmallPer>([&](int i) { return r.item_key(i); }, r.items(), 0u, 0u, 32, K, -1, sh.ls, sh.sel,
                                   &thr);
  } else {
    cnt = list_select_g<kSmallPer>([&](int j) { return order_key(r.scores[j]); }, r.n, 0u, 0u, 32, K, -1, sh.ls,
                                   sh.sel, &thr);
  }
  int32_t* tk = topk_out + (int64_t)t * K;
  for (int i = tid; i < K; i += kFThreads) {
    const int32_t p = i < cnt ? sh.sel[i] : -1;
    tk[i] = p < 0 ? -1 : (cand ? r.pool[p >> 3] * kBlock + (p & 7) : p);
  }
}

struct Layout {
  int32_t G, seg_b;
  size_t hist, cnt_a, cnt_b, ids_a, keys_a, ids_b, keys_b, bm, total;  // byte offsets
};

Layout make_layout(int32_t n_q, int32_t width, int32_t M, bool cand, bool rescore = false) {
  Layout L;
  const int64_t nbw = (width + kBlock - 1) / kBlock;
  const int64_t items = cand ? 8LL * M : nbw;
  L.G = (int32_t)((items + kSlice - 1) / kSlice);
  if (L.G < 1) L.G = 1;
  const size_t nq = (size_t)n_q, G = (size_t)L.G;
  L.hist = 0;
  L.cnt_a = L.hist + nq * kBins * 4;
  L.cnt_b = L.cnt_a + nq * G * 4;
  L.ids_a = L.cnt_b + nq * G * 4;
  L.keys_a = L.ids_a + nq * G * kSlice * 4;
  L.ids_b = L.keys_a + nq * G * kSlice * 4;
  L.seg_b = rescore ? kSlice * kBlock : kSegB;
  L.keys_b = L.ids_b + (cand ? 0 : nq * G * L.seg_b * 4);
  L.bm = L.keys_b + (cand ? 0 : nq * G * L.seg_b * 4);
  L.total = L.bm + (cand ? 0 : nq * (size_t)nbw * 4);
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

namespace csa2 {
namespace {

// Zeroes n 32-bit words (the histogram region of an allocation-free call; a kernel rather
// than a memset, so the call may be captured into a HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Argument checks of both selection entry points, before anything is launched or looked
// up; the workspace itself is checked by the caller.  kProceed: arguments valid, work to do.
constexpr int kProceed = 1;
int block_topk_check(const float* scores, const float* block_max, int32_t n_q, int32_t width, const int32_t* q_nvis,
                     const int32_t* pool_blocks, int32_t block, int32_t M, int32_t K, const int32_t* pool_out,
                     const int32_t* topk_out) {
  if (n_q < 0 || width < 0) return CSA2_ERR_INVALID_ARG;
  if (block != kBlock || M < 1 || M > kMaxPool || K < 1 || K > kMaxTopK) return CSA2_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  const bool cand = pool_blocks != nullptr;
  const bool want_topk = topk_out != nullptr;
  // pool-only mode (no Top-K): the pool from the caller's block scores; scores may be NULL
  if (!q_nvis || (want_topk ? !scores : (cand || !pool_out || !block_max))) return CSA2_ERR_INVALID_ARG;
  if (cand && (pool_out || block_max || (int64_t)width != 8LL * M)) return CSA2_ERR_INVALID_ARG;
  // a Full-mode Top-K is taken as the row's global Top-K, which is the Top-K inside the pool
  // only when the M - 1 older pool blocks' maxima alone outrank every entry outside the pool
  if (!cand && want_topk && M - 1 < K) return CSA2_ERR_UNSUPPORTED;
  if (n_q > 65535) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(block_max) |
       reinterpret_cast<uintptr_t>(topk_out) | reinterpret_cast<uintptr_t>(pool_out)) & 3)
    return CSA2_ERR_INVALID_ARG;
  if (make_layout(n_q, width, M, cand).G > kMaxG) return CSA2_ERR_UNSUPPORTED;  // rows longer than 2^20 blocks
  return kProceed;
}

// The three launches (after block_topk_check), shared by csa2_block_topk (the caller's
// workspace), csa2_block_topk_noalloc (the fixed scratch array, whose histogram region is
// cleared first) and csa2_block_topk_prebuilt (hist_ready: the histogram region already holds
// K1's counts, so K1 is skipped; the one-launch path for short rows clears the region instead).
int block_topk_launch(const float* scores, const float* block_max, int32_t n_q, int32_t width, const int32_t* q_nvis,
                      const int32_t* pool_blocks, int32_t M, int32_t K, int32_t* pool_out, int32_t* topk_out,
                      void* workspace, size_t ws_bytes, bool clear_hist, void* stream,
                      const Rescore* rsc = nullptr, bool hist_ready = false) {
  const bool cand = pool_blocks != nullptr;
  const bool want_topk = topk_out != nullptr;
  if (reinterpret_cast<uintptr_t>(workspace) & 3) return CSA2_ERR_INVALID_ARG;
  const Layout L = make_layout(n_q, width, M, cand, rsc != nullptr);
  if (!workspace || ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
  char* w = (char*)workspace;
  Ws ws;
  ws.hist = (uint32_t*)(w + L.hist);
  ws.cnt_a = (int32_t*)(w + L.cnt_a);
  ws.cnt_b = (int32_t*)(w + L.cnt_b);
  ws.ids_a = (int32_t*)(w + L.ids_a);
  ws.keys_a = (uint32_t*)(w + L.keys_a);
  ws.ids_b = (int32_t*)(w + L.ids_b);
  ws.keys_b = (uint32_t*)(w + L.keys_b);
  ws.bm = cand ? nullptr : (float*)(w + L.bm);
  ws.G = L.G;
  ws.seg_b = L.seg_b;
  const Rescore rs = rsc ? *rsc : Rescore{nullptr, nullptr, nullptr, nullptr};
  const float* bm = block_max ? block_max : ws.bm;
  const bool want_pool = pool_out != nullptr;
  hipStream_t s = (hipStream_t)stream;
  // short rows (every key fits in one workgroup's registers): the one-launch path
  const int64_t nbw = ((int64_t)width + kBlock - 1) / kBlock;
  const bool small = rsc == nullptr && (cand ? 8LL * M <= kSmallMax
                                              : (want_topk ? width <= kSmallMax : nbw - 1 <= kSmallMax));
  if (small) {
    const dim3 gs((!cand && want_pool && want_topk) ? 2 : 1, n_q);
    if (cand)
      hipLaunchKernelGGL(topk_small_kernel<true>, gs, dim3(kFThreads), 0, s, want_pool, want_topk, scores, block_max,
                         width, q_nvis, pool_blocks, M, K, pool_out, topk_out);
    else
      hipLaunchKernelGGL(topk_small_kernel<false>, gs, dim3(kFThreads), 0, s, want_pool, want_topk, scores, block_max,
                         width, q_nvis, pool_blocks, M, K, pool_out, topk_out);
    int st0 = check_launch();
    if (st0 != CSA2_OK || !hist_ready) return st0;
    const int64_t words = (int64_t)n_q * kBins;  // the prebuilt counts are not read: clear them
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, s, ws.hist, words);
    return check_launch();
  }
  if (clear_hist) {
    const int64_t words = (int64_t)n_q * kBins;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, s, ws.hist, words);
    const int st = check_launch();
    if (st != CSA2_OK) return st;
  }
  if (!hist_ready) {
    const bool wide = n_q >= kHWideRows;
    const int32_t sl = wide ? kHSliceWide : kHSlice;
    const int32_t G1 = (L.G * kSlice + sl - 1) / sl;
    const dim3 g1(G1, n_q), b1(wide ? kHThreadsWide : kHThreads);
    if (cand && wide)
      hipLaunchKernelGGL((topk_hist_kernel<true, kHSliceWide, kHThreadsWide>), g1, b1, 0, s, scores, block_max, width,
                         q_nvis, pool_blocks, M, K, ws);
    else if (cand)
      hipLaunchKernelGGL((topk_hist_kernel<true, kHSlice, kHThreads>), g1, b1, 0, s, scores, block_max, width, q_nvis,
                         pool_blocks, M, K, ws);
    else if (wide)
      hipLaunchKernelGGL((topk_hist_kernel<false, kHSliceWide, kHThreadsWide>), g1, b1, 0, s, scores, block_max, width,
                         q_nvis, pool_blocks, M, K, ws);
    else
      hipLaunchKernelGGL((topk_hist_kernel<false, kHSlice, kHThreads>), g1, b1, 0, s, scores, block_max, width, q_nvis,
                         pool_blocks, M, K, ws);
    const int st1 = check_launch();
    if (st1 != CSA2_OK) return st1;
  }
  int st = CSA2_OK;
  if (cand)
    hipLaunchKernelGGL(topk_collect_kernel<true>, dim3(L.G, n_q), dim3(kGThreads), 0, s, want_pool, want_topk, scores,
                       bm, width, q_nvis, pool_blocks, M, K, ws, rs);
  else if (rsc)
    hipLaunchKernelGGL((topk_collect_kernel<false, true>), dim3(L.G, n_q), dim3(kGThreads), 0, s, want_pool, want_topk,
                       scores, bm, width, q_nvis, pool_blocks, M, K, ws, rs);
  else
    hipLaunchKernelGGL(topk_collect_kernel<false>, dim3(L.G, n_q), dim3(kGThreads), 0, s, want_pool, want_topk, scores,
                       bm, width, q_nvis, pool_blocks, M, K, ws, rs);
  st = check_launch();
  if (st != CSA2_OK) return st;
  const dim3 gf((!cand && want_pool && want_topk) ? 2 : 1, n_q);
  if (cand)
    hipLaunchKernelGGL(topk_final_kernel<true>, gf, dim3(kFThreads), 0, s, want_pool, want_topk, scores, bm, width,
                       q_nvis, pool_blocks, M, K, ws, pool_out, topk_out);
  else if (rsc)
    hipLaunchKernelGGL((topk_final_kernel<false, true>), gf, dim3(kFThreads), 0, s, want_pool, want_topk, scores, bm,
                       width, q_nvis, pool_blocks, M, K, ws, pool_out, topk_out);
  else
    hipLaunchKernelGGL(topk_final_kernel<false>, gf, dim3(kFThreads), 0, s, want_pool, want_topk, scores, bm, width,
                       q_nvis, pool_blocks, M, K, ws, pool_out, topk_out);
  return check_launch();
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_block_topk(const float* scores, const float* block_max, int32_t n_q,
                               int32_t width, const int32_t* q_nvis, const int32_t* pool_blocks,
                               int32_t block, int32_t M, int32_t K, int32_t* pool_out,
                               int32_t* topk_out, void* workspace, size_t ws_bytes, void* stream) {
  const int st = csa2::block_topk_check(scores, block_max, n_q, width, q_nvis, pool_blocks, block, M, K, pool_out,
                                        topk_out);
  if (st != csa2::kProceed) return st;
  return csa2::block_topk_launch(scores, block_max, n_q, width, q_nvis, pool_blocks, M, K, pool_out, topk_out,
                                 workspace, ws_bytes, false, stream);
}

extern "C" int csa2_block_topk_prebuilt(const float* scores, const float* block_max, int32_t n_q, int32_t width,
                                        const int32_t* q_nvis, int32_t block, int32_t M, int32_t K, int32_t* pool_out,
                                        int32_t* topk_out, void* workspace, size_t ws_bytes, void* stream) {
  if (n_q > 0 && !block_max) return CSA2_ERR_INVALID_ARG;  // the counts were taken from these maxima
  const int st = csa2::block_topk_check(scores, block_max, n_q, width, q_nvis, nullptr, block, M, K, pool_out,
                                        topk_out);
  if (st != csa2::kProceed) return st;
  return csa2::block_topk_launch(scores, block_max, n_q, width, q_nvis, nullptr, M, K, pool_out, topk_out, workspace,
                                 ws_bytes, false, stream, nullptr, true);
}

extern "C" size_t csa2_block_topk_rescore_workspace(int32_t n_q, int32_t width, int32_t M, int32_t K) {
  (void)K;
  if (n_q <= 0 || width < 0 || M < 1) return 0;
  return csa2::make_layout(n_q, width, M, false, true).total;
}

extern "C" int csa2_block_topk_rescore(const float* block_max, int32_t n_q, int32_t width, const int32_t* q_nvis,
                                       const uint16_t* q_idx_bf16, const float* head_w, const uint8_t* idx_cache,
                                       const int64_t* q_base, int32_t M, int32_t K, int32_t* pool_out,
                                       int32_t* topk_out, void* workspace, size_t ws_bytes, void* stream) {
  using namespace csa2;
  if (n_q < 0 || width < 0) return CSA2_ERR_INVALID_ARG;
  if (M < 1 || M > kMaxPool || K < 1 || K > kMaxTopK || M - 1 < K) return CSA2_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!block_max || !q_nvis || !q_idx_bf16 || !head_w || !idx_cache || !q_base || !topk_out)
    return CSA2_ERR_INVALID_ARG;
  if (n_q > 65535 || width > kMaxIndexWidth) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_idx_bf16) | reinterpret_cast<uintptr_t>(idx_cache)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(block_max) | reinterpret_cast<uintptr_t>(head_w) |
       reinterpret_cast<uintptr_t>(topk_out) | reinterpret_cast<uintptr_t>(pool_out)) & 3)
    return CSA2_ERR_INVALID_ARG;
  if (make_layout(n_q, width, M, false, true).G > kMaxG) return CSA2_ERR_UNSUPPORTED;
  const Rescore rsc{q_idx_bf16, head_w, idx_cache, q_base};
  return block_topk_launch(nullptr, block_max, n_q, width, q_nvis, nullptr, M, K, pool_out, topk_out, workspace,
                           ws_bytes, false, stream, &rsc);
}

// ------------------------------------------------------------------ allocation-free variant
// csa2_block_topk for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid hipMalloc): its workspace is this fixed array, one copy per device,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.

static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<uintptr_t> scratch_addr[csa2::kMaxDevices];
std::mutex scratch_setup;

// The device address of `scratch` on the current device (0 on a HIP error), looked up on the
// device's first call with that device current.
uintptr_t scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= csa2::kMaxDevices) return 0;
  uintptr_t a = scratch_addr[dev].load(std::memory_order_acquire);
  if (a != 0) return a;
  std::lock_guard<std::mutex> lock(scratch_setup);
  a = scratch_addr[dev].load(std::memory_order_relaxed);
  if (a == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return 0;
    a = reinterpret_cast<uintptr_t>(ptr);
    scratch_addr[dev].store(a, std::memory_order_release);
  }
  return a;
}
}  // namespace

extern "C" int csa2_block_topk_noalloc(const float* scores, const float* block_max, int32_t n_q, int32_t width,
                                       const int32_t* q_nvis, const int32_t* pool_blocks, int32_t block, int32_t M,
                                       int32_t K, int32_t* pool_out, int32_t* topk_out, void* stream) {
  using namespace csa2;
  // argument errors first (the checks of csa2_block_topk), then the size limit, then set-up
  const int st = block_topk_check(scores, block_max, n_q, width, q_nvis, pool_blocks, block, M, K, pool_out,
                                  topk_out);
  if (st != kProceed) return st;
  if (csa2_block_topk_workspace(n_q, width, M, K) > (size_t)CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_ERR_SCRATCH;
  const uintptr_t a = scratch_address();
  if (a == 0) return CSA2_ERR_HIP;
  return block_topk_launch(scores, block_max, n_q, width, q_nvis, pool_blocks, M, K, pool_out, topk_out,
                           reinterpret_cast<void*>(a), CSA2_NOALLOC_SCRATCH_BYTES, true, stream);
}
