// sparse_attn.hip -- sparse latent attention over the selected FP4 entries joined with the
// sliding window, for gfx950.
//
// Follows [ZB] "把 KV Cache 压缩推到极致" §3.3.2.1 (key = value = c, the output is a convex
// combination of the selected content vectors) and §3.3.2 (one joint sparse attention
// over the selected main-KV entries and the layer's SWA KV).  FP4 is storage only: the
// entries are dequantised before the matmuls ([ZB] §2.4.4).
//
// Design.  A workgroup of 4 waves serves one query, 16 of its 64 heads and a run of its key
// chunks (64 keys each: the selected entries, gathered 288-byte rows, then the window rows);
// the chunks' rows are fetched a chunk ahead into registers and decoded once into one
// row-major bf16 LDS tile.  A query's chunks are split across workgroups (one chunk each at
// batch 4: the chain of dependent loads per workgroup stays short), each writing an
// unnormalised partial (o, m, l) that a merge kernel combines exactly like flash-decoding.
// From 8 queries on, one workgroup serves all 64 heads of a (query, split), so each chunk is
// decoded once per query; once the batch alone fills the CUs there are no splits.
// Every key value is exact in bf16: an E2M1 code times an E4M3 scale has at
// most 6 significant bits, an FP8 window value 4, a bf16 window value is one; the query is
// bf16 as given.  So QK^T has exact products for inputs of any magnitude, with fp32 sums.
//   QK^T  wave w scores keys 16w .. 16w + 15 of the chunk for the 16 heads
//         (v_mfma_f32_16x16x32_bf16, the query in registers as 16 A fragments).
//   softmax  online across chunks in fp32; the chunk's per-head maximum and the exponentials'
//         row sums are combined across the 4 waves through LDS in a fixed order, so every wave
//         holds the same running maximum and sum.
//   PV    wave w accumulates output dims 128w .. 128w + 127 over the chunk's 64 keys.  The
//         probabilities go to LDS as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi), which
//         represent p to about 2^-17 relative, and each part is one MFMA; the key-major value
//         operand comes from the same tile by transposing LDS reads (ds_read_b64_tr_b16).
// The grid spreads its work over all 8 XCDs (workgroups are dealt to them round-robin): a
// batch smaller than 8 queries must not leave XCDs idle while others run a second round of
// workgroups.  Without splits, a query's 4 head groups share an XCD and gather the same keys
// through its L2.
//
// The window rows come either as bf16 rows or as 584-byte FP8 window rows (the window KV
// kept in FP8, [ZB] §2.4.4; DeepSeek-V4's FP8 KV entry, [ZB] §3.1 and [DF] §4.6), read
// consecutively or from per-sequence ring buffers.
#include "csa2_device.hpp"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadGroup = 16;                   // heads per workgroup
constexpr int kGroups = kHeads / kHeadGroup;     // workgroups per query
constexpr int kChunk = 64;                       // keys per chunk
constexpr int kKStride = kD + 8;                 // bf16 per key row in LDS (1040 B: 8-B aligned rows)
constexpr int kPStride = kChunk + 8;             // bf16 per probability row
constexpr int kXcds = 8;
constexpr int kCUs = 256;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));  // 16 B at an 8-B boundary

struct __attribute__((aligned(16))) AttnShared {
  __bf16 k[kChunk * kKStride] __attribute__((aligned(16)));   // decoded keys, row-major [key][dim]
  __bf16 p[2][kHeadGroup * kPStride] __attribute__((aligned(16)));  // probabilities, hi and lo parts
  float cmax[kWaves][kHeadGroup];  // per wave: the chunk's maximum logit of each head
  float csum[kWaves][kHeadGroup];  // per wave: the chunk's exponential sum of each head
  int32_t valid[kChunk];
};

// The all-heads kernel's shared block: the same key tile, and each wave's own probabilities.
struct __attribute__((aligned(16))) WideShared {
  __bf16 k[kChunk * kKStride] __attribute__((aligned(16)));
  __bf16 p[kWaves][2][kHeadGroup * kPStride] __attribute__((aligned(16)));  // per wave: hi, lo
  int32_t valid[kChunk];
};

// Raw bytes of one key slot for one thread (a quarter of a key), fetched a chunk ahead: a
// selected entry's 64 payload bytes and 8 E4M3 scale bytes, or a window row's quarter (256
// bytes of bf16, or 144 bytes of an FP8 row: 112 code bytes, 32 bf16 bytes), with the FP8
// row's 8-byte scale word.  The scale words of both kinds sit in sw, so the loads that fill it
// write one place (different array slots made the compiler move the array to scratch).
struct KeyRaw {
  uint4 d[16];
  uint2 sw;
  int kind;  // 0 empty, 1 selected entry, 2 window row
};

__device__ __forceinline__ uint32_t bf16x2_of(float a, float b) {
  // both values are exact in bf16 here (at most 8 significant bits), so the rounding of the
  // conversion never acts
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Gather and decode of one query's keys: thread (kk, qq) handles quarter qq (dims 128 qq ..
// 128 qq + 127) of key slot kk of every 64-key chunk.  Keys 0 .. K-1 are the selected entries
// (topk ids relative to the sequence's first cache row), keys K .. K + nswa - 1 the window
// rows: bf16 rows, or 584-byte FP8 rows (kFp8Win), read consecutively or from per-sequence
// rings.
template <bool kFp8Win>
struct KeyStager {
  const uint8_t* kv_cache;
  const int32_t* topk_row;
  int32_t K;
  const void* swa_v;
  int64_t swa_ring;
  int64_t base, woff, wseg;
  int32_t nswa;
  int kk, qq;

  __device__ __forceinline__ KeyStager(const uint8_t* kv_cache_, const int32_t* topk, int32_t K_, const void* swa_v_,
                                       int64_t swa_ring_, int64_t base_, int64_t swa_start, int32_t swa_len, int tid)
      : kv_cache(kv_cache_), topk_row(topk), K(K_), swa_v(swa_v_), swa_ring(swa_ring_), base(base_) {
    nswa = min(max(swa_len, 0), kMaxSwa);
    // window row r lives at wseg + (woff + r) wrapped into the ring (no ring: wseg + woff + r)
    woff = swa_start;
    wseg = 0;
    if (swa_ring > 0) {
      woff %= swa_ring;
      if (woff < 0) woff += swa_ring;
      wseg = swa_start - woff;
    }
    // wave qq stages quarter qq of all 64 keys: consecutive lanes write consecutive key rows,
    // which start 4 banks apart, so the 16-byte LDS stores of a wave do not conflict
    kk = tid & 63;
    qq = tid >> 6;
  }

  // the selected-entry id of this thread's key slot in chunk c (a window row or past the end:
  // -1), read straight into a register so the key loads need no barrier
  __device__ __forceinline__ int32_t load_id(int c) const {
    const int x = c * kChunk + kk;
    return x < K ? topk_row[x] : -1;
  }

  // buffer row of window row r (wrapped inside the sequence's ring when there is one)
  __device__ __forceinline__ int64_t window_row(int r) const {
    int64_t row = woff + r;
    if (swa_ring > 0 && row >= swa_ring) row -= swa_ring;  // r < 128 <= swa_ring
    return row + wseg;
  }

  // raw loads of this thread's key quarter for chunk c (id: load_id(c))
  __device__ __forceinline__ void fetch(int c, int32_t id, KeyRaw& r) const {
    const int x = c * kChunk + kk;
    r.kind = 0;
    if (x < K) {
      if (id >= 0) {
        r.kind = 1;
        const uint8_t* row = kv_cache + (base + id) * kKvBytes;
#pragma unroll
        for (int v = 0; v < 4; v++) r.d[v] = reinterpret_cast<const uint4*>(row + 64 * qq)[v];
        const uint2 sw = *reinterpret_cast<const uint2*>(row + 256 + 8 * qq);
        r.sw = sw;
      }
    } else if (x - K < nswa) {
      r.kind = 2;
      const int64_t row = window_row(x - K);
      if constexpr (kFp8Win) {
        // NoPE codes of dims 112 qq .. 112 qq + 111, RoPE bf16 of dims 448 + 16 qq .. + 15, scales
        const uint8_t* src = static_cast<const uint8_t*>(swa_v) + row * kSwa8Bytes;
#pragma unroll
        for (int j = 0; j < 7; j++) {
          const u32x4_a8 v = *reinterpret_cast<const u32x4_a8*>(src + 112 * qq + 16 * j);
          r.d[j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const u32x4_a8 v = *reinterpret_cast<const u32x4_a8*>(src + kDNope + 32 * qq + 16 * j);
          r.d[7 + j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
        const uint2 sw = *reinterpret_cast<const uint2*>(src + kDNope + 2 * kDRope);
        r.sw = sw;
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(swa_v) + row * kD + 128 * qq);
#pragma unroll
        for (int v = 0; v < 16; v++) r.d[v] = src[v];
      }
    }
  }

  // decode to bf16 (exact) and store the key quarter row-major in LDS (sh: either
  // kernel's shared block, each with the key tile k and the slot flags valid)
  template <class Shared>
  __device__ __forceinline__ void stage(const KeyRaw& r, Shared& sh) const {
    __bf16* krow = sh.k + kk * kKStride + 128 * qq;
    if (r.kind == 1) {
      // the 8 E4M3 scales of this quarter: the codes convert at scale 1 (v_cvt_scalef32 applies
      // only a power-of-two scale) and each value is multiplied by its group's scale in fp32
      const uint32_t sw[2] = {r.sw.x, r.sw.y};
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const uint32_t wd[4] = {r.d[v].x, r.d[v].y, r.d[v].z, r.d[v].w};
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int grp = 2 * v + (q4 >> 1);  // local group of 16 dims
          const float S = e4m3_value((sw[grp >> 2] >> (8 * (grp & 3))) & 255u);
          const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q4], 1.0f, 0);
          const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q4], 1.0f, 1);
          const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q4], 1.0f, 2);
          const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q4], 1.0f, 3);
          *reinterpret_cast<uint4*>(krow + 32 * v + 8 * q4) =
              make_uint4(bf16x2_of(f0[0] * S, f0[1] * S), bf16x2_of(f1[0] * S, f1[1] * S), bf16x2_of(f2[0] * S, f2[1] * S),
                         bf16x2_of(f3[0] * S, f3[1] * S));
        }
      }
    } else if (r.kind == 2) {
      if constexpr (kFp8Win) {
        // this thread decodes NoPE dims 112 qq .. 112 qq + 111 (codes at the same byte
        // offsets) and RoPE dims 448 + 16 qq .. + 15 (bf16 at bytes 448 + 32 qq, copied)
        const uint64_t scb = (uint64_t)r.sw.x | ((uint64_t)r.sw.y << 32);
        __bf16* kq = sh.k + kk * kKStride;
#pragma unroll
        for (int j = 0; j < 7; j++) {
          const uint4 c4 = r.d[j];
          const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const int grp = (112 * qq + 16 * j + 8 * h) >> 6;  // scale group of these 8 dims
            const uint32_t code = (uint32_t)(scb >> (8 * grp)) & 255u;
            const float X = __builtin_ldexpf(1.0f, (int)code - 127);  // a power of two: exact
            const f32x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[2 * h], 1.0f, false);
            const f32x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[2 * h], 1.0f, true);
            const f32x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[2 * h + 1], 1.0f, false);
            const f32x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[2 * h + 1], 1.0f, true);
            *reinterpret_cast<uint4*>(kq + 112 * qq + 16 * j + 8 * h) =
                make_uint4(bf16x2_of(a0[0] * X, a0[1] * X), bf16x2_of(a1[0] * X, a1[1] * X),
                           bf16x2_of(a2[0] * X, a2[1] * X), bf16x2_of(a3[0] * X, a3[1] * X));
          }
        }
#pragma unroll
        for (int j = 0; j < 2; j++) *reinterpret_cast<uint4*>(kq + kDNope + 16 * qq + 8 * j) = r.d[7 + j];
      } else {
#pragma unroll
        for (int v = 0; v < 16; v++) *reinterpret_cast<uint4*>(krow + 8 * v) = r.d[v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; v++) *reinterpret_cast<uint4*>(krow + 8 * v) = make_uint4(0u, 0u, 0u, 0u);
    }
    if (qq == 0) sh.valid[kk] = r.kind != 0 ? 1 : 0;
  }
};

// Reductions over the 16 lanes of a DPP row (data movement on the VALU instead of LDS
// shuffles): rotations by 8 and 4 inside the row, then two quad permutations; every lane
// ends with the row's result.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, dpp<0x128>(v));    // row_ror:8
  v = __builtin_fmaxf(v, dpp<0x124>(v));    // row_ror:4
  v = __builtin_fmaxf(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
  return __builtin_fmaxf(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0xB1>(v);
  return v + dpp<0x4E>(v);
}

// Window rows: kFp8Win selects 584-byte FP8 rows instead of bf16 rows.
template <bool kFp8Win>
__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_cache,
    const int64_t* __restrict__ q_base, const int32_t* __restrict__ topk, int32_t K,
    const void* __restrict__ swa_v, int64_t swa_ring, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float scale, int32_t n_q, int32_t n_chunks, int32_t chunks_per_split,
    int32_t n_splits, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  __shared__ AttnShared sh;
  // workgroup -> (query, head group, split).  Workgroups are dealt to the 8 XCDs round-robin,
  // so slot j of XCD x is workgroup 8j + x.  A unit's workgroups take consecutive slots of one
  // XCD: with splits, a unit is a (query, head group) and its workgroups are the splits; without,
  // a unit is a query and its workgroups are the 4 head groups, which gather the same keys
  // through one L2.  Units go round-robin over the XCDs, so every XCD gets work even for a
  // batch of 1.
  const int L = blockIdx.x;
  const int x = L % kXcds, j = L / kXcds;
  const int per = n_splits > 1 ? n_splits : kGroups;
  const int unit = (j / per) * kXcds + x, k = j % per;
  const int t = n_splits > 1 ? unit / kGroups : unit;
  const int hg = n_splits > 1 ? unit % kGroups : k;
  const int split = n_splits > 1 ? k : 0;
  if (t >= n_q) return;
  const int c_begin = split * chunks_per_split;
  const int c_end = min(c_begin + chunks_per_split, n_chunks);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int h0 = kHeadGroup * hg;  // first head of the group
  KeyStager<kFp8Win> ks(kv_cache, topk + (int64_t)t * K, K, swa_v, swa_ring, q_base[t], swa_start[t], swa_len[t], tid);

  // Loads go out in dependency order so that their round trips overlap: this thread's entry
  // ids of the first two chunks, the query, then the first chunk's key rows.
  int32_t id_next = c_begin < c_end ? ks.load_id(c_begin) : -1;
  int32_t id_after = c_begin + 1 < c_end ? ks.load_id(c_begin + 1) : -1;
  __builtin_amdgcn_sched_barrier(0);
  // query fragments (A of QK^T): head h0 + i, dims 32s + 8g .. +7, bf16 as given
  bf16x8 qa[16];
  {
    const uint16_t* qh = q + ((int64_t)t * kHeads + h0 + i) * kD + 8 * g;
#pragma unroll
    for (int sd = 0; sd < 16; sd++) qa[sd] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qh + 32 * sd));
  }
  __builtin_amdgcn_sched_barrier(0);
  KeyRaw raw;
  if (c_begin < c_end) ks.fetch(c_begin, id_next, raw);

  f32x4 o[8];  // output dims 128w + 16dt + i, heads 4g + r
#pragma unroll
  for (int d = 0; d < 8; d++) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    m_run[r] = -__builtin_inff();
    l_run[r] = 0.0f;
  }

  for (int c = c_begin; c < c_end; c++) {
    __syncthreads();  // the previous chunk's LDS reads are done
    ks.stage(raw, sh);
    if (c + 1 < c_end) {  // the next chunk's gather overlaps this chunk's math
      ks.fetch(c + 1, id_after, raw);
      id_after = c + 2 < c_end ? ks.load_id(c + 2) : -1;
    }
    __syncthreads();

    // ---- S = Q K^T for keys 16w .. 16w + 15 of the chunk (lane: heads 4g + r, key 16w + i)
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 4) {
      bf16x8 kb[4];
#pragma unroll
      for (int sd = 0; sd < 4; sd++)
        kb[sd] = *reinterpret_cast<const bf16x8*>(sh.k + (16 * w + i) * kKStride + 32 * (s0 + sd) + 8 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sd = 0; sd < 4; sd++) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s0 + sd], kb[sd], sacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- the chunk's maximum per head across the 4 waves
    const bool ok = sh.valid[16 * w + i] != 0;
    float lg[4], cm[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      lg[r] = ok ? sacc[r] * scale : -__builtin_inff();
      cm[r] = row16_max(lg[r]);
    }
    if (i == 0) {
#pragma unroll
      for (int r = 0; r < 4; r++) sh.cmax[w][4 * g + r] = cm[r];
    }
    __syncthreads();
    float alpha[4], mn[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = 4 * g + r;
      const float cmx = __builtin_fmaxf(__builtin_fmaxf(sh.cmax[0][h], sh.cmax[1][h]),
                                        __builtin_fmaxf(sh.cmax[2][h], sh.cmax[3][h]));
      mn[r] = __builtin_fmaxf(m_run[r], cmx);
      alpha[r] = (mn[r] == -__builtin_inff()) ? 1.0f : __expf(m_run[r] - mn[r]);
    }
    // ---- probabilities of this wave's 16 keys, as bf16 hi + lo parts, and their row sums
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float p = (lg[r] == -__builtin_inff()) ? 0.0f : __expf(lg[r] - mn[r]);
      const __bf16 hi = (__bf16)p;
      const __bf16 lo = (__bf16)(p - (float)hi);
      sh.p[0][(4 * g + r) * kPStride + 16 * w + i] = hi;
      sh.p[1][(4 * g + r) * kPStride + 16 * w + i] = lo;
      ps[r] = row16_sum(p);
    }
    if (i == 0) {
#pragma unroll
      for (int r = 0; r < 4; r++) sh.csum[w][4 * g + r] = ps[r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = 4 * g + r;
      l_run[r] = l_run[r] * alpha[r] + (((sh.csum[0][h] + sh.csum[1][h]) + sh.csum[2][h]) + sh.csum[3][h]);
      m_run[r] = mn[r];
    }
    // rescale O only when some head's running maximum moved (later chunks rarely move it)
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f || alpha[2] != 1.0f || alpha[3] != 1.0f)) {
#pragma unroll
      for (int d = 0; d < 8; d++) {
#pragma unroll
        for (int r = 0; r < 4; r++) o[d][r] *= alpha[r];
      }
    }
    // ---- O[:, 128w ..] += P V over the chunk's 64 keys: A = P [head i][keys 32ks + 8g ..],
    // B = V [keys][dim 128w + 16dt + i] by two transposing LDS reads of 4 keys each
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ks2++) {
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(&sh.p[0][i * kPStride + 32 * ks2 + 8 * g]);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(&sh.p[1][i * kPStride + 32 * ks2 + 8 * g]);
      const int kb0 = 32 * ks2 + 8 * g + (i >> 2);
      s16x4 lo4[8], hi4[8];
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const __bf16* p0 = sh.k + kb0 * kKStride + 128 * w + 16 * dt + 4 * (i & 3);
        lo4[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0));
        hi4[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0 + 4 * kKStride));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4[dt], hi4[dt], 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[dt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: lane holds O[head h0 + 4g + r][dim 128w + 16dt + i]; rows of 16 floats.
  // One split: the normalised output and lse.  Several: this split's unnormalised o and its
  // (m, l) per head, slot (t, split, head) of the workspace.
  const bool single = n_splits == 1;
  const int64_t slot = (int64_t)t * n_splits + split;
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; r++) inv[r] = single ? (l_run[r] > 0.0f ? 1.0f / l_run[r] : 0.0f) : 1.0f;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int h = h0 + 4 * g + r;
    float* orow = (single ? out + ((int64_t)t * kHeads + h) * kD : ws_o + (slot * kHeads + h) * kD) + 128 * w + i;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) orow[16 * dt] = o[dt][r] * inv[r];
  }
  if (w == 0 && i == 0) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = h0 + 4 * g + r;
      if (!single) {
        ws_ml[(slot * kHeads + h) * 2 + 0] = m_run[r];
        ws_ml[(slot * kHeads + h) * 2 + 1] = l_run[r];
      } else if (lse != nullptr) {
        lse[(int64_t)t * kHeads + h] = l_run[r] > 0.0f ? m_run[r] + __logf(l_run[r]) : -__builtin_inff();
      }
    }
  }
}

// All 64 heads of a query in one workgroup, every chunk of its keys: wave w owns heads
// 16w .. 16w + 15 and all 512 output dims, so the 4 waves share one decoded key tile per
// chunk and each runs its softmax alone (no cross-wave exchange, two barriers per chunk).
// Used when the batch alone fills the GPU (no key splits), where a quarter of the
// workgroups, each decoding a chunk once for 64 heads, beats one workgroup per head group.
// The arithmetic per (head, key) is the head-group kernel's: exact bf16 QK^T products,
// fp32 sums, online fp32 softmax, P as bf16 hi + lo parts in PV.
template <bool kFp8Win>
__global__ __launch_bounds__(kThreads) void sparse_attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_cache,
    const int64_t* __restrict__ q_base, const int32_t* __restrict__ topk, int32_t K,
    const void* __restrict__ swa_v, int64_t swa_ring, const int64_t* __restrict__ swa_start,
    const int32_t* __restrict__ swa_len, float scale, int32_t n_q, int32_t n_chunks, int32_t chunks_per_split,
    int32_t n_splits, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  __shared__ WideShared sh;
  // workgroup -> (query, split): a query's splits take consecutive slots of one XCD (slot j
  // of XCD x is workgroup 8j + x) and queries go round-robin over the XCDs
  const int L = blockIdx.x;
  const int x = L % kXcds, j = L / kXcds;
  const int t = (j / n_splits) * kXcds + x, split = j % n_splits;
  if (t >= n_q) return;
  const int c_begin = split * chunks_per_split;
  const int c_end = min(c_begin + chunks_per_split, n_chunks);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  KeyStager<kFp8Win> ks(kv_cache, topk + (int64_t)t * K, K, swa_v, swa_ring, q_base[t], swa_start[t], swa_len[t], tid);

  int32_t id_next = c_begin < c_end ? ks.load_id(c_begin) : -1;
  int32_t id_after = c_begin + 1 < c_end ? ks.load_id(c_begin + 1) : -1;
  __builtin_amdgcn_sched_barrier(0);
  // query fragments (A of QK^T): head 16w + i, dims 32s + 8g .. +7, bf16 as given
  bf16x8 qa[16];
  {
    const uint16_t* qh = q + ((int64_t)t * kHeads + 16 * w + i) * kD + 8 * g;
#pragma unroll
    for (int sd = 0; sd < 16; sd++) qa[sd] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qh + 32 * sd));
  }
  __builtin_amdgcn_sched_barrier(0);
  KeyRaw raw;
  if (c_begin < c_end) ks.fetch(c_begin, id_next, raw);

  f32x4 o[32];  // output dims 16dt + i, heads 16w + 4g + r
#pragma unroll
  for (int d = 0; d < 32; d++) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    m_run[r] = -__builtin_inff();
    l_run[r] = 0.0f;
  }
  __bf16* ph_w = sh.p[w][0];
  __bf16* pl_w = sh.p[w][1];

  for (int c = c_begin; c < c_end; c++) {
    __syncthreads();  // the previous chunk's LDS reads are done
    ks.stage(raw, sh);
    if (c + 1 < c_end) {  // the next chunk's gather overlaps this chunk's math
      ks.fetch(c + 1, id_after, raw);
      id_after = c + 2 < c_end ? ks.load_id(c + 2) : -1;
    }
    __syncthreads();

    // ---- S = Q K^T for the chunk's 4 tiles of 16 keys (lane: heads 4g + r, key 16kt + i)
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 2) {
      bf16x8 kb[2][4];
#pragma unroll
      for (int sd = 0; sd < 2; sd++) {
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
          kb[sd][kt] = *reinterpret_cast<const bf16x8*>(sh.k + (16 * kt + i) * kKStride + 32 * (s0 + sd) + 8 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sd = 0; sd < 2; sd++) {
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s0 + sd], kb[sd][kt], sacc[kt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- online softmax over the chunk, within the wave
    float lg[4][4], cm[4];
#pragma unroll
    for (int r = 0; r < 4; r++) cm[r] = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      const bool ok = sh.valid[16 * kt + i] != 0;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        lg[kt][r] = ok ? sacc[kt][r] * scale : -__builtin_inff();
        cm[r] = __builtin_fmaxf(cm[r], lg[kt][r]);
      }
    }
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float mn = __builtin_fmaxf(m_run[r], row16_max(cm[r]));
      alpha[r] = (mn == -__builtin_inff()) ? 1.0f : __expf(m_run[r] - mn);
      float rs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        const float pr = (lg[kt][r] == -__builtin_inff()) ? 0.0f : __expf(lg[kt][r] - mn);
        const __bf16 hi = (__bf16)pr;
        const __bf16 lo = (__bf16)(pr - (float)hi);
        ph_w[(4 * g + r) * kPStride + 16 * kt + i] = hi;
        pl_w[(4 * g + r) * kPStride + 16 * kt + i] = lo;
        rs += pr;
      }
      l_run[r] = l_run[r] * alpha[r] + row16_sum(rs);
      m_run[r] = mn;
    }
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f || alpha[2] != 1.0f || alpha[3] != 1.0f)) {
#pragma unroll
      for (int d = 0; d < 32; d++) {
#pragma unroll
        for (int r = 0; r < 4; r++) o[d][r] *= alpha[r];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's P stores are in LDS
    __builtin_amdgcn_wave_barrier();
    // ---- O += P V over the chunk's 64 keys: A = P [head i][keys 32ks + 8g ..] (hi, lo),
    // B = V [keys][dim 16dt + i] by two transposing LDS reads of 4 keys each
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ks2++) {
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(ph_w + i * kPStride + 32 * ks2 + 8 * g);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(pl_w + i * kPStride + 32 * ks2 + 8 * g);
      const int kb0 = 32 * ks2 + 8 * g + (i >> 2);
#pragma unroll
      for (int dt0 = 0; dt0 < 32; dt0 += 8) {
        s16x4 lo4[8], hi4[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const __bf16* p0 = sh.k + kb0 * kKStride + 16 * (dt0 + u) + 4 * (i & 3);
          lo4[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0));
          hi4[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0 + 4 * kKStride));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4[u], hi4[u], 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, o[dt0 + u], 0, 0, 0);
          o[dt0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[dt0 + u], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: lane holds O[head 16w + 4g + r][dim 16dt + i].  One split: the normalised
  // output and lse.  Several: this split's unnormalised o and its (m, l) per head, slot
  // (t, split, head) of the workspace.  The rows go out through the idle key tile: each wave
  // stages its 16 heads x 256 dims in fp32, then reads whole rows back as float4, so every
  // global store instruction writes 1 KB.
  const bool single = n_splits == 1;
  const int64_t slot = (int64_t)t * n_splits + split;
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; r++) inv[r] = single ? (l_run[r] > 0.0f ? 1.0f / l_run[r] : 0.0f) : 1.0f;
  if (i == 0) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = 16 * w + 4 * g + r;
      if (!single) {
        ws_ml[(slot * kHeads + h) * 2 + 0] = m_run[r];
        ws_ml[(slot * kHeads + h) * 2 + 1] = l_run[r];
      } else if (lse != nullptr) {
        lse[(int64_t)t * kHeads + h] = l_run[r] > 0.0f ? m_run[r] + __logf(l_run[r]) : -__builtin_inff();
      }
    }
  }
  constexpr int kOStride = 256 + 4;  // floats per staged row (the padding spreads the banks)
  static_assert(kWaves * 16 * kOStride * 4 <= (int)sizeof(sh.k), "staged rows fit in the key tile");
  float* stage_o = reinterpret_cast<float*>(sh.k) + w * 16 * kOStride;
  float* orow0 = (single ? out + (int64_t)t * kHeads * kD : ws_o + slot * kHeads * kD) + (int64_t)16 * w * kD;
  __syncthreads();  // every wave is done reading the key tile
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int dt = 0; dt < 16; dt++) {
#pragma unroll
      for (int r = 0; r < 4; r++) stage_o[(4 * g + r) * kOStride + 16 * dt + i] = o[16 * half + dt][r] * inv[r];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows are in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int row = 0; row < 16; row++) {
      const float4 v = *reinterpret_cast<const float4*>(stage_o + row * kOStride + 4 * lane);
      *reinterpret_cast<float4*>(orow0 + (int64_t)row * kD + 256 * half + 4 * lane) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next half overwrites the rows
    __builtin_amdgcn_wave_barrier();
  }
}

// Combine the split partials of one (query, head): out = sum_s o_s e^(m_s - M) / L.  Every
// split's (m, l) and o slice load at once (splits <= kMaxSplits), then one pass combines.
constexpr int kMaxSplits = (kMaxTopK + kMaxSwa + kChunk - 1) / kChunk;

// kUnitHeads: heads per unit of the attention launch, 16 for the head-group kernel (a unit is a
// (query, head group)), 64 for the all-heads kernel (a unit is a query).
template <int kUnitHeads>
__global__ __launch_bounds__(128) void sparse_attn_merge_kernel(const float* __restrict__ ws_o,
                                                                const float* __restrict__ ws_ml,
                                                                int32_t n_splits, int32_t n_q,
                                                                float* __restrict__ out,
                                                                float* __restrict__ lse) {
  // workgroup -> (query, head) on the XCD that ran the head's unit in the attention launch (the
  // same dealing: slot j of XCD x, kUnitHeads heads per unit), so the partials it reads were
  // written through that XCD's L2
  constexpr int kUnitsPerQuery = kHeads / kUnitHeads;
  const int L = blockIdx.x, x = L % kXcds, j = L / kXcds;
  const int unit = (j / kUnitHeads) * kXcds + x;
  const int t = unit / kUnitsPerQuery, h = (unit % kUnitsPerQuery) * kUnitHeads + j % kUnitHeads, tid = threadIdx.x;
  if (t >= n_q) return;
  float m[kMaxSplits], l[kMaxSplits];
  float4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    if (s < n_splits) {
      const int64_t slot = ((int64_t)t * n_splits + s) * kHeads + h;
      const float2 ml = *reinterpret_cast<const float2*>(ws_ml + slot * 2);
      m[s] = ml.x;
      l[s] = ml.y;
      v[s] = reinterpret_cast<const float4*>(ws_o + slot * kD)[tid];
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++)
    if (s < n_splits && l[s] > 0.0f) M = __builtin_fmaxf(M, m[s]);
  float Lsum = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    if (s < n_splits && l[s] > 0.0f) {
      const float e = __expf(m[s] - M);
      Lsum += l[s] * e;
      acc.x += v[s].x * e;
      acc.y += v[s].y * e;
      acc.z += v[s].z * e;
      acc.w += v[s].w * e;
    }
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  reinterpret_cast<float4*>(out + ((int64_t)t * kHeads + h) * kD)[tid] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse != nullptr && tid == 0) lse[(int64_t)t * kHeads + h] = Lsum > 0.0f ? M + __logf(Lsum) : -__builtin_inff();
}

// How a query's chunks are split.  From kWideFrom queries on, the all-heads kernel: one
// workgroup per (query, split), each chunk decoded once for all 64 heads, with as many splits
// as fill the CUs once (none once the batch alone fills them).  Below, the head-group kernel:
// 4 workgroups per (query, split), at most one workgroup per CU (a workgroup's registers
// and LDS allow one per CU), all of them running at once -- one chunk each at batch 4.
constexpr int32_t kWideFrom = 8;

struct Plan {
  int32_t n_chunks, chunks_per_split, n_splits;
  bool wide;
};

Plan make_plan(int32_t n_q, int32_t K) {
  Plan p;
  p.n_chunks = (K + kMaxSwa + kChunk - 1) / kChunk;
  p.wide = n_q >= kWideFrom;
  const int32_t wgs = (p.wide ? 1 : kGroups) * (n_q > 0 ? n_q : 1);
  int32_t want = kCUs / wgs;
  if (want < 1) want = 1;
  if (want > p.n_chunks) want = p.n_chunks;
  p.chunks_per_split = (p.n_chunks + want - 1) / want;
  p.n_splits = (p.n_chunks + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

}  // namespace
}  // namespace csa2

extern "C" size_t csa2_sparse_attn_workspace(int32_t n_q, int32_t K) {
  using namespace csa2;
  if (n_q <= 0 || K < 0) return 0;
  const Plan p = make_plan(n_q, K);
  if (p.n_splits <= 1) return 0;
  return (size_t)n_q * p.n_splits * kHeads * (kD + 2) * sizeof(float);
}

namespace csa2 {
namespace {

template <bool kFp8Win>
int launch_sparse_attn(const uint16_t* q_bf16, const uint8_t* kv_cache, const int64_t* q_base,
                       const int32_t* topk, int32_t K, const void* swa, int64_t swa_ring,
                       const int64_t* swa_start, const int32_t* swa_len, float scale, float* out,
                       float* lse, int32_t n_q, void* workspace, size_t ws_bytes, void* stream) {
  if (n_q < 0 || K < 0 || swa_ring < 0) return CSA2_ERR_INVALID_ARG;
  if (swa_ring > 0 && swa_ring < kMaxSwa) return CSA2_ERR_INVALID_ARG;  // a ring holds the window
  if (K > kMaxTopK) return CSA2_ERR_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!q_bf16 || !kv_cache || !q_base || !swa || !swa_start || !swa_len || !out)
    return CSA2_ERR_INVALID_ARG;
  if (K > 0 && !topk) return CSA2_ERR_INVALID_ARG;
  if (n_q > (1 << 24)) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_bf16) | reinterpret_cast<uintptr_t>(kv_cache) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(swa) & (kFp8Win ? 7 : 15)) return CSA2_ERR_INVALID_ARG;
  const Plan p = make_plan(n_q, K);
  const size_t need = csa2_sparse_attn_workspace(n_q, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  float* ws_o = (float*)workspace;
  float* ws_ml = need > 0 ? ws_o + (size_t)n_q * p.n_splits * kHeads * kD : nullptr;
  // units (see the kernels) rounded up to whole rows of 8, times the workgroups per unit: the
  // all-heads kernel's unit is a query with its splits; the head-group kernel's is a (query,
  // head group) with its splits, or without splits a query with its 4 head groups
  const bool hg_units = !p.wide && p.n_splits > 1;
  const int64_t units = hg_units ? (int64_t)n_q * kGroups : (int64_t)n_q;
  const int64_t per = (p.wide || hg_units) ? p.n_splits : kGroups;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * per;
  if (grid > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  if (p.wide)
    hipLaunchKernelGGL(sparse_attn_wide_kernel<kFp8Win>, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       q_bf16, kv_cache, q_base, topk, K, swa, swa_ring, swa_start, swa_len, scale, n_q, p.n_chunks,
                       p.chunks_per_split, p.n_splits, out, lse, ws_o, ws_ml);
  else
    hipLaunchKernelGGL(sparse_attn_kernel<kFp8Win>, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       q_bf16, kv_cache, q_base, topk, K, swa, swa_ring, swa_start, swa_len, scale, n_q, p.n_chunks,
                       p.chunks_per_split, p.n_splits, out, lse, ws_o, ws_ml);
  int st = check_launch();
  if (st != CSA2_OK || p.n_splits <= 1) return st;
  const int64_t merge_grid = (units + kXcds - 1) / kXcds * kXcds * (p.wide ? kHeads : kHeadGroup);
  if (p.wide)
    hipLaunchKernelGGL(sparse_attn_merge_kernel<kHeads>, dim3((unsigned)merge_grid), dim3(128), 0, (hipStream_t)stream,
                       ws_o, ws_ml, p.n_splits, n_q, out, lse);
  else
    hipLaunchKernelGGL(sparse_attn_merge_kernel<kHeadGroup>, dim3((unsigned)merge_grid), dim3(128), 0,
                       (hipStream_t)stream, ws_o, ws_ml, p.n_splits, n_q, out, lse);
  return check_launch();
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_sparse_attn(const uint16_t* q_bf16, const uint8_t* kv_cache,
                                const int64_t* q_base, const int32_t* topk, int32_t K,
                                const uint16_t* swa_bf16, const int64_t* swa_start,
                                const int32_t* swa_len, float scale, float* out, float* lse,
                                int32_t n_q, void* workspace, size_t ws_bytes, void* stream) {
  return csa2::launch_sparse_attn<false>(q_bf16, kv_cache, q_base, topk, K, swa_bf16, 0, swa_start, swa_len, scale,
                                         out, lse, n_q, workspace, ws_bytes, stream);
}

extern "C" int csa2_sparse_attn_swa_fp8(const uint16_t* q_bf16, const uint8_t* kv_cache,
                                        const int64_t* q_base, const int32_t* topk, int32_t K,
                                        const uint8_t* swa8, int64_t swa_ring,
                                        const int64_t* swa_start, const int32_t* swa_len, float scale,
                                        float* out, float* lse, int32_t n_q, void* workspace,
                                        size_t ws_bytes, void* stream) {
  return csa2::launch_sparse_attn<true>(q_bf16, kv_cache, q_base, topk, K, swa8, swa_ring, swa_start, swa_len, scale,
                                        out, lse, n_q, workspace, ws_bytes, stream);
}
