// sparse_attn.hip -- sparse latent attention over the selected FP4 entries joined with the
// sliding window, for gfx950.
//
// Follows [ZB] "把 KV Cache 压缩推到极致" §3.3.2.1 (key = value = c, the output is a convex
// combination of the selected content vectors) and §3.3.2 (one joint sparse attention
// over the selected main-KV entries and the layer's SWA KV).  FP4 is storage only: the
// entries are dequantised before the matmuls ([ZB] §2.4.4).
//
// Design.  A workgroup of 4 waves serves one query; wave w owns heads 16w .. 16w+15.
// Keys are processed in chunks of 64: the selected entries (gathered 288-byte rows,
// prefetched one chunk ahead) and the window rows are decoded once into LDS as f16, row
// major (exact: an E2M1 code times an E4M3 scale has at most 6 significant bits; bf16
// window values are exact in f16's normal range).  QK^T reads the key rows directly; PV
// takes its key-major operand from the same tile with transposing LDS reads
// (ds_read_b64_tr_b16), so no second copy is stored.  Both matmuls run on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation; the softmax is online across chunks in
// fp32.  For small batches the key chunks of a query are split across workgroups and a
// merge kernel combines the partial (o, m, l) exactly like flash-decoding.
//
// The window rows come either as bf16 rows or as 584-byte FP8 window rows (the window KV
// kept in FP8, [ZB] §2.4.4; DeepSeek-V4's FP8 KV entry, [ZB] §3.1 and [DF] §4.6), read
// consecutively or from per-sequence ring buffers.  An FP8 row decodes exactly into f16
// (an E4M3 value times a power-of-two scale has 4 significant bits) as long as the
// products stay in f16's range (groups with amax >= 2^-10 or so; smaller groups lose their
// smallest values to f16 underflow).
#include "csa2_device.hpp"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 64;
constexpr int kKStride = kD + 8;        // f16 elements per key row in LDS (1040 B: 8-B aligned rows)
constexpr int kPStride = kChunk + 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));  // 16 B at an 8-B boundary


struct __attribute__((aligned(16))) AttnShared {
  _Float16 k[kChunk * kKStride] __attribute__((aligned(16)));  // decoded keys, row-major [key][dim]
  _Float16 p[kWaves * 16 * kPStride] __attribute__((aligned(16)));  // per-wave probabilities [head][key]
  int32_t valid[kChunk];
};

// Raw bytes of one key slot for one thread (a quarter of a key), prefetched a chunk ahead:
// a selected entry's 64 payload bytes and 8 E4M3 scale bytes, or a window row's quarter
// (256 bytes of bf16, or 144 bytes of an FP8 row: 112 code bytes, 32 bf16 bytes), with the
// FP8 row's 8-byte scale word.  The scale words of both kinds sit in sw, so the two loads
// that fill it write one place (with different array slots the compiler merged them into
// a store at a computed index, which put the array in scratch memory).
struct KeyRaw {
  uint4 d[16];
  uint2 sw;
  int kind;       // 0 empty, 1 selected entry, 2 window row
};

// Gather and decode of one query's keys: thread (kk, qq) of a 256-thread workgroup handles
// quarter qq (dims 128 qq .. 128 qq + 127) of key slot kk of every 64-key chunk.  Keys 0 .. K-1 are the selected entries
// (topk ids relative to the sequence's first cache row), keys K .. K + nswa - 1 the window
// rows.  Window rows are bf16 rows, or 584-byte FP8 rows (kFp8Win), read consecutively or
// from per-sequence rings.
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
    // wave qq stages quarter qq of all 64 keys: consecutive lanes write consecutive key
    // rows, which start 4 banks apart, so the 16-byte LDS stores of a wave do not conflict
    kk = tid & 63;
    qq = tid >> 6;
  }

  // the selected-entry id of this thread's key slot in chunk c (a window row or past the
  // end: -1), read straight into a register so the key loads need no barrier
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

  // decode to f16 (exact) and store the key quarter row-major in LDS
  __device__ __forceinline__ void stage(const KeyRaw& r, AttnShared& sh) const {
    _Float16* krow = sh.k + kk * kKStride + 128 * qq;
    if (r.kind == 1) {
      // v_cvt_scalef32_pk_f16_fp4 applies only a power-of-two scale, so the codes convert
      // at scale 1 and a packed f16 multiply applies the E4M3 scale (exact: at most 6
      // significant bits, inside f16's normal range)
      // the 8 E4M3 scales of this quarter as f16 (every E4M3 value is exact in f16)
      f16x2 sc2[4];
      sc2[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sw.x, 1.0f, false);
      sc2[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sw.x, 1.0f, true);
      sc2[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sw.y, 1.0f, false);
      sc2[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sw.y, 1.0f, true);
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const uint32_t wd[4] = {r.d[v].x, r.d[v].y, r.d[v].z, r.d[v].w};
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int grp = 2 * v + (q4 >> 1);  // local group of 16 dims
          const _Float16 S = sc2[grp >> 1][grp & 1];
          const f16x2 S2 = {S, S};
          const f16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q4], 1.0f, 0) * S2;
          const f16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q4], 1.0f, 1) * S2;
          const f16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q4], 1.0f, 2) * S2;
          const f16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q4], 1.0f, 3) * S2;
          const f16x8 pk = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
          *reinterpret_cast<f16x8*>(krow + 32 * v + 8 * q4) = pk;
        }
      }
    } else if (r.kind == 2) {
      if constexpr (kFp8Win) {
        // this thread decodes NoPE dims 112 qq .. 112 qq + 111 (codes at the same byte
        // offsets) and RoPE dims 448 + 16 qq .. + 15 (bf16 at bytes 448 + 32 qq)
        const uint64_t scb = (uint64_t)r.sw.x | ((uint64_t)r.sw.y << 32);
        _Float16* kq = sh.k + kk * kKStride;
#pragma unroll
        for (int j = 0; j < 7; j++) {
          const uint4 c4 = r.d[j];
          const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const int grp = (112 * qq + 16 * j + 8 * h) >> 6;  // scale group of these 8 dims
            const uint32_t code = (uint32_t)(scb >> (8 * grp)) & 255u;
            const _Float16 X = (_Float16)__builtin_ldexpf(1.0f, (int)code - 127);
            const f16x2 X2 = {X, X};
            const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[2 * h], 1.0f, false) * X2;
            const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[2 * h], 1.0f, true) * X2;
            const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[2 * h + 1], 1.0f, false) * X2;
            const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[2 * h + 1], 1.0f, true) * X2;
            const f16x8 pk = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
            *reinterpret_cast<f16x8*>(kq + 112 * qq + 16 * j + 8 * h) = pk;
          }
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const uint4 u4 = r.d[7 + j];
          const uint32_t u[4] = {u4.x, u4.y, u4.z, u4.w};
          f16x8 pk;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            pk[2 * e] = (_Float16)bf16_bits_to_f32(u[e] & 0xFFFFu);
            pk[2 * e + 1] = (_Float16)bf16_bits_to_f32(u[e] >> 16);
          }
          *reinterpret_cast<f16x8*>(kq + kDNope + 16 * qq + 8 * j) = pk;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const uint32_t wd[4] = {r.d[v].x, r.d[v].y, r.d[v].z, r.d[v].w};
          f16x8 pk;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            pk[2 * e] = (_Float16)bf16_bits_to_f32(wd[e] & 0xFFFFu);
            pk[2 * e + 1] = (_Float16)bf16_bits_to_f32(wd[e] >> 16);
          }
          *reinterpret_cast<f16x8*>(krow + 8 * v) = pk;
        }
      }
    } else {
      f16x8 z;
#pragma unroll
      for (int e = 0; e < 8; e++) z[e] = (_Float16)0.0f;
#pragma unroll
      for (int v = 0; v < 16; v++) *reinterpret_cast<f16x8*>(krow + 8 * v) = z;
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
    const int32_t* __restrict__ swa_len, float scale, int32_t n_chunks, int32_t chunks_per_split,
    int32_t n_splits, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  __shared__ AttnShared sh;
  const int t = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int c_begin = split * chunks_per_split;
  const int c_end = min(c_begin + chunks_per_split, n_chunks);
  KeyStager<kFp8Win> ks(kv_cache, topk + (int64_t)t * K, K, swa_v, swa_ring, q_base[t], swa_start[t], swa_len[t],
                         tid);

  // Loads go out in dependency order so that their round trips overlap: this thread's
  // entry ids of the first two chunks, the query, then the first chunk's key rows (which
  // wait only for the first id), and the query is converted after the key loads are out.
  int32_t id_next = c_begin < c_end ? ks.load_id(c_begin) : -1;
  int32_t id_after = c_begin + 1 < c_end ? ks.load_id(c_begin + 1) : -1;
  __builtin_amdgcn_sched_barrier(0);
  // query fragments: head 16w + i, dims 32s + 8g .. +7, as f16 (exact in the normal range)
  uint4 qraw[16];
  {
    const uint16_t* qh = q + ((int64_t)t * kHeads + 16 * w + i) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; s++) qraw[s] = *reinterpret_cast<const uint4*>(qh + 32 * s);
  }
  __builtin_amdgcn_sched_barrier(0);
  KeyRaw raw;
  if (c_begin < c_end) ks.fetch(c_begin, id_next, raw);
  __builtin_amdgcn_sched_barrier(0);
  f16x8 qa[16];
#pragma unroll
  for (int s = 0; s < 16; s++) {
    const uint32_t wd[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
    for (int v = 0; v < 4; v++) {
      qa[s][2 * v] = (_Float16)bf16_bits_to_f32(wd[v] & 0xFFFFu);
      qa[s][2 * v + 1] = (_Float16)bf16_bits_to_f32(wd[v] >> 16);
    }
  }

  f32x4 o[32];
#pragma unroll
  for (int d = 0; d < 32; d++) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    m_run[r] = -__builtin_inff();
    l_run[r] = 0.0f;
  }

  for (int c = c_begin; c < c_end; c++) {
    __syncthreads();  // the previous chunk's LDS reads are done
    ks.stage(raw, sh);
    if (c + 1 < c_end) {  // next chunk's gather overlaps this chunk's math; its id was loaded a chunk ago
      ks.fetch(c + 1, id_after, raw);
      id_after = c + 2 < c_end ? ks.load_id(c + 2) : -1;
    }
    __syncthreads();

    // ---- S = Q K^T for 4 tiles of 16 keys
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // groups of 4 dim steps: the group's 16 B fragments are read before its 16 MFMAs, so the
    // reads overlap one another instead of each MFMA waiting for its own LDS round trip
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 4) {
      f16x8 kb[4][4];
#pragma unroll
      for (int s = 0; s < 4; s++) {
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
          kb[s][kt] = *reinterpret_cast<const f16x8*>(sh.k + (16 * kt + i) * kKStride + 32 * (s0 + s) + 8 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; s++) {
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[s0 + s], kb[s][kt], sacc[kt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- online softmax over this chunk; lane holds rows (heads) 4g + r, column (key) 16kt + i
    float pv[4][4];
    float cmax[4];
#pragma unroll
    for (int r = 0; r < 4; r++) cmax[r] = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      const bool ok = sh.valid[16 * kt + i] != 0;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        pv[kt][r] = ok ? sacc[kt][r] * scale : -__builtin_inff();
        cmax[r] = __builtin_fmaxf(cmax[r], pv[kt][r]);
      }
    }
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float mn = __builtin_fmaxf(m_run[r], row16_max(cmax[r]));
      alpha[r] = (mn == -__builtin_inff()) ? 1.0f : __expf(m_run[r] - mn);
      float rs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        const float p = (pv[kt][r] == -__builtin_inff()) ? 0.0f : __expf(pv[kt][r] - mn);
        pv[kt][r] = p;
        rs += p;
      }
      l_run[r] = l_run[r] * alpha[r] + row16_sum(rs);
      m_run[r] = mn;
    }
    // rescale O only when some head's running maximum moved (later chunks rarely move it)
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f || alpha[2] != 1.0f || alpha[3] != 1.0f)) {
#pragma unroll
      for (int d = 0; d < 32; d++) {
#pragma unroll
        for (int r = 0; r < 4; r++) o[d][r] *= alpha[r];
      }
    }
    _Float16* pw = sh.p + w * 16 * kPStride;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int r = 0; r < 4; r++) pw[(4 * g + r) * kPStride + 16 * kt + i] = (_Float16)pv[kt][r];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's P stores are in LDS
    __builtin_amdgcn_wave_barrier();
    // ---- O += P V.  A = P [head i][keys 32ks + 8g ..].  B = V[keys][dim 16dt + i]: two
    // transposing LDS reads give this lane 8 consecutive keys of its dim from the row-major tile
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const f16x8 pa = *reinterpret_cast<const f16x8*>(pw + i * kPStride + 32 * ks + 8 * g);
      const int kb = 32 * ks + 8 * g + (i >> 2);
      // groups of 8 dim tiles: 16 transposing reads, then the group's 8 MFMAs
#pragma unroll
      for (int dt0 = 0; dt0 < 32; dt0 += 8) {
        s16x4 lo[8], hi[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const _Float16* p0 = sh.k + kb * kKStride + 16 * (dt0 + u) + 4 * (i & 3);
          lo[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0));
          hi[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p0 + 4 * kKStride));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const f16x8 vb = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo[u], hi[u], 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[dt0 + u], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: lane holds O[head 16w + 4g + r][dim 16dt + i].  The rows go out through
  // the (now idle) key tile in LDS: each wave writes its 16 heads x 256 dims in fp32, then
  // reads back whole rows as float4, so every global store instruction covers 1 KB.
  const bool single = n_splits == 1;
  const int64_t slot = (int64_t)t * n_splits + split;
  float scale_r[4];
#pragma unroll
  for (int r = 0; r < 4; r++) scale_r[r] = single ? (l_run[r] > 0.0f ? 1.0f / l_run[r] : 0.0f) : 1.0f;
  if (i == 0) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = 16 * w + 4 * g + r;
      if (single) {
        if (lse != nullptr)
          lse[(int64_t)t * kHeads + h] = l_run[r] > 0.0f ? m_run[r] + __logf(l_run[r]) : -__builtin_inff();
      } else {
        ws_ml[(slot * kHeads + h) * 2 + 0] = m_run[r];
        ws_ml[(slot * kHeads + h) * 2 + 1] = l_run[r];
      }
    }
  }
  constexpr int kOStride = 256 + 4;  // floats per staged row (padding spreads the banks)
  float* stage_o = reinterpret_cast<float*>(sh.k) + w * 16 * kOStride;  // 16.3 KB per wave
  float* orow0 = single ? out + ((int64_t)t * kHeads + 16 * w) * kD : ws_o + (slot * kHeads + 16 * w) * kD;
  __syncthreads();  // every wave is done reading the key tile
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int dt = 0; dt < 16; dt++) {
#pragma unroll
      for (int r = 0; r < 4; r++) stage_o[(4 * g + r) * kOStride + 16 * dt + i] = o[16 * half + dt][r] * scale_r[r];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows are in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int row = 0; row < 16; row++) {
      const float4 v = *reinterpret_cast<const float4*>(stage_o + row * kOStride + 4 * lane);
      *reinterpret_cast<float4*>(orow0 + (int64_t)row * kD + 256 * half + 4 * lane) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next half overwrites the rows
    __builtin_amdgcn_wave_barrier();
  }
}

// Combine the split partials of one (query, head): out = sum_s o_s e^(m_s - M) / L.  Every
// split's (m, l) and o slice load at once (splits <= kMaxSplits), then one pass combines.
constexpr int kMaxSplits = (kMaxTopK + kMaxSwa + kChunk - 1) / kChunk;

__global__ __launch_bounds__(128) void sparse_attn_merge_kernel(const float* __restrict__ ws_o,
                                                                const float* __restrict__ ws_ml,
                                                                int32_t n_splits, float* __restrict__ out,
                                                                float* __restrict__ lse) {
  const int t = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
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
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    if (s < n_splits && l[s] > 0.0f) {
      const float e = __expf(m[s] - M);
      L += l[s] * e;
      acc.x += v[s].x * e;
      acc.y += v[s].y * e;
      acc.z += v[s].z * e;
      acc.w += v[s].w * e;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  reinterpret_cast<float4*>(out + ((int64_t)t * kHeads + h) * kD)[tid] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse != nullptr && tid == 0) lse[(int64_t)t * kHeads + h] = L > 0.0f ? M + __logf(L) : -__builtin_inff();
}

struct Plan {
  int32_t n_chunks, chunks_per_split, n_splits;
};

Plan make_plan(int32_t n_q, int32_t K) {
  Plan p;
  p.n_chunks = (K + kMaxSwa + kChunk - 1) / kChunk;
  int32_t want = (512 + n_q - 1) / (n_q > 0 ? n_q : 1);
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
  if (n_q > 65535) return CSA2_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_bf16) | reinterpret_cast<uintptr_t>(kv_cache) |
       reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(swa) & (kFp8Win ? 7 : 15)) return CSA2_ERR_INVALID_ARG;
  const Plan p = make_plan(n_q, K);
  const size_t need = csa2_sparse_attn_workspace(n_q, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  float* ws_o = (float*)workspace;
  float* ws_ml = need > 0 ? ws_o + (size_t)n_q * p.n_splits * kHeads * kD : nullptr;
  hipLaunchKernelGGL(sparse_attn_kernel<kFp8Win>, dim3(p.n_splits, n_q), dim3(kThreads), 0,
                     (hipStream_t)stream, q_bf16, kv_cache, q_base, topk, K, swa, swa_ring, swa_start,
                     swa_len, scale, p.n_chunks, p.chunks_per_split, p.n_splits, out, lse, ws_o,
                     ws_ml);
  int st = check_launch();
  if (st != CSA2_OK || p.n_splits <= 1) return st;
  hipLaunchKernelGGL(sparse_attn_merge_kernel, dim3(kHeads, n_q), dim3(128), 0, (hipStream_t)stream,
                     ws_o, ws_ml, p.n_splits, out, lse);
  return check_launch();
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_sparse_attn(const uint16_t* q_bf16, const uint8_t* kv_cache,
                                const int64_t* q_base, const int32_t* topk, int32_t K,
                                const uint16_t* swa_bf16, const int64_t* swa_start,
                                const int32_t* swa_len, float scale, float* out, float* lse,
                                int32_t n_q, void* workspace, size_t ws_bytes, void* stream) {
  return csa2::launch_sparse_attn<false>(q_bf16, kv_cache, q_base, topk, K, swa_bf16, 0, swa_start,
                                         swa_len, scale, out, lse, n_q, workspace, ws_bytes, stream);
}

extern "C" int csa2_sparse_attn_swa_fp8(const uint16_t* q_bf16, const uint8_t* kv_cache,
                                        const int64_t* q_base, const int32_t* topk, int32_t K,
                                        const uint8_t* swa8, int64_t swa_ring,
                                        const int64_t* swa_start, const int32_t* swa_len, float scale,
                                        float* out, float* lse, int32_t n_q, void* workspace,
                                        size_t ws_bytes, void* stream) {
  return csa2::launch_sparse_attn<true>(q_bf16, kv_cache, q_base, topk, K, swa8, swa_ring, swa_start,
                                        swa_len, scale, out, lse, n_q, workspace, ws_bytes, stream);
}
