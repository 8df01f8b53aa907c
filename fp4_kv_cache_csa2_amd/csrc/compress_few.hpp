// compress_few.hpp -- the compressor for a few entries (the appends of a decode step) as
// workgroup-level device functions, shared by the append kernel of compress_pack.hip and the
// fused append + indexer-scoring kernel of append_index.hip (gfx950).
//
// The same formulas and bit-exactness rules as compress_pack.hip ([DF] "CSA2 与每 token 890
// 字节" §4.2 and §4.4, [ZB] "把 KV Cache 压缩推到极致" §2.3.1 and §2.4.4): every fp32 step
// is one IEEE round-to-nearest operation in a fixed order (contraction off, correctly
// rounded divisions, the projection an explicit ascending fma chain), so every kernel that
// packs an entry with these pieces writes the same bytes.
//
// compress_few_entry: one workgroup per entry and 32 consecutive indexer outputs, so it
// copies only its 32 rows of W_idx (one direct-to-LDS 1 KB row per instruction, issued
// first) while it pools, rotates and packs its entry; lane o < 32 then runs output o's
// 512-step chain from LDS and lanes 0 .. 3 pack the 32 outputs (one MXFP4 group).
// compress_entry_wg: one workgroup per entry and all 128 outputs, each chain reading its
// W_idx row from global memory; it keeps the packed indexer row in LDS for its caller.
// compress_entry_lds: the same for a workgroup that holds its CU alone, with every W_idx row
// copied into LDS at the start.
#pragma once
#include "csa2_device.hpp"

namespace csa2 {

constexpr int kFewOut = 32;       // indexer outputs per workgroup of compress_few_entry: one MXFP4 group
constexpr int kFewWRow = kD + 8;  // bf16 per W_idx row in LDS (1040 B: rows start 4 banks apart)

// Lane l < 64 of the first wave: channels 8l .. 8l + 7 of the entry pooled from its m latent
// rows (a_i = w_i / (w_0 + w_1), c = a_0 x_0 + a_1 x_1, each product and sum rounded; m = 1:
// the latent itself), the rope tail (channels 448 .. 511) rotated by the entry's angles.
__device__ __forceinline__ void pool_rope8(const uint16_t* __restrict__ lat, int m, const float* __restrict__ pool_w,
                                           const float* __restrict__ cs, int lane, float (&c)[8]) {
#pragma clang fp contract(off)
  const int ch0 = 8 * lane;
  if (m == 1) {
    const uint4 u = *reinterpret_cast<const uint4*>(lat + ch0);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      c[2 * q] = bf16_bits_to_f32(w4[q] & 0xFFFFu);
      c[2 * q + 1] = bf16_bits_to_f32(w4[q] >> 16);
    }
  } else {
    const uint4 u0 = *reinterpret_cast<const uint4*>(lat + ch0);
    const uint4 u1 = *reinterpret_cast<const uint4*>(lat + kD + ch0);
    typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));  // pool_w is 4-byte aligned
    const f32x4_a4 wa0 = *reinterpret_cast<const f32x4_a4*>(pool_w + ch0);
    const f32x4_a4 wa1 = *reinterpret_cast<const f32x4_a4*>(pool_w + ch0 + 4);
    const f32x4_a4 wb0 = *reinterpret_cast<const f32x4_a4*>(pool_w + kD + ch0);
    const f32x4_a4 wb1 = *reinterpret_cast<const f32x4_a4*>(pool_w + kD + ch0 + 4);
    const float w0[8] = {wa0.x, wa0.y, wa0.z, wa0.w, wa1.x, wa1.y, wa1.z, wa1.w};
    const float w1[8] = {wb0.x, wb0.y, wb0.z, wb0.w, wb1.x, wb1.y, wb1.z, wb1.w};
    const uint32_t xa[4] = {u0.x, u0.y, u0.z, u0.w}, xb[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const float ws = w0[q] + w1[q];
      const float a0 = w0[q] / ws, a1 = w1[q] / ws;
      const uint32_t ba = (q & 1) ? (xa[q >> 1] >> 16) : (xa[q >> 1] & 0xFFFFu);
      const uint32_t bb = (q & 1) ? (xb[q >> 1] >> 16) : (xb[q >> 1] & 0xFFFFu);
      const float p0 = a0 * bf16_bits_to_f32(ba);
      const float p1 = a1 * bf16_bits_to_f32(bb);
      c[q] = p0 + p1;
    }
  }
  if (ch0 >= kDNope) {  // rope tail: pairs (448+2i, 449+2i)
    const int i0 = (ch0 - kDNope) / 2;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float x0 = c[2 * q], x1 = c[2 * q + 1];
      const float co = cs[i0 + q], si = cs[kDRope / 2 + i0 + q];
      const float t0 = x0 * co, t1 = x1 * si, t2 = x0 * si, t3 = x1 * co;
      c[2 * q] = t0 - t1;
      c[2 * q + 1] = t2 + t3;
    }
  }
}

// The whole first wave: the main-KV bytes of channels 8l .. 8l + 7 (E2M1 codes, one E4M3
// scale per 16 channels shared by a lane pair) into row dst (NULL: nothing is written).
__device__ __forceinline__ void pack_kv8(const float (&c)[8], int lane, uint8_t* __restrict__ dst) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; q++) amax = __builtin_fmaxf(amax, __builtin_fabsf(c[q]));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));  // the 2 lanes of a 16-channel group
  const uint32_t sb = e4m3_encode(amax / 6.0f);
  const float S = e4m3_value(sb);
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < 8; q++) word |= e2m1_encode(c[q], S) << (4 * q);
  if (dst != nullptr) {
    *reinterpret_cast<uint32_t*>(dst + 4 * lane) = word;
    if ((lane & 1) == 0) dst[256 + (lane >> 1)] = (uint8_t)sb;
  }
}

// Four lanes 4g + sub of one wave pack MXFP4 group g: k8 holds the group's outputs
// 8 sub .. 8 sub + 7; returns their E2M1 codes (output 8 sub + i in nibble i) and sets
// the group's E8M0 scale code.
__device__ __forceinline__ uint32_t pack_idx8(const float* k8, uint32_t& code) {
#pragma clang fp contract(off)
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; q++) {
    v[q] = k8[q];
    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[q]));
  }
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
  code = e8m0_scale_code(amax);
  const float X = __builtin_ldexpf(1.0f, (int)code - 127);
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < 8; q++) word |= e2m1_encode(v[q], X) << (4 * q);
  return word;
}

// The indexer projection of one output: sum over the 512 channels of w[ch] * c[ch] as one
// fma chain in ascending channel order from +0; step v takes channels 8v .. 8v + 7 (the
// bf16 bits of w in wv).
__device__ __forceinline__ float chain8(float a, const uint4 wv, const float* __restrict__ c8) {
  const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
  const float4 c0 = *reinterpret_cast<const float4*>(c8);
  const float4 c1 = *reinterpret_cast<const float4*>(c8 + 4);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[0] & 0xFFFFu), c0.x, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[0] >> 16), c0.y, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[1] & 0xFFFFu), c0.z, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[1] >> 16), c0.w, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[2] & 0xFFFFu), c1.x, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[2] >> 16), c1.y, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[3] & 0xFFFFu), c1.z, a);
  a = __builtin_fmaf(bf16_bits_to_f32(w4[3] >> 16), c1.w, a);
  return a;
}

struct FewShared {
  __attribute__((aligned(16))) uint16_t w[kFewOut * kFewWRow];
  __attribute__((aligned(16))) float c[kD];
  float k[kFewOut];
};

// Packs outputs o0 .. o0 + 31 of one entry (and, when o0 == 0, its main-KV row) into cache
// row `row` (a negative row writes nothing).  lat: the entry's m latent rows (bf16
// [m, 512]); cs: its 64 RoPE values (32 cosines, then 32 sines).  Every thread of the
// workgroup calls it (it holds barriers); the first wave does the work.
__device__ __forceinline__ void compress_few_entry(const uint16_t* __restrict__ lat, int m,
                                                   const float* __restrict__ pool_w, const float* __restrict__ cs,
                                                   const uint16_t* __restrict__ w_idx, int o0, int64_t row,
                                                   uint8_t* __restrict__ kv_out, uint8_t* __restrict__ idx_out,
                                                   FewShared& sh) {
  const int lane = threadIdx.x;
  if (lane < 64) {  // the first wave (wave-uniform)
    for (int r = 0; r < kFewOut; r++)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(w_idx + (int64_t)(o0 + r) * kD + 8 * lane),
          (void __attribute__((address_space(3)))*)&sh.w[r * kFewWRow], 16, 0, 0);
    float c[8];
    pool_rope8(lat, m, pool_w, cs, lane, c);
    *reinterpret_cast<float4*>(&sh.c[8 * lane]) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(&sh.c[8 * lane + 4]) = make_float4(c[4], c[5], c[6], c[7]);
    if (o0 == 0) pack_kv8(c, lane, row >= 0 ? kv_out + row * kKvBytes : nullptr);  // one workgroup per entry
  }
  __builtin_amdgcn_s_waitcnt(0);  // the W_idx rows have landed in LDS
  __syncthreads();
  if (lane < kFewOut) {  // output o0 + lane
    float a = 0.0f;
    const uint16_t* wr = &sh.w[lane * kFewWRow];
#pragma unroll 8
    for (int v = 0; v < kD / 8; v++) a = chain8(a, *reinterpret_cast<const uint4*>(wr + 8 * v), &sh.c[8 * v]);
    sh.k[lane] = a;
  }
  __syncthreads();
  if (lane < 4) {  // the MXFP4 group of these 32 outputs: 4 lanes, 8 outputs each
    uint32_t code;
    const uint32_t word = pack_idx8(&sh.k[8 * lane], code);
    if (row >= 0) idx_store_word(idx_out, row, o0 / 32, lane, word, code);  // group o0 / 32 of the row
  }
}

struct EntryShared {
  __attribute__((aligned(16))) float c[kD];
  float k[kIdxDim];
  __attribute__((aligned(16))) uint8_t idx_row[kIdxBytes + 12];  // the packed indexer row (68 B)
};

// Packs one whole entry (main-KV row and indexer row) into cache row `row` (negative: the
// caches are not written) and leaves the packed indexer row in sh.idx_row.  Every thread of
// the workgroup (at least 128 threads) calls it: the first wave pools, rotates and packs the
// main KV, threads o < 128 run output o's chain with its W_idx row read from global memory,
// and lanes 0 .. 15 pack the 4 MXFP4 groups.
__device__ __forceinline__ void compress_entry_wg(const uint16_t* __restrict__ lat, int m,
                                                  const float* __restrict__ pool_w, const float* __restrict__ cs,
                                                  const uint16_t* __restrict__ w_idx, int64_t row,
                                                  uint8_t* __restrict__ kv_out, uint8_t* __restrict__ idx_out,
                                                  EntryShared& sh) {
  const int tid = threadIdx.x;
  if (tid < 64) {  // the first wave (wave-uniform)
    float c[8];
    pool_rope8(lat, m, pool_w, cs, tid, c);
    *reinterpret_cast<float4*>(&sh.c[8 * tid]) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(&sh.c[8 * tid + 4]) = make_float4(c[4], c[5], c[6], c[7]);
    pack_kv8(c, tid, row >= 0 ? kv_out + row * kKvBytes : nullptr);
  }
  __syncthreads();
  if (tid < kIdxDim) {  // output tid: its W_idx row streams in 16 steps of 4 pieces, two steps ahead
    const uint4* wr = reinterpret_cast<const uint4*>(w_idx + (int64_t)tid * kD);
    constexpr int kStep = 4, kAhead = 2, kSteps = kD / 8 / kStep;
    uint4 buf[kAhead + 1][kStep];
#pragma unroll
    for (int s = 0; s < kAhead; s++)
#pragma unroll
      for (int i = 0; i < kStep; i++) buf[s][i] = wr[kStep * s + i];
    float a = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; s++) {
      if (s + kAhead < kSteps) {
#pragma unroll
        for (int i = 0; i < kStep; i++) buf[(s + kAhead) % (kAhead + 1)][i] = wr[kStep * (s + kAhead) + i];
      }
#pragma unroll
      for (int i = 0; i < kStep; i++) a = chain8(a, buf[s % (kAhead + 1)][i], &sh.c[8 * (kStep * s + i)]);
    }
    sh.k[tid] = a;
  }
  __syncthreads();
  if (tid < 16) {  // group g = tid / 4: outputs 32g + 8 sub .. + 7
    const int g = tid >> 2, sub = tid & 3;
    uint32_t code;
    const uint32_t word = pack_idx8(&sh.k[32 * g + 8 * sub], code);
    *reinterpret_cast<uint32_t*>(&sh.idx_row[16 * g + 4 * sub]) = word;
    if (sub == 0) sh.idx_row[64 + g] = (uint8_t)code;
    if (row >= 0) idx_store_word(idx_out, row, g, sub, word, code);
  }
  __syncthreads();
}

// A workgroup barrier that waits only for this wave's LDS accesses (s_waitcnt lgkmcnt(0)),
// not for its outstanding global loads and stores as __syncthreads' release fence does; the
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// W_idx in LDS, one 1 KB row per output, rows 1040 bytes apart so that the 64 chains of a wave
// (one row each) read different banks
constexpr int kWRowBytes = 2 * kD + 16;
struct WRows {
  __attribute__((aligned(16))) uint8_t r[kIdxDim * kWRowBytes];
};

// compress_entry_wg for a workgroup of kWavesWg >= 4 waves that holds its CU alone (its LDS
// takes most of the CU), so that the 128 KB of W_idx have the CU's memory path to themselves:
// waves 3 .. kWavesWg - 1 copy the rows into wl (one direct-to-LDS instruction per 1 KB row,
// every one issued at the start), the first wave pools, rotates and packs the main KV while
// they land, and waves 1 and 2 run output o = tid - 64's chain from LDS (the same chain8
// order as compress_entry_wg, so the bytes are the same).  Every wave calls it and passes
// three barriers; it returns with the packed indexer row in sh.idx_row.  The cache stores are
// not waited for.
template <int kWavesWg>
__device__ __forceinline__ void compress_entry_lds(const uint16_t* __restrict__ lat, int m,
                                                   const float* __restrict__ pool_w, const float* __restrict__ cs,
                                                   const uint16_t* __restrict__ w_idx, int64_t row,
                                                   uint8_t* __restrict__ kv_out, uint8_t* __restrict__ idx_out,
                                                   EntryShared& sh, WRows& wl) {
  static_assert(kWavesWg >= 4, "a pooling wave, two chain waves and at least one copying wave");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave >= 3) {  // copy rows wave - 3, wave - 3 + (kWavesWg - 3), ...
    for (int r = wave - 3; r < kIdxDim; r += kWavesWg - 3)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(w_idx + (int64_t)r * kD + 8 * lane),
          (void __attribute__((address_space(3)))*)&wl.r[r * kWRowBytes], 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed
    lds_barrier();                  // 1: the pooled entry and every row are in LDS
    lds_barrier();                  // 2
    lds_barrier();                  // 3
  } else if (wave == 0) {
    float c[8];
    pool_rope8(lat, m, pool_w, cs, tid, c);
    *reinterpret_cast<float4*>(&sh.c[8 * tid]) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(&sh.c[8 * tid + 4]) = make_float4(c[4], c[5], c[6], c[7]);
    lds_barrier();  // 1
    pack_kv8(c, tid, row >= 0 ? kv_out + row * kKvBytes : nullptr);
    lds_barrier();  // 2: every output is in sh.k
    if (tid < 16) {  // group g = tid / 4: outputs 32g + 8 sub .. + 7
      const int g = tid >> 2, sub = tid & 3;
      uint32_t code;
      const uint32_t word = pack_idx8(&sh.k[32 * g + 8 * sub], code);
      *reinterpret_cast<uint32_t*>(&sh.idx_row[16 * g + 4 * sub]) = word;
      if (sub == 0) sh.idx_row[64 + g] = (uint8_t)code;
      if (row >= 0) idx_store_word(idx_out, row, g, sub, word, code);
    }
    lds_barrier();  // 3: sh.idx_row is complete
  } else {  // waves 1 and 2: output o's chain
    const int o = tid - 64;
    lds_barrier();  // 1
    const uint8_t* wr = &wl.r[o * kWRowBytes];
    float a = 0.0f;
#pragma unroll 8
    for (int v = 0; v < kD / 8; v++) a = chain8(a, *reinterpret_cast<const uint4*>(wr + 16 * v), &sh.c[8 * v]);
    sh.k[o] = a;
    lds_barrier();  // 2
    lds_barrier();  // 3
  }
}

}  // namespace csa2
