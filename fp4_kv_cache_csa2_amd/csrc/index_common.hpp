// index_common.hpp -- constants and per-tile helpers shared by the indexer kernels: the
// FP4 -> bf16 MFMA fragment conversion, the E8M0 scale, the block-of-8 maximum and the
// half-wave sum.
#pragma once
#include "csa2_device.hpp"

namespace csa2 {
namespace idx {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;

__device__ __forceinline__ bf16x8 cvt_fp4x8(uint32_t word, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float e8m0_scale(uint32_t code) {
  return __builtin_ldexpf(1.0f, (int)code - 127);
}

// 68-byte records (the MXFP4 query, the record an append has just packed) leave their
// 16-byte pieces only 4-byte aligned; gfx950 serves dword-aligned dwordx4 loads
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// 32 E2M1 codes (16 bytes) in the order the payload stores them: an FP4 MFMA operand
typedef int32_t fp4x32 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// The scoring kernels give lane (n, g) of a wave, for entry (or head) n, the MX groups g and
// 2 + g: channels 32g .. 32g + 31 and 64 + 32g .. 64 + 32g + 31, which are planes g and 2 + g
// of an indexer-K tile.  Both operands of a contraction use the same channel split, so the
// dot products are those of the natural channel order.

// One 32-entry tile of q . k on the block-scaled FP4 MFMA (32 heads x 32 entries x 64 dims
// per instruction).  Lane (n, g) holds, for both operands, its two 32-code MX groups (g in
// the first instruction, 2 + g in the second) and the scale word shifted right by 8g, so
// that byte 0 is group g's E8M0 code and byte 2 group 2 + g's.  Operand A is the query, B the
// entries.  The dot products are the MX definition: E2M1 values times 2^(code - 127), exact
// products, fp32 sums.
__device__ __forceinline__ f32x16 mfma_fp4_tile(const fp4x32 (&qa)[2], uint32_t qsc, const u32x4_a4& lo,
                                                const u32x4_a4& hi, uint32_t ksc, f32x16 acc) {
  const i32x8 a0 = {qa[0][0], qa[0][1], qa[0][2], qa[0][3], 0, 0, 0, 0};
  const i32x8 a1 = {qa[1][0], qa[1][1], qa[1][2], qa[1][3], 0, 0, 0, 0};
  const i32x8 b0 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
  const i32x8 b1 = {(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3], 0, 0, 0, 0};
  // format 4 = E2M1 for both operands; scale byte 0 (group g), then byte 2 (group 2 + g)
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc, 4, 4, 0, (int)qsc, 0, (int)ksc);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc, 4, 4, 2, (int)qsc, 2, (int)ksc);
  return acc;
}

// the MXFP4 query record of one head (68 B: 64 code bytes in channel order, 4 E8M0 bytes):
// lane group g takes code bytes 16g .. 16g + 15 and 32 + 16g .. 32 + 16g + 15 (groups g and
// 2 + g) and the scale word shifted right by 8g
__device__ __forceinline__ void load_fp4_query(const uint8_t* rec, int g, fp4x32 (&qa)[2], uint32_t& qsc) {
  const u32x4_a4 lo = *reinterpret_cast<const u32x4_a4*>(rec + 16 * g);
  const u32x4_a4 hi = *reinterpret_cast<const u32x4_a4*>(rec + 32 + 16 * g);
  qa[0] = fp4x32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
  qa[1] = fp4x32{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  qsc = *reinterpret_cast<const uint32_t*>(rec + 64) >> (8 * g);
}

// MXFP4 packing of 8 channels of a 32-channel group held by 4 consecutive lanes (the OCP
// MXFP4 rules of the indexer-K packer): raw holds the 8 bf16 values; returns their 8 E2M1
// codes (channel 8i + q in bits 4q .. 4q + 3) and sets code to the group's E8M0 scale.  The
// group's amax comes from two shuffles inside the 4 lanes, which must all run it together.
__device__ __forceinline__ uint32_t mxfp4_pack8(const uint4 raw, uint32_t& code) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
  code = e8m0_scale_code(amax);
  const float X = __builtin_ldexpf(1.0f, (int)code - 127);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) word |= e2m1_encode(x[i], X) << (4 * i);
  return word;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their no-wait maxima).
// Vector memory operations complete in issue order, so this waits for all but the n youngest.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// lane (n, g)'s share of one indexer-K entry: planes g (lo) and 2 + g (hi) and the entry's
// whole scale word
struct RawTile {
  u32x4_a4 lo, hi;
  uint32_t sc;
  bool valid;
};

// buffer cache-policy bits of the loads: 0, or kLoadStream (non-temporal) for bytes that one
// wave reads once (the decode scan's stream; each tile line is touched by one load)
constexpr int kLoadStream = 2;

// Loads lane (n, g)'s share of entry r of a tile-layout buffer resource (r counts entries from
// the buffer's first tile); r < 0 reads past the buffer's end, which returns zeros.
template <int kAux>
__device__ __forceinline__ void load_entry_share(__amdgpu_buffer_rsrc_t rs, int32_t r, int g, RawTile& t) {
  constexpr int32_t kPastEnd = 1 << 30;
  const int32_t off = r >= 0 ? idx_plane_off32(r, g) : kPastEnd;
  const int32_t soff = r >= 0 ? idx_scale_off32(r) : kPastEnd;
  t.lo = __builtin_bit_cast(u32x4_a4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kAux));
  t.hi = __builtin_bit_cast(u32x4_a4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 2 * kIdxPlaneBytes, 0, kAux));
  t.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, kAux);
}

// lane (n, g)'s share of a 68-byte record (64 payload bytes in channel order, then the scale
// word), e.g. one an append has just packed into LDS
__device__ __forceinline__ void load_record_share(const uint8_t* rec, int g, RawTile& t) {
  t.lo = *reinterpret_cast<const u32x4_a4*>(rec + 16 * g);
  t.hi = *reinterpret_cast<const u32x4_a4*>(rec + 32 + 16 * g);
  t.sc = *reinterpret_cast<const uint32_t*>(rec + 64);
}

// A buffer resource over the tiles that hold entries first .. first + n - 1 of a tile-layout
// cache (n >= 0), and the index, counted from the resource's first tile, of entry `first`.
// Loads of entries past the last of those tiles return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t idx_rsrc(const uint8_t* cache, int64_t first, int32_t n,
                                                          int32_t& first_rel) {
  first_rel = (int32_t)(first & 31);
  const int32_t tiles = n > 0 ? (first_rel + n + 31) >> 5 : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(cache + (first >> 5) * kIdxTileBytes), (short)0,
                                           tiles * kIdxTileBytes, 0x00020000);
}

// max(a, b) as one v_med3_f32 (the median of a, b and FLT_MAX): a NaN operand is ignored
// like fmaxf does, without the quieting instructions fmaxf costs on these operands; +inf
// saturates to FLT_MAX (only infinite inputs make one)
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, __FLT_MAX__); }

// ReLU as one v_med3_f32: clamp(x, 0, FLT_MAX); a NaN gives 0, like a comparison x > 0
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, __FLT_MAX__); }

// max over the 8 lanes of each aligned group of 8 (DPP within rows)
__device__ __forceinline__ float max8_lanes(float v) {
  v = max2(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = max2(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = max2(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// the score of a lane, or -inf for a slot with no visible entry.  Written as an addition so
// that every lane needs the sum: a select lets the compiler move the whole tile computation
// (the wave-wide MFMAs and the cross-lane head sum) under the valid lanes' exec mask, which
// it does for the block-scaled FP4 MFMA.  sum is finite for a valid slot (sum + 0 = sum,
// -0 becoming +0) and 0 for an empty one (loads past the end return zeros).
__device__ __forceinline__ float masked_score(float sum, bool valid) {
  return sum + (valid ? 0.0f : -__builtin_inff());
}

// v(lane) + v(lane ^ 32)
__device__ __forceinline__ float sum_halves(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}

}  // namespace idx

// longest score row (entries) of csa2_index_score: byte offsets into a sequence's tiles
// (2176 B per 32 entries) stay below 2^30, where the kernels' past-the-end offset lies
constexpr int32_t kMaxIndexWidth = 1 << 23;

// batches of at least this many Full-mode queries take the many-query kernel
constexpr int kMqMinQueries = 64;
int launch_index_score_mq_fp4q(const uint8_t* q_fp4, const float* head_w, const uint8_t* idx_cache,
                               const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width,
                               float* scores, float* block_max, void* stream);
int launch_index_score_mq(const uint16_t* q_idx_bf16, const float* head_w, const uint8_t* idx_cache,
                          const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                          float* block_max, void* stream);
}  // namespace csa2
