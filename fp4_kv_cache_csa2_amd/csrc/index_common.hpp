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

// indexer rows are 68 bytes, so a row's 16-byte pieces are only 4-byte aligned; gfx950
// serves dword-aligned global dwordx4 loads
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// 32 E2M1 codes (16 bytes) in the order the payload stores them: an FP4 MFMA operand
typedef int32_t fp4x32 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// One 32-entry tile of q . k on the block-scaled FP4 MFMA (32 heads x 32 entries x 64 dims
// per instruction).  Lane (n, g) holds, for both operands, the 64 codes of dims
// 64g .. 64g + 63 of its head / entry as two 32-code MX blocks (blocks 2g and 2g + 1, each
// block one instruction) and the row's scale word shifted so that byte 0 is block 2g's E8M0
// code and byte 1 block 2g + 1's.  Operand A is the query, B the entries.  The dot products
// are the MX definition: E2M1 values times 2^(code - 127), exact products, fp32 sums.
__device__ __forceinline__ f32x16 mfma_fp4_tile(const fp4x32 (&qa)[2], uint32_t qsc, const u32x4_a4& lo,
                                                const u32x4_a4& hi, uint32_t ksc, f32x16 acc) {
  const i32x8 a0 = {qa[0][0], qa[0][1], qa[0][2], qa[0][3], 0, 0, 0, 0};
  const i32x8 a1 = {qa[1][0], qa[1][1], qa[1][2], qa[1][3], 0, 0, 0, 0};
  const i32x8 b0 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
  const i32x8 b1 = {(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3], 0, 0, 0, 0};
  // format 4 = E2M1 for both operands; scale byte 0 (block 2g), then byte 1 (block 2g + 1)
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc, 4, 4, 0, (int)qsc, 0, (int)ksc);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc, 4, 4, 1, (int)qsc, 1, (int)ksc);
  return acc;
}

// the MXFP4 query record of one head (68 B: 64 code bytes, 4 E8M0 bytes): lane group g
// takes code bytes 32g .. 32g + 31 and the scale bytes of blocks 2g, 2g + 1
__device__ __forceinline__ void load_fp4_query(const uint8_t* rec, int g, fp4x32 (&qa)[2], uint32_t& qsc) {
  const u32x4_a4 lo = *reinterpret_cast<const u32x4_a4*>(rec + 32 * g);
  const u32x4_a4 hi = *reinterpret_cast<const u32x4_a4*>(rec + 32 * g + 16);
  qa[0] = fp4x32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
  qa[1] = fp4x32{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  qsc = *reinterpret_cast<const uint32_t*>(rec + 64) >> (16 * g);
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

struct RawTile {
  u32x4_a4 lo, hi;
  uint32_t sc;
  bool valid;
};

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

// longest score row (entries) of csa2_index_score: byte offsets into a sequence's cache
// (68 B per entry) stay below 2^31
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
