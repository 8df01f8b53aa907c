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
int launch_index_score_mq(const uint16_t* q_idx_bf16, const float* head_w, const uint8_t* idx_cache,
                          const int64_t* q_base, const int32_t* q_nvis, int32_t n_q, int32_t width, float* scores,
                          float* block_max, void* stream);
}  // namespace csa2
