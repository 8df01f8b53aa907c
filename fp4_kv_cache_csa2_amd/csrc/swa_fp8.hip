// swa_fp8.hip -- packs sliding-window rows into FP8 window rows for gfx950.
//
// The window KV keeps FP8 precision ([ZB] "把 KV Cache 压缩推到极致" §2.4.4); its row takes
// DeepSeek-V4's FP8 KV entry ([ZB] §3.1 and [DF] "CSA2 与每 token 890 字节" §4.6: 448 FP8
// NoPE channels, 64 BF16 RoPE channels and 8 scale bytes = 584 B).  Scale per 64 NoPE
// channels: the OCP MX rule with E4M3's largest exponent, X = 2^(floor(log2 amax) - 8),
// stored as E8M0; elements are nearest-even E4M3 codes of x / X, saturating at 448.
//
// One wave packs one row: lane l reads channels 8l .. 8l+7 (one 16-byte load), lanes
// 0..55 form the seven scale groups of 8 lanes, lanes 56..63 carry the RoPE tail.  Rows
// land at caller-chosen slots, so a decode step appends its new tokens into ring buffers.
#include "csa2_device.hpp"

namespace csa2 {
namespace {

constexpr int kRowsPerBlock = 4;

// E8M0 code of the MX scale for E4M3 elements: floor(log2 amax) - 8 + 127, clamped to
// [0, 254]; 0 for a zero (or subnormal) group, 254 for a group holding an infinity.
__device__ __forceinline__ uint32_t e8m0_scale_code_e4m3(float amax) {
  const int eb = (int)((__float_as_uint(amax) >> 23) & 255);
  if (eb == 255) return 254;
  const int code = eb - 8;
  return (uint32_t)(eb == 0 || code < 0 ? 0 : code);
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void swa_pack_fp8_kernel(
    const uint16_t* __restrict__ rows, int64_t n, const int64_t* __restrict__ dst_rows,
    uint8_t* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= n) return;  // uniform per wave
  const int64_t dst = dst_rows != nullptr ? dst_rows[r] : r;
  if (dst < 0) return;
  const int lane = threadIdx.x & 63;
  const uint4 u = reinterpret_cast<const uint4*>(rows + r * kD)[lane];
  uint8_t* o = out + dst * kSwa8Bytes;  // 8-byte aligned: 584 = 8 x 73
  const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    v[2 * e] = bf16_bits_to_f32(wd[e] & 0xFFFFu);
    v[2 * e + 1] = bf16_bits_to_f32(wd[e] >> 16);
  }
  // group maximum over 8 lanes (NaN never wins a comparison, as in a max over values)
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float a = __builtin_fabsf(v[e]);
    amax = a > amax ? a : amax;
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const float b = __shfl_xor(amax, d);
    amax = b > amax ? b : amax;
  }
  const uint32_t code = e8m0_scale_code_e4m3(amax);
  const int shift = 127 - (int)code;  // x / X = x * 2^(127 - code), exact
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    uint32_t c = e4m3_encode(__builtin_ldexpf(__builtin_fabsf(v[e]), shift));
    if (v[e] < 0.0f && c != 0) c |= 0x80u;
    if (e < 4) lo |= c << (8 * e);
    else hi |= c << (8 * (e - 4));
  }
  // the seven scale codes come from lanes 0, 8, .., 48
  uint32_t sc[7];
#pragma unroll
  for (int g = 0; g < 7; g++) sc[g] = (uint32_t)__shfl((int)code, 8 * g);
  if (lane < 56) {
    *reinterpret_cast<uint2*>(o + 8 * lane) = make_uint2(lo, hi);
  } else {
    uint2* rp = reinterpret_cast<uint2*>(o + kDNope + 16 * (lane - 56));
    rp[0] = make_uint2(u.x, u.y);
    rp[1] = make_uint2(u.z, u.w);
  }
  if (lane == 0)
    *reinterpret_cast<uint2*>(o + kDNope + 2 * kDRope) =
        make_uint2(sc[0] | sc[1] << 8 | sc[2] << 16 | sc[3] << 24, sc[4] | sc[5] << 8 | sc[6] << 16);
}

}  // namespace
}  // namespace csa2

extern "C" int csa2_swa_pack_fp8(const uint16_t* rows_bf16, int64_t n, const int64_t* dst_rows,
                                 uint8_t* out, void* stream) {
  using namespace csa2;
  if (n < 0) return CSA2_ERR_INVALID_ARG;
  if (n == 0) return CSA2_OK;
  if (!rows_bf16 || !out) return CSA2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(rows_bf16) & 15) return CSA2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(out) & 7) return CSA2_ERR_INVALID_ARG;
  const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFFLL) return CSA2_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(swa_pack_fp8_kernel, dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0,
                     (hipStream_t)stream, rows_bf16, n, dst_rows, out);
  return check_launch();
}
