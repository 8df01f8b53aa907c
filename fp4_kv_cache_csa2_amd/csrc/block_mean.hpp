// block_mean.hpp -- one HISA block-mean record built by 16 lanes (gfx950).
//
// [ZB] "把 KV Cache 压缩推到极致" §2.3.4 (the HISA paragraphs): every block of 8 consecutive
// entries keeps the mean of its indexer keys for the coarse search.  The record is the fp32
// sum of the block's exact dequantised keys in ascending position order, divided once (IEEE)
// by the entry count, packed in the indexer-K format (MXFP4: E2M1 codes, one E8M0 scale per
// 32 channels).  Lane 4g + sub of the 16 builds channels 32g + 8sub .. 32g + 8sub + 7: its
// payload word (bytes 4sub .. 4sub + 3 of plane g) and its group's scale code.
#pragma once
#include "csa2_device.hpp"

namespace csa2 {

// cache: the indexer-K cache (tile layout); first: the block's first entry; cnt: its entries
// (1 .. 8); last: NULL, or a 68-byte record (64 payload bytes in channel order, then the 4
// scale bytes) of the block's last entry that the caller has just packed and that is read
// from there instead of the cache.  The lanes 4g .. 4g + 3 of one group must run together
// (the scale is their common maximum).
__device__ __forceinline__ uint32_t block_mean_word(const uint8_t* cache, int64_t first, int cnt, const uint8_t* last,
                                                   int g, int sub, uint32_t& code) {
#pragma clang fp contract(off)  // the same IEEE operations, in the same order, as the definition
  float sum[8];
  for (int e = 0; e < cnt; e++) {  // ascending positions: the fp32 running sum
    const bool rec = last != nullptr && e == cnt - 1;
    const uint32_t w = rec ? *reinterpret_cast<const uint32_t*>(last + 16 * g + 4 * sub)
                           : *reinterpret_cast<const uint32_t*>(cache + idx_plane_off(first + e, g) + 4 * sub);
    const uint32_t sc = rec ? last[64 + g] : cache[idx_scale_off(first + e) + g];
    const float X = __builtin_ldexpf(1.0f, (int)sc - 127);
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const uint32_t c = (w >> (4 * q)) & 15u;
      const float m = e2m1_mag(c & 7u) * X;  // exact: at most 3 significant bits times 2^k
      const float v = (c & 8u) ? -m : m;
      sum[q] = e == 0 ? v : sum[q] + v;
    }
  }
  float mean[8];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; q++) {
    mean[q] = sum[q] / (float)cnt;  // IEEE division (exact for a full block of 8)
    amax = __builtin_fmaxf(amax, __builtin_fabsf(mean[q]));
  }
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
  code = e8m0_scale_code(amax);
  const float X = __builtin_ldexpf(1.0f, (int)code - 127);
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < 8; q++) word |= e2m1_encode(mean[q], X) << (4 * q);
  return word;
}

}  // namespace csa2
