// csa2_device.hpp -- internal helpers shared by the gfx950 kernels of libcsa2.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/csa2.h"

namespace csa2 {

constexpr int kD = 512;       // latent width
constexpr int kDRope = 64;    // rope tail
constexpr int kDNope = kD - kDRope;
constexpr int kHeads = 64;    // attention heads
constexpr int kIdxHeads = 32; // indexer heads
constexpr int kIdxDim = 128;  // indexer head dim
constexpr int kKvBytes = 288;
constexpr int kIdxBytes = 68;
constexpr int kSwa8Bytes = 584;  // FP8 window row: 448 E4M3 codes, 64 bf16, 7 scale bytes, 1 pad
constexpr int kBlock = 8;     // candidate block size
constexpr int kMaxPool = 2048;
constexpr int kMaxTopK = 512;
constexpr int kMaxSwa = 128;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// The indexer-K cache in HBM: tiles of 32 entries, 2176 bytes each.  Entry j sits in tile
// j / 32 at slot e = j % 32.  Its payload bytes 16p .. 16p + 15 (plane p = 0 .. 3: the E2M1
// codes of channels 32p .. 32p + 31, one MX group) are at byte 512p + 16e of the tile and its
// four E8M0 scale bytes at byte 2048 + 4e.  Each plane of a tile is one contiguous 512-byte
// run, so a wave reads a whole tile with two fully coalesced 1 KB loads and one 128-byte
// load, and no cache line is fetched twice.
constexpr int kIdxTileEntries = 32;
constexpr int kIdxTileBytes = 2176;
constexpr int kIdxPlaneBytes = 512;
constexpr int kIdxScaleOff = 2048;

// byte offset of plane p of entry j, and of its scale word (j >= 0, within one buffer of
// fewer than 2^31 bytes for the 32-bit forms)
__host__ __device__ __forceinline__ constexpr int64_t idx_plane_off(int64_t j, int p) {
  return (j >> 5) * kIdxTileBytes + kIdxPlaneBytes * p + 16 * (j & 31);
}
__host__ __device__ __forceinline__ constexpr int64_t idx_scale_off(int64_t j) {
  return (j >> 5) * kIdxTileBytes + kIdxScaleOff + 4 * (j & 31);
}
__host__ __device__ __forceinline__ constexpr int32_t idx_plane_off32(int32_t j, int p) {
  return (j >> 5) * kIdxTileBytes + kIdxPlaneBytes * p + 16 * (j & 31);
}
__host__ __device__ __forceinline__ constexpr int32_t idx_scale_off32(int32_t j) {
  return (j >> 5) * kIdxTileBytes + kIdxScaleOff + 4 * (j & 31);
}

// one writer lane of an indexer-K record: the payload word of channels 32g + 8sub .. + 7
// (bytes 4sub .. 4sub + 3 of plane g) and, from lane sub = 0, group g's E8M0 code
__device__ __forceinline__ void idx_store_word(uint8_t* cache, int64_t j, int g, int sub, uint32_t word,
                                               uint32_t code) {
  *reinterpret_cast<uint32_t*>(cache + idx_plane_off(j, g) + 4 * sub) = word;
  if (sub == 0) cache[idx_scale_off(j) + g] = (uint8_t)code;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// E2M1 magnitude code -> value (exact), 3-bit code.
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  const uint32_t e = c >> 1, m = c & 1;
  return e == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
}

// OCP E4M3FN byte -> value (exact; 0x7F / 0xFF are never produced by the packer).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  float v = e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8 + m), (int)e - 10);
  return (b & 0x80) ? -v : v;
}

// Nearest-even E4M3 code of x >= 0, saturating at 448 (0x7E); NaN and +inf also give 0x7E.
// One rounding step (rint after an exact power-of-two scaling), so the code is exact.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  if (!(x < 448.0f)) return 0x7E;
  if (x < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9 (code 8 is 2^-6)
    return (uint32_t)__builtin_rintf(x * 512.0f);
  }
  const int E = (int)((__float_as_uint(x) >> 23) & 255) - 127;  // x is a normal fp32
  const float r = __builtin_rintf(__builtin_ldexpf(x, 3 - E));   // [8, 16], ties to even
  const uint32_t code = ((uint32_t)(E + 7) << 3) + ((uint32_t)r - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 code of e on the grid {0,.5,1,1.5,2,3,4,6} * S by exact midpoint comparisons,
// ties to the even code, saturating at 6; the sign bit only on a non-zero code.
// An infinite element saturates explicitly: at the largest scale (2^127, a group holding an
// infinity) the upper midpoints overflow to +inf, which every finite |e| (at most FLT_MAX <
// 2.5 * 2^127) correctly stays below.
__device__ __forceinline__ uint32_t e2m1_encode(float e, float S) {
  if (!(S > 0.0f)) return 0;
  const float a = __builtin_fabsf(e);
  uint32_t c;
  if (a == __builtin_inff()) {
    c = 7;
  } else {
    c = (a > 0.25f * S) + (a > 0.75f * S) + (a > 1.25f * S) + (a > 1.75f * S) + (a > 2.5f * S) +
        (a > 3.5f * S) + (a > 5.0f * S);
    c += (a == 0.75f * S) + (a == 1.75f * S) + (a == 3.5f * S);  // odd-side ties round up
  }
  return (e < 0.0f && c != 0) ? (c | 8u) : c;
}

// OCP MX shared-scale rule for E2M1 elements: floor(log2 amax) - 2 + 127, clamped; a
// group holding an infinity takes the largest finite scale, 254.
__device__ __forceinline__ uint32_t e8m0_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int eb = (int)((__float_as_uint(amax) >> 23) & 255);  // 0 for subnormal amax
  if (eb == 255) return 254;
  const int code = eb == 0 ? 0 : eb - 2;
  return (uint32_t)(code < 0 ? 0 : (code > 254 ? 254 : code));
}

// The selection's first pass counts the ranking keys (order_key) of a row's items in
// kSelBins bins of their top 12 bits; the decode scan can count its block maxima the same way
// (csa2_append_index_score_sel).
constexpr int kSelBins = 4096;
constexpr int kSelBinShift = 20;

// Order-preserving map fp32 -> uint32 (larger float -> larger key); NaN ranks as -inf.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) f = -__builtin_inff();
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

inline int check_launch() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Workgroups of `threads` threads of `kernel` that fit on the current device at once, for
// grids sized to one round of resident workgroups.  Computed on a device's first call and
// kept in `cache` (one slot per device, zero = not known yet).  The figure is the same
// whichever call computes it, and the slots are atomics, so concurrent first calls on any
// threads may both compute and store it without a data race.
constexpr int kMaxDevices = 64;
template <typename Kernel>
int resident_workgroups(Kernel kernel, int threads, std::atomic<int> (&cache)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
      per_cu = 2;
    v = cus * per_cu;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace csa2
