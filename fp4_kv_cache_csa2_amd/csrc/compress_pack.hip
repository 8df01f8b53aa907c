// compress_pack.hip -- compressor pooling, RoPE, main-KV FP4 pack, indexer-K projection
// and MXFP4 pack, one fused kernel for gfx950.
//
// Follows [DF] "CSA2 与每 token 890 字节" §4.2 (compressor equation) and §4.4 (entry
// formats); [ZB] "把 KV Cache 压缩推到极致" §2.3.1 (indexer K projected from the main-KV
// entry) and §2.4.4 (RoPE then quantise; E2M1 with one E4M3 scale per 16 channels).
//
// Bit-exactness: every fp32 step is a single IEEE round-to-nearest operation in a fixed
// order (contraction is off in this file, divisions are correctly rounded, the
// projection is an explicit ascending fma chain), and the quantisers decide codes by
// exact comparisons, so the packed bytes do not depend on instruction scheduling.
#include "compress_few.hpp"

#pragma clang fp contract(off)

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kWChunk = 64;  // channels of W_idx staged per step

// Bulk packing: kEnt entries per workgroup amortise the W_idx reads over many entries.
template <int kEnt>
__global__ __launch_bounds__(kThreads) void compress_pack_kernel(
    const uint16_t* __restrict__ latent, int64_t n_entries, int m, const float* __restrict__ pool_w,
    const float* __restrict__ rope_cs, const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_out,
    uint8_t* __restrict__ idx_out, const int64_t* __restrict__ dst_rows, int64_t w_stride) {
  __shared__ float s_c[kEnt][kD];          // rotated fp32 entries
  __shared__ float s_k[kEnt][kIdxDim];     // projected indexer keys
  __shared__ uint16_t s_w[2][kWChunk][kIdxDim + 8];  // W_idx^T chunks (bf16 bits)
  const int t = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * kEnt;
  // cache row that entry j is written to (a negative row drops the entry)
  auto out_row = [&](int64_t j) -> int64_t { return dst_rows != nullptr ? dst_rows[j] : j; };
  // ---- phase A: pooling, RoPE, main-KV pack
  // thread -> (entry e, channels 32p..32p+31)
  const int e = t >> 4, p = t & 15;
  const int64_t j = j0 + e;
  if (e < kEnt && j < n_entries) {
    float c[32];
    const int ch0 = 32 * p;
    if (m == 1) {
      const uint4* src = reinterpret_cast<const uint4*>(latent + j * kD + ch0);
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const uint4 u = src[v];
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          c[8 * v + 2 * q] = bf16_bits_to_f32(w4[q] & 0xFFFFu);
          c[8 * v + 2 * q + 1] = bf16_bits_to_f32(w4[q] >> 16);
        }
      }
    } else {
      // a_i = w_i / (w_0 + w_1); c = a_0 x_0 + a_1 x_1, each product and sum rounded; the
      // weights are the entry's own rows when they are per token (w_stride = 2 * 512)
      const float* pw = pool_w + j * w_stride;
      const uint4* s0 = reinterpret_cast<const uint4*>(latent + (2 * j) * kD + ch0);
      const uint4* s1 = reinterpret_cast<const uint4*>(latent + (2 * j + 1) * kD + ch0);
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const uint4 u0 = s0[v], u1 = s1[v];
        const uint32_t a4[4] = {u0.x, u0.y, u0.z, u0.w};
        const uint32_t b4[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const int ch = ch0 + 8 * v + q;
          const float w0 = pw[ch], w1 = pw[kD + ch];
          const float ws = w0 + w1;
          const float a0 = w0 / ws, a1 = w1 / ws;
          const uint32_t xa = (q & 1) ? (a4[q >> 1] >> 16) : (a4[q >> 1] & 0xFFFFu);
          const uint32_t xb = (q & 1) ? (b4[q >> 1] >> 16) : (b4[q >> 1] & 0xFFFFu);
          const float p0 = a0 * bf16_bits_to_f32(xa);
          const float p1 = a1 * bf16_bits_to_f32(xb);
          c[8 * v + q] = p0 + p1;
        }
      }
    }
    if (p >= kDNope / 32) {  // rope tail: pairs (448+2i, 449+2i)
      const float* cs = rope_cs + j * kDRope;
      const int i0 = (ch0 - kDNope) / 2;
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const float x0 = c[2 * q], x1 = c[2 * q + 1];
        const float co = cs[i0 + q], si = cs[kDRope / 2 + i0 + q];
        const float t0 = x0 * co, t1 = x1 * si, t2 = x0 * si, t3 = x1 * co;
        c[2 * q] = t0 - t1;
        c[2 * q + 1] = t2 + t3;
      }
    }
#pragma unroll
    for (int q = 0; q < 32; q++) s_c[e][ch0 + q] = c[q];

    // two groups of 16 channels: E4M3 scale + E2M1 codes
    uint32_t pay[4];
    uint32_t scl = 0;
#pragma unroll
    for (int g = 0; g < 2; g++) {
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; q++) amax = __builtin_fmaxf(amax, __builtin_fabsf(c[16 * g + q]));
      const uint32_t sb = e4m3_encode(amax / 6.0f);
      const float S = e4m3_value(sb);
      scl |= sb << (8 * g);
#pragma unroll
      for (int w = 0; w < 2; w++) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 8; q++) word |= e2m1_encode(c[16 * g + 8 * w + q], S) << (4 * q);
        pay[2 * g + w] = word;
      }
    }
    const int64_t row = out_row(j);
    if (row >= 0) {
      uint8_t* dst = kv_out + row * kKvBytes;
      *reinterpret_cast<uint4*>(dst + 16 * p) = make_uint4(pay[0], pay[1], pay[2], pay[3]);
      *reinterpret_cast<uint16_t*>(dst + 256 + 2 * p) = (uint16_t)scl;
    }
  }
    __syncthreads();

  // ---- phase B: indexer projection k[o] = sum_ch W[o][ch] c~[ch], ascending fma chain.
  // thread -> output o, entries h*kHalf .. h*kHalf + kHalf - 1.  W_idx streams through
  // LDS in transposed chunks of 64 channels ([ch][o], double-buffered) so every chain
  // step reads its weight from LDS without bank conflicts and no step waits on global
  // memory.
  constexpr int kHalf = kEnt / 2;
  const int o = t & (kIdxDim - 1), h = t >> 7;
  float acc[kHalf];
#pragma unroll
  for (int e = 0; e < kHalf; e++) acc[e] = 0.0f;
  uint4 stage[4];
  auto fetch = [&](int chunk) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int u = t + kThreads * q;  // 1024 pieces of 8 bf16: row u/8, part u%8
      stage[q] = *reinterpret_cast<const uint4*>(w_idx + (int64_t)(u >> 3) * kD + kWChunk * chunk + 8 * (u & 7));
    }
  };
  auto spill = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int u = t + kThreads * q, row = u >> 3, part = u & 7;
      const uint32_t w4[4] = {stage[q].x, stage[q].y, stage[q].z, stage[q].w};
#pragma unroll
      for (int v = 0; v < 4; v++) {
        s_w[buf][8 * part + 2 * v][row] = (uint16_t)(w4[v] & 0xFFFFu);
        s_w[buf][8 * part + 2 * v + 1][row] = (uint16_t)(w4[v] >> 16);
      }
    }
  };
  fetch(0);
  spill(0);
  __syncthreads();
  for (int chunk = 0; chunk < kD / kWChunk; chunk++) {
    const int buf = chunk & 1;
    if (chunk + 1 < kD / kWChunk) fetch(chunk + 1);
#pragma unroll 2
    for (int cb = 0; cb < kWChunk; cb += 4) {
      float wf[4];
#pragma unroll
      for (int q = 0; q < 4; q++) wf[q] = bf16_bits_to_f32(s_w[buf][cb + q][o]);
#pragma unroll
      for (int e = 0; e < kHalf; e++) {
        const float4 cv = *reinterpret_cast<const float4*>(&s_c[kHalf * h + e][kWChunk * chunk + cb]);
        float a = acc[e];
        a = __builtin_fmaf(wf[0], cv.x, a);
        a = __builtin_fmaf(wf[1], cv.y, a);
        a = __builtin_fmaf(wf[2], cv.z, a);
        a = __builtin_fmaf(wf[3], cv.w, a);
        acc[e] = a;
      }
    }
    if (chunk + 1 < kD / kWChunk) spill(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < kHalf; e++) s_k[kHalf * h + e][o] = acc[e];
    __syncthreads();

  // ---- phase C: MXFP4 pack.  4 threads per (entry, group of 32), 8 elements each
  if (t < kEnt * 16) {
    const int gi = t >> 2, sub = t & 3;
    const int e = gi >> 2, g = gi & 3;
    const int64_t j = j0 + e;
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; q++) {
      v[q] = s_k[e][32 * g + 8 * sub + q];
      amax = __builtin_fmaxf(amax, __builtin_fabsf(v[q]));
    }
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
    const uint32_t code = e8m0_scale_code(amax);
    const float X = __builtin_ldexpf(1.0f, (int)code - 127);
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 8; q++) word |= e2m1_encode(v[q], X) << (4 * q);
    const int64_t row = j < n_entries ? out_row(j) : -1;
    if (row >= 0) idx_store_word(idx_out, row, g, sub, word, code);
  }
}

// ---------------------------------------------------------------------------------------
// Few entries (the appends of a decode step): one workgroup of one wave per (entry, 32
// consecutive indexer outputs), the body in compress_few.hpp.
__global__ __launch_bounds__(64) void compress_few_kernel(
    const uint16_t* __restrict__ latent, int m, const float* __restrict__ pool_w, const float* __restrict__ rope_cs,
    const uint16_t* __restrict__ w_idx, uint8_t* __restrict__ kv_out, uint8_t* __restrict__ idx_out,
    const int64_t* __restrict__ dst_rows, int64_t w_stride) {
  __shared__ FewShared sh;
  const int64_t j = blockIdx.x;
  const int64_t row = dst_rows != nullptr ? dst_rows[j] : j;
  compress_few_entry(latent + j * m * kD, m, pool_w + j * w_stride, rope_cs + j * kDRope, w_idx, blockIdx.y * kFewOut, row, kv_out,
                     idx_out, sh);
}

}  // namespace
}  // namespace csa2

namespace {
int launch_compress(const uint16_t* latent_bf16, int64_t n_entries, int m, const float* pool_w,
                    int per_token_w, const float* rope_cs, const uint16_t* w_idx_bf16, uint8_t* kv_out, uint8_t* idx_out,
                    const int64_t* dst_rows, void* stream) {
  using namespace csa2;
  if (n_entries < 0 || (per_token_w != 0 && per_token_w != 1)) return CSA2_ERR_INVALID_ARG;
  if (m != 1 && m != 2) return CSA2_ERR_UNSUPPORTED;
  if (n_entries == 0) return CSA2_OK;
  if (!latent_bf16 || !rope_cs || !w_idx_bf16 || !kv_out || !idx_out) return CSA2_ERR_INVALID_ARG;
  if (m == 2 && !pool_w) return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(latent_bf16) | reinterpret_cast<uintptr_t>(w_idx_bf16) |
       reinterpret_cast<uintptr_t>(kv_out) | reinterpret_cast<uintptr_t>(idx_out)) & 15)
    return CSA2_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(rope_cs) | reinterpret_cast<uintptr_t>(pool_w)) & 3 ||
      reinterpret_cast<uintptr_t>(dst_rows) & 7)
    return CSA2_ERR_INVALID_ARG;
  // floats from one entry's weight rows to the next: 0 for the static [m, 512] weights
  const int64_t w_stride = (per_token_w && m > 1) ? (int64_t)m * kD : 0;
  if (n_entries <= 64) {
    hipLaunchKernelGGL(compress_few_kernel, dim3((unsigned)n_entries, kIdxDim / kFewOut), dim3(64), 0,
                       (hipStream_t)stream, latent_bf16, m, pool_w, rope_cs, w_idx_bf16, kv_out, idx_out, dst_rows,
                       w_stride);
  } else {
    const int64_t grid = (n_entries + 15) / 16;
    if (grid > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(compress_pack_kernel<16>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, latent_bf16, n_entries, m, pool_w, rope_cs, w_idx_bf16,
                       kv_out, idx_out, dst_rows, w_stride);
  }
  return check_launch();
}
}  // namespace

extern "C" int csa2_compress_pack(const uint16_t* latent_bf16, int64_t n_entries, int m,
                                  const float* pool_w, int per_token_w, const float* rope_cs,
                                  const uint16_t* w_idx_bf16, uint8_t* kv_out, uint8_t* idx_out,
                                  void* stream) {
  return launch_compress(latent_bf16, n_entries, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_out, idx_out, nullptr,
                         stream);
}

extern "C" int csa2_compress_append(const uint16_t* latent_bf16, int64_t n_entries, int m,
                                    const float* pool_w, int per_token_w, const float* rope_cs,
                                    const uint16_t* w_idx_bf16, const int64_t* dst_rows,
                                    uint8_t* kv_cache, uint8_t* idx_cache, void* stream) {
  if (!dst_rows && n_entries > 0) return CSA2_ERR_INVALID_ARG;
  return launch_compress(latent_bf16, n_entries, m, pool_w, per_token_w, rope_cs, w_idx_bf16, kv_cache, idx_cache,
                         dst_rows, stream);
}
