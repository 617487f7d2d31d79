// MXFP4 quantisation of the indexer's query and key vectors.
//
// Pages: the indexer's query-key path runs in MXFP4 ("DeepSeek V4技术揭秘",
// §一 基础设施; FP4 on the indexer path, sz-guanghua.com.cn ifanr repost,
// 百萬長上下文); this is the step that produces those operands from real
// values.  The conversion follows OCP Microscaling v1.0 (restated): per
// 32-element block the shared exponent is X = floor(log2(amax)) - 2 (2 is
// E2M1's largest exponent), clamped to [-127, 127], an all-zero block taking
// -127 (this library's reading); each element x / 2^X goes to the nearest E2M1
// magnitude {0, 0.5, 1, 1.5, 2, 3, 4, 6}, a tie to the magnitude with an even
// code, past 6 saturated; the sign bit of x is kept.  Element 2i is the low
// nibble of byte i, as the indexer reads it.
//
// Every step is exact in fp32 (the maximum, the exponent of a float, scaling
// by a power of two, comparisons with the midpoints of the E2M1 grid), so the
// codes are those of the definition applied to the input values, bit for bit.
// An HBM stream: one thread per 32-element block, 64 B (bf16) or 128 B (fp32)
// read and 17 B written.
#include "common.hpp"

namespace {

constexpr int kQThreads = 256;

// E2M1 magnitude code of v >= 0 (v already divided by the block scale): the
// count of grid midpoints below v, each midpoint going to the even code of
// its two neighbours (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0,
// 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0); past 5 everything is 6 (saturated).
CSA_DEV uint32_t e2m1_magnitude_code(float v) {
  return uint32_t(v > 0.25f) + uint32_t(v >= 0.75f) + uint32_t(v > 1.25f) + uint32_t(v >= 1.75f) +
         uint32_t(v > 2.5f) + uint32_t(v >= 3.5f) + uint32_t(v > 5.0f);
}

template <int kInF32>
__global__ __launch_bounds__(kQThreads) void mxfp4_quantize_kernel(const void* __restrict__ x, long n_blocks,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ e8m0) {
  const long blk = long(blockIdx.x) * kQThreads + threadIdx.x;
  if (blk >= n_blocks) return;
  float v[32];
  if constexpr (kInF32) {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(x) + blk * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const v4f w = __builtin_nontemporal_load(p + q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = w[e];
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + blk * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = __builtin_nontemporal_load(p + q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
        v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // X = floor(log2(amax)) - 2; for fp32 inputs floor(log2(amax)) <= 127, so
  // X <= 125 and 2^-X is a normal float; a zero block takes X = -127
  const int X = amax > 0.f ? max(ilogbf(amax) - 2, -127) : -127;
  const float inv = __uint_as_float(uint32_t(127 - X) << 23);   // 2^-X, exact
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t sign = (__float_as_uint(v[i]) >> 31) << 3;
    const uint32_t c = sign | e2m1_magnitude_code(fabsf(v[i]) * inv);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  *reinterpret_cast<uint4*>(codes + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  e8m0[blk] = uint8_t(X + 127);
}

}  // namespace

extern "C" csa_status_t csa_mxfp4_quantize(const void* x, int32_t in_dtype, int64_t n_vec, int32_t d,
                                           uint8_t* codes, uint8_t* e8m0, void* stream) {
  if (!x || !codes || !e8m0) return CSA_EINVAL;
  if (in_dtype != CSA_BF16 && in_dtype != CSA_F32) return CSA_EINVAL;
  if (n_vec < 0 || d <= 0 || d % 32 != 0) return CSA_EINVAL;
  const long n_blocks = long(n_vec) * (d / 32);
  if (n_blocks == 0) return CSA_OK;
  const long grid = (n_blocks + kQThreads - 1) / kQThreads;
  if (grid > 0x7FFFFFFFL) return CSA_ENOTSUP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == CSA_F32)
    hipLaunchKernelGGL(mxfp4_quantize_kernel<1>, dim3(unsigned(grid)), dim3(kQThreads), 0, st, x, n_blocks, codes,
                       e8m0);
  else
    hipLaunchKernelGGL(mxfp4_quantize_kernel<0>, dim3(unsigned(grid)), dim3(kQThreads), 0, st, x, n_blocks, codes,
                       e8m0);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}
