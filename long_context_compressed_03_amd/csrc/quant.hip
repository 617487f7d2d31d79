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
// An HBM stream: 64 B (bf16) or 128 B (fp32) read and 17 B written per
// 32-element block.
#include "mxfp4.hpp"

namespace {

constexpr int kQThreads = 256;

// kL lanes per 32-element block (4 for bf16, 8 for fp32), each holding 16
// contiguous input bytes, so a wave's load is one contiguous 1 KB span; a
// thread takes kIter such lanes, kQThreads apart, with all their loads issued
// first.  The block's maximum goes through kL lanes with xor shuffles, and
// lane p writes the codes of its elements (bytes [p*kE/2, (p+1)*kE/2) of the
// block's 16).
constexpr int kIter = 4;

// One lane's 16 input bytes (kE elements of a 32-element block whose kL
// lanes are adjacent and aligned): the block's shared exponent X (through
// xor shuffles over the kL lanes) and the lane's kE E2M1 codes, element i in
// bits [4i, 4i + 4).
template <int kInF32>
CSA_DEV uint32_t convert_lane(const u32x4& w, int& X) {
  constexpr int kL = kInF32 ? 8 : 4;
  constexpr int kE = 32 / kL;
  float v[kE];
  if constexpr (kInF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kE; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < kL; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  X = mxfp4_block_exponent(amax);
  const float inv = mxfp4_inv_scale(X);
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const uint32_t sign = (__float_as_uint(v[i]) >> 31) << 3;
    word |= (sign | e2m1_magnitude_code(fabsf(v[i]) * inv)) << (4 * i);
  }
  return word;
}

template <int kInF32>
__global__ __launch_bounds__(kQThreads) void mxfp4_quantize_kernel(const void* __restrict__ x, long n_blocks,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ e8m0) {
  constexpr int kL = kInF32 ? 8 : 4;       // lanes per block
  constexpr int kE = 32 / kL;              // elements per lane
  const long n_lanes = n_blocks * kL;
  const long gl0 = long(blockIdx.x) * (kQThreads * kIter) + threadIdx.x;
  u32x4 w[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const long gl = min(gl0 + long(it) * kQThreads, n_lanes - 1);   // lanes past the end re-read the last one
    w[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) + gl * 16));
  }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const long gl = gl0 + long(it) * kQThreads;
    const long blk = gl / kL;
    const int part = int(gl % kL);
    int X;
    const uint32_t word = convert_lane<kInF32>(w[it], X);
    if (blk < n_blocks) {                  // whole groups of kL lanes alike
      uint8_t* out = codes + blk * 16 + part * (kE / 2);
      // streaming stores: the operands are read later, by another kernel
      if constexpr (kE == 8) __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(out));
      else __builtin_nontemporal_store(uint16_t(word), reinterpret_cast<uint16_t*>(out));
      if (part == 0) __builtin_nontemporal_store(uint8_t(X + 127), e8m0 + blk);
    }
  }
}

// The cache append's indexer keys: for each sequence whose token at pos[b]
// completes a block (the rule of csa_kv_cache_append), vector
// b * cap + (pos[b] + 1) / m - 1 of x is converted as above; lane mapping as
// above, a vector's d / 32 blocks in consecutive lanes.
template <int kInF32>
__global__ __launch_bounds__(64) void mxfp4_quantize_appended_kernel(const void* __restrict__ x,
                                                                     const int32_t* __restrict__ pos, int B, int cap,
                                                                     int m, int d, uint8_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ e8m0) {
  constexpr int kL = kInF32 ? 8 : 4;
  constexpr int kE = 32 / kL;
  const int per_vec = (d / 32) * kL;       // lanes per vector
  const long gl = long(blockIdx.x) * 64 + threadIdx.x;
  const int b = int(min(gl / per_vec, long(B) - 1));
  const int p = pos[b];
  const bool done = gl < long(B) * per_vec && p >= 0 && (p + 1) % m == 0 && (p + 1) / m - 1 < cap;
  const long vec = long(b) * cap + (done ? (p + 1) / m - 1 : 0);
  const int lane_in_vec = int(gl - long(b) * per_vec);
  const int lv = done ? lane_in_vec : 0;
  const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) + (vec * per_vec + lv) * 16);
  int X;
  const uint32_t word = convert_lane<kInF32>(w, X);   // every lane joins the shuffles
  if (!done) return;
  const long blk = vec * (d / 32) + lv / kL;
  const int part = lv % kL;
  uint8_t* out = codes + blk * 16 + part * (kE / 2);
  if constexpr (kE == 8) *reinterpret_cast<uint32_t*>(out) = word;
  else *reinterpret_cast<uint16_t*>(out) = uint16_t(word);
  if (part == 0) e8m0[blk] = uint8_t(X + 127);
}

}  // namespace

extern "C" csa_status_t csa_mxfp4_quantize(const void* x, int32_t in_dtype, int64_t n_vec, int32_t d,
                                           uint8_t* codes, uint8_t* e8m0, void* stream) {
  if (!x || !codes || !e8m0) return CSA_EINVAL;
  if (in_dtype != CSA_BF16 && in_dtype != CSA_F32) return CSA_EINVAL;
  if (n_vec < 0 || d <= 0 || d % 32 != 0) return CSA_EINVAL;
  const long n_blocks = long(n_vec) * (d / 32);
  if (n_blocks == 0) return CSA_OK;
  const long lanes = n_blocks * (in_dtype == CSA_F32 ? 8 : 4);
  const long grid = (lanes + kQThreads * kIter - 1) / (kQThreads * kIter);
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

extern "C" csa_status_t csa_mxfp4_quantize_appended(const void* x, int32_t in_dtype, const int32_t* pos, int32_t B,
                                                    int32_t cap, int32_t m, int32_t d, uint8_t* codes,
                                                    uint8_t* e8m0, void* stream) {
  if (!x || !pos || !codes || !e8m0) return CSA_EINVAL;
  if (in_dtype != CSA_BF16 && in_dtype != CSA_F32) return CSA_EINVAL;
  if (B < 0 || cap < 0 || m < 1 || d <= 0 || d % 32 != 0) return CSA_EINVAL;
  if (B == 0 || cap == 0) return CSA_OK;
  const long lanes = long(B) * (d / 32) * (in_dtype == CSA_F32 ? 8 : 4);
  const long grid = (lanes + 63) / 64;
  if (grid > 0x7FFFFFFFL || long(B) * cap * (d / 32) > 0x7FFFFFFFFFFFL) return CSA_ENOTSUP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == CSA_F32)
    hipLaunchKernelGGL(mxfp4_quantize_appended_kernel<1>, dim3(unsigned(grid)), dim3(64), 0, st, x, pos, B, cap, m, d,
                       codes, e8m0);
  else
    hipLaunchKernelGGL(mxfp4_quantize_appended_kernel<0>, dim3(unsigned(grid)), dim3(64), 0, st, x, pos, B, cap, m, d,
                       codes, e8m0);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}
