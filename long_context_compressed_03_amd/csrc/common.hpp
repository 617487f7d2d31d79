// Shared device helpers for the gfx950 (CDNA4) kernels of libcsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

#include "../../include/csa.h"

#define CSA_DEV __device__ __forceinline__
#define CSA_DEV_HOST_INLINE __host__ __device__ __forceinline__

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

// ----------------------------------------------------------------- bf16 --
CSA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to the nearest bf16, ties to even, packed low/high:
// one V_CVT_PK_BF16_F32 (checked on gfx950 to round exactly like the
// integer recipe below on normal, subnormal and tie inputs).
CSA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{lo, hi}, v2bf_t));
}

// Two fp32 values split as hi + lo, both bf16 pairs: hi is the nearest bf16 of
// each value and lo the nearest bf16 of the (exact, fp32) remainder, so hi + lo
// carries 16 significant bits.  A product with a bf16 operand taken as
// hi * x + lo * x (two matrix-core passes) then loses about 2^-17 of each value
// instead of the 2^-9 of a single bf16 rounding.
CSA_DEV void split_bf16x2(float a, float b, uint32_t* hi, uint32_t* lo) {
  const uint32_t h = pack_bf16x2(a, b);
  *hi = h;
  *lo = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xFFFF0000u));
}

// Round fp32 to the nearest bf16, ties to even (finite inputs).
CSA_DEV uint16_t f32_to_bf16(float x) { return uint16_t(pack_bf16x2(x, 0.f)); }

// --------------------------------------------------------- fp8 E4M3FN --
// Decode an OCP E4M3FN code (not NaN) to fp32.  Every E4M3 value is also an
// exact bf16 value (3 mantissa bits, exponents -9 .. 8).
CSA_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t mnt = c & 7u;
  float mag;
  if (e == 0) {
    mag = float(mnt) * 0.001953125f;  // mnt * 2^-9
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (mnt << 20));  // 2^(e-7) * (1 + mnt/8)
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

// Round fp32 to E4M3FN, nearest-even, saturating at +-448.
CSA_DEV uint32_t f32_to_e4m3(float x) {
  uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {               // below 2^-6: subnormal grid 2^-9
    code = uint32_t(__builtin_rintf(a * 512.f));  // 0..8; 8 == smallest normal code
  } else {
    int e = int((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
    float sc = a * __uint_as_float(uint32_t(127 + 3 - e) << 23);  // a * 2^(3-e) in [8, 16)
    uint32_t r = uint32_t(__builtin_rintf(sc));                   // 8 .. 16
    if (r == 16u) { r = 8u; e += 1; }
    code = (uint32_t(e + 7) << 3) | (r - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | s;
}

// ------------------------------------------------------ wave reductions --
// v combined over the lane pairs (l, l ^ 16) (kX == 16) or (l, l ^ 32)
// (kX == 32) as op(value of the lower lane, value of the upper lane), the same
// on both lanes, through the CDNA4 row-swap permutes (no LDS round trip).
template <int kX, typename Op>
CSA_DEV float swap_combine(float v, Op op) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (kX == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}
// max / sum over the four lanes l % 16 + {0, 16, 32, 48} (one MFMA C column)
CSA_DEV float column_max(float v) {
  auto mx = [](float x, float y) { return fmaxf(x, y); };
  return swap_combine<32>(swap_combine<16>(v, mx), mx);
}
CSA_DEV float column_sum(float v) {
  auto add = [](float x, float y) { return x + y; };
  return swap_combine<32>(swap_combine<16>(v, add), add);
}
// v of the lane n places along its 16-lane row (DPP row rotation).
template <int kN>
CSA_DEV float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + kN, 0xF, 0xF, false));
}
// max / sum over all 64 lanes: the column combine, then rotations by 8, 4, 2, 1
// within each row; every lane forms the same pairwise tree, so all lanes hold
// bit-identical results.
CSA_DEV float wave_max_all(float v) {
  v = column_max(v);
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
CSA_DEV float wave_sum_all(float v) {
  v = column_sum(v);
  v = v + row_ror<8>(v);
  v = v + row_ror<4>(v);
  v = v + row_ror<2>(v);
  return v + row_ror<1>(v);
}

CSA_DEV float wave_max_xor(float v, int lane_mask) { return fmaxf(v, __shfl_xor(v, lane_mask)); }

template <int kLanes>
CSA_DEV float group_max(float v) {
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
template <int kLanes>
CSA_DEV float group_sum(float v) {
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// v of the lane n places lower in its 16-lane row, 0 for the row's first n
// lanes (DPP row shift).
template <int kN>
CSA_DEV uint32_t row_shr(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x110 + kN, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each 16-lane row, then the totals of the rows below (read from
// lanes 15, 31, 47) are added.  ALU only, no LDS round trip.
CSA_DEV uint32_t wave_inclusive_scan(uint32_t v) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 15));
  const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 31));
  const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 47));
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Block-wide exclusive prefix sum of one uint32 per thread (blockDim.x a
// multiple of 64, at most 1024).  `smem` needs blockDim.x/64 + 1 words.
// Returns the exclusive prefix; *total receives the block sum.  tail_sync:
// end with a barrier so that `smem` may be written again right away (a last
// use of `smem` in the kernel can skip it).
CSA_DEV uint32_t block_exclusive_scan(uint32_t v, uint32_t* smem, uint32_t* total, bool tail_sync = true) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) smem[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const uint32_t x = lane < nw ? smem[lane] : 0u;
    const uint32_t xi = wave_inclusive_scan(x);
    if (lane < nw) smem[lane] = xi - x;  // exclusive wave offsets
    if (lane == nw - 1) smem[16] = xi;
  }
  __syncthreads();
  uint32_t r = smem[wid] + incl - v;
  *total = smem[16];
  if (tail_sync) __syncthreads();
  return r;
}

// Block-wide AND / OR of one uint32 per thread (blockDim.x a multiple of 64,
// at most 1024); `smem` needs 16 words.
CSA_DEV uint32_t block_reduce_and(uint32_t v, uint32_t* smem) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v &= __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) smem[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0xFFFFFFFFu;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) r &= smem[w];
  __syncthreads();
  return r;
}
CSA_DEV uint32_t block_reduce_or(uint32_t v, uint32_t* smem) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) smem[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0u;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) r |= smem[w];
  __syncthreads();
  return r;
}

// --------------------------------------------------------------- status --
// Packed items of several sequences (the varlen calls): sequence b owns items
// cu[b] .. cu[b + 1] - 1 (cu[0] = 0, non-decreasing).  Sequence of item r
// (r < cu[B]), by binary search over the B + 1 offsets.
CSA_DEV int csa_packed_seq(const int32_t* __restrict__ cu, int B, int r) {
  int lo = 0, hi = B;   // cu[lo] <= r < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

#define CSA_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return CSA_EHIP;    \
  } while (0)

// Dynamic LDS above 64 KB needs a per-kernel opt-in.  It is set once per
// (kernel, device) and the record of what was set is guarded by a mutex, so
// host threads may launch concurrently.
inline hipError_t csa_lds_opt_in(const void* fn, size_t bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

static inline bool csa_dtype_ok(int32_t dt) { return dt == CSA_BF16 || dt == CSA_F32 || dt == CSA_FP8_E4M3; }
