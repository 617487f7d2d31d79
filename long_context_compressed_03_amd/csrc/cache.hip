// Decode-time KV cache append: the raw sliding window as a mirrored ring, and
// the compressed cache's entry appended when a block of m tokens completes.
//
// Pages: the window of the newest uncompressed tokens is kept in bf16 beside
// the compressed entries, which may be stored in fp8 (ferris DeepSeek-V4
// analysis, 工程层, heterogeneous KV cache); every m tokens' K/V become one
// entry (blog.nickys.cn, 三大架构改动 §1 CSA, §2 HCA).  The layout below is
// this library's.
//
// Ring: each sequence owns 2L rows.  Token p is written to rows p mod L and
// p mod L + L, so the newest min(L, p + 1) tokens always sit in one run of
// consecutive rows, and the attention calls read them as a plain raw buffer
// of 2L rows whose row 0 stands for position raw_pos0 = q0 - (q0 mod L),
// q0 = max(0, p - L + 1).  The m rows of a just-completed block start at row
// (p - m + 1) mod L, also one run.
//
// One launch: the compression kernels' append forms (compress.hip) write the
// new rows and pool the completed block in place, taking the block's newest
// row from the input, so the pooled entry is bit-identical to what
// csa_compress_kv gives for the same block.  For m <= L the m - 1 older rows
// they read are never the two rows being written.
#include "compress_core.hpp"
#include "mxfp4.hpp"

namespace {

using namespace csa_cmp;

// The indexer key append (m < 32, d = 128): 16-lane group g serves sequence
// 4 * blockIdx.x + g.  It writes the token's key row (both ring copies) and
// logit, pools the block the token completes exactly as compress_group_at
// pools its K side (the same operations in the same order, newest row from
// the input), and stores the pooled fp32 entry in MXFP4: lane c holds
// columns [8c, 8c + 8), so a 32-column block is 4 adjacent lanes.
struct IxAppendArgs {
  const void* k_new;
  const float* z_new;
  const int32_t* pos;
  int B, L, m, cap;
  void* k_ring;
  float* z_ring;
  uint8_t* codes;
  uint8_t* e8m0;
};

template <int kInF32>
CSA_DEV void indexer_key_append_at(const IxAppendArgs& x, int blk) {
  const void* __restrict__ k_new = x.k_new;
  const float* __restrict__ z_new = x.z_new;
  const int32_t* __restrict__ pos = x.pos;
  const int B = x.B, L = x.L, m = x.m, cap = x.cap;
  void* k_ring = x.k_ring;
  float* z_ring = x.z_ring;
  uint8_t* codes = x.codes;
  uint8_t* e8m0 = x.e8m0;
  const int lane_c = threadIdx.x & (kGroup - 1);
  const int b = blk * 4 + int(threadIdx.x / kGroup);
  if (b >= B) return;                      // whole 16-lane groups leave together
  const int p = pos[b];
  const AppendPlan pl = append_plan(p, L, m, cap);
  constexpr int kEl = kInF32 ? 4 : 2;
  constexpr int kLaneBytes = kColsPerLane * kEl;
  const size_t ring0 = size_t(b) * 2 * L;
  const uint8_t* kn = static_cast<const uint8_t*>(k_new) + size_t(b) * kHeadDim * kEl;
  if (p >= 0) {
    const int s = p % L;
#pragma unroll
    for (int h = 0; h < kLaneBytes / 16; ++h) {
      const uint4 xk = *reinterpret_cast<const uint4*>(kn + lane_c * kLaneBytes + h * 16);
#pragma unroll
      for (int copy = 0; copy < 2; ++copy)
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(k_ring) +
                                  (ring0 + s + size_t(copy) * L) * kHeadDim * kEl + lane_c * kLaneBytes + h * 16) = xk;
    }
    if (lane_c < 2) z_ring[ring0 + s + size_t(lane_c) * L] = z_new[b];
  }
  if (!pl.done) return;

  const size_t row0 = ring0 + pl.first_row;
  const float* z = z_ring + row0;
  auto zat = [&](int x) -> float { return *(x == m - 1 ? z_new + b : z + x); };
  auto krow = [&](int jj, float* out) {
    const bool nw = jj == m - 1;
    load_row8<kInF32>(nw ? static_cast<const void*>(kn) : k_ring, nw ? size_t(0) : row0 + jj, lane_c, out);
  };
  float zmax = 0.f, inv = 0.f;
  auto stats = [&]() {
    zmax = -INFINITY;
    for (int x = lane_c; x < m; x += kGroup) zmax = fmaxf(zmax, zat(x));
    zmax = group_max<kGroup>(zmax);
    float zsum = 0.f;
    for (int x = lane_c; x < m; x += kGroup) zsum += expf(zat(x) - zmax);
    zsum = group_sum<kGroup>(zsum);
    inv = 1.f / zsum;
  };
  float ak[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ak[i] = 0.f;
  constexpr int kU = 4;
  int j = 0;
  for (; j + kU <= m; j += kU) {
    float kr[kU][8], a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) krow(j + u, kr[u]);
    if (j == 0) stats();
#pragma unroll
    for (int u = 0; u < kU; ++u) a[u] = expf(zat(j + u) - zmax) * inv;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ak[i] = fmaf(a[u], kr[u][i], ak[i]);
    }
  }
  if (m < kU) stats();
  for (; j < m; ++j) {
    float kr[8];
    krow(j, kr);
    const float a = expf(zat(j) - zmax) * inv;
#pragma unroll
    for (int i = 0; i < 8; ++i) ak[i] = fmaf(a, kr[i], ak[i]);
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(ak[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int X = mxfp4_block_exponent(amax);
  const float sc = mxfp4_inv_scale(X);
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sign = (__float_as_uint(ak[i]) >> 31) << 3;
    word |= (sign | e2m1_magnitude_code(fabsf(ak[i]) * sc)) << (4 * i);
  }
  const size_t entry = size_t(b) * cap + pl.entry;
  *reinterpret_cast<uint32_t*>(codes + entry * (kHeadDim / 2) + lane_c * 4) = word;
  if ((lane_c & 3) == 0) e8m0[entry * (kHeadDim / 32) + (lane_c >> 2)] = uint8_t(X + 127);
}

template <int kInF32>
__global__ __launch_bounds__(64) void indexer_key_append_kernel(IxAppendArgs x) {
  indexer_key_append_at<kInF32>(x, int(blockIdx.x));
}

// Both appends of a CSA layer's decode token in one launch: blocks [0, nb)
// take the K/V append (cache_append_short_at), blocks [nb, 2 nb) the indexer
// key append, each on its own rings and caches (nothing one writes is read
// by the other), with the same code as the two separate calls.
template <int kInF32, int kOut>
__global__ __launch_bounds__(64) void decode_append_kernel(AppendArgs a, IxAppendArgs x, int nb) {
  if (int(blockIdx.x) < nb)
    cache_append_short_at<kInF32, kOut>(a, int(blockIdx.x));
  else
    indexer_key_append_at<kInF32>(x, int(blockIdx.x) - nb);
}

template <int kInF32>
hipError_t launch_decode_append(int ckv_dtype, const AppendArgs& a, const IxAppendArgs& x, hipStream_t st) {
  const int nb = (a.B + 3) / 4;
  const dim3 grid(unsigned(2 * nb));
  switch (ckv_dtype) {
    case CSA_BF16: hipLaunchKernelGGL((decode_append_kernel<kInF32, CSA_BF16>), grid, dim3(64), 0, st, a, x, nb); break;
    case CSA_F32: hipLaunchKernelGGL((decode_append_kernel<kInF32, CSA_F32>), grid, dim3(64), 0, st, a, x, nb); break;
    default: hipLaunchKernelGGL((decode_append_kernel<kInF32, CSA_FP8_E4M3>), grid, dim3(64), 0, st, a, x, nb);
  }
  return hipGetLastError();
}

}  // namespace

size_t csa_kv_append_workspace_size(int) { return 0; }

extern "C" csa_status_t csa_indexer_key_append(const void* k_new, const float* z_new, int32_t io_dtype,
                                               const int32_t* pos, int32_t B, int32_t d, int32_t L_ring,
                                               void* k_ring, float* z_ring, int32_t m, int32_t cap,
                                               uint8_t* codes, uint8_t* e8m0, void* stream) {
  if (!k_new || !z_new || !pos || !k_ring || !z_ring || !codes || !e8m0) return CSA_EINVAL;
  if (io_dtype != CSA_BF16 && io_dtype != CSA_F32) return CSA_EINVAL;
  if (d != kHeadDim || B < 0 || m < 1 || cap < 0 || L_ring < m) return CSA_EINVAL;
  if (m >= 32) return CSA_ENOTSUP;
  if (long(B) * 2 * L_ring > 0x7FFFFFFFL) return CSA_ENOTSUP;
  if (B == 0) return CSA_OK;
  const dim3 grid(unsigned((B + 3) / 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const IxAppendArgs x{k_new, z_new, pos, B, L_ring, m, cap, k_ring, z_ring, codes, e8m0};
  if (io_dtype == CSA_F32)
    hipLaunchKernelGGL(indexer_key_append_kernel<1>, grid, dim3(64), 0, st, x);
  else
    hipLaunchKernelGGL(indexer_key_append_kernel<0>, grid, dim3(64), 0, st, x);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}

extern "C" csa_status_t csa_kv_cache_append(const void* k_new, const void* v_new, const float* z_new, int32_t io_dtype,
                                            const int32_t* pos, int32_t B, int32_t d, int32_t L_ring, void* k_ring,
                                            void* v_ring, float* z_ring, int32_t m, int32_t cap, int32_t ckv_dtype,
                                            void* ck, void* cv, float* ck_scale, float* cv_scale, int32_t* raw_pos0,
                                            void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!k_new || !v_new || !z_new || !pos || !k_ring || !v_ring || !z_ring || !ck || !cv || !raw_pos0)
    return CSA_EINVAL;
  if (io_dtype != CSA_BF16 && io_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(ckv_dtype)) return CSA_EINVAL;
  if (ckv_dtype == CSA_FP8_E4M3 && (!ck_scale || !cv_scale)) return CSA_EINVAL;
  if (d != kHeadDim || B < 0 || m < 1 || cap < 0 || L_ring < m) return CSA_EINVAL;
  if (long(B) * 2 * L_ring > 0x7FFFFFFFL) return CSA_ENOTSUP;
  if (B == 0) return CSA_OK;
  const csa_cmp::AppendArgs a{k_new, v_new, z_new, pos, k_ring, v_ring, z_ring, raw_pos0, B, L_ring, m, cap,
                              ck, cv, ck_scale, cv_scale};
  const hipError_t e = csa_cmp::launch_cache_append(io_dtype, ckv_dtype, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA_OK : CSA_EHIP;
}

extern "C" csa_status_t csa_decode_append(const void* k_new, const void* v_new, const float* z_new,
                                          const void* ki_new, const float* zi_new, int32_t io_dtype,
                                          const int32_t* pos, int32_t B, int32_t d, int32_t m, int32_t cap,
                                          int32_t L_ring, void* k_ring, void* v_ring, float* z_ring,
                                          int32_t ckv_dtype, void* ck, void* cv, float* ck_scale, float* cv_scale,
                                          int32_t* raw_pos0, int32_t Li_ring, void* ki_ring, float* zi_ring,
                                          uint8_t* codes, uint8_t* e8m0, void* stream) {
  if (!k_new || !v_new || !z_new || !ki_new || !zi_new || !pos || !k_ring || !v_ring || !z_ring || !ck || !cv ||
      !raw_pos0 || !ki_ring || !zi_ring || !codes || !e8m0)
    return CSA_EINVAL;
  if (io_dtype != CSA_BF16 && io_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(ckv_dtype)) return CSA_EINVAL;
  if (ckv_dtype == CSA_FP8_E4M3 && (!ck_scale || !cv_scale)) return CSA_EINVAL;
  if (d != kHeadDim || B < 0 || m < 1 || cap < 0 || L_ring < m || Li_ring < m) return CSA_EINVAL;
  if (m >= 32) return CSA_ENOTSUP;
  if (long(B) * 2 * L_ring > 0x7FFFFFFFL || long(B) * 2 * Li_ring > 0x7FFFFFFFL) return CSA_ENOTSUP;
  if (B == 0) return CSA_OK;
  const csa_cmp::AppendArgs a{k_new, v_new, z_new, pos, k_ring, v_ring, z_ring, raw_pos0, B, L_ring, m, cap,
                              ck, cv, ck_scale, cv_scale};
  const IxAppendArgs x{ki_new, zi_new, pos, B, Li_ring, m, cap, ki_ring, zi_ring, codes, e8m0};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = io_dtype == CSA_F32 ? launch_decode_append<1>(ckv_dtype, a, x, st)
                                           : launch_decode_append<0>(ckv_dtype, a, x, st);
  return e == hipSuccess ? CSA_OK : CSA_EHIP;
}
