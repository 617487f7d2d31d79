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
// (p - m + 1) mod L, also one run, and the compression kernels pool them in
// place (a second launch, after the writes).
//
// One 64-thread block per sequence copies the two rows of K and of V (4 row
// copies, 16 B per thread per step) and the logit, then writes the plan the
// compression launch reads and the window base.
#include "compress_core.hpp"

namespace {

__global__ __launch_bounds__(64) void ring_append_kernel(const uint8_t* __restrict__ k_new,
                                                        const uint8_t* __restrict__ v_new,
                                                        const float* __restrict__ z_new,
                                                        const int32_t* __restrict__ pos, int B, int row_bytes, int L,
                                                        uint8_t* k_ring, uint8_t* v_ring, float* z_ring, int m,
                                                        int cap, int32_t* plan, int32_t* raw_pos0) {
  const int b = blockIdx.x;
  const int p = pos[b];
  const int chunks = row_bytes / 16;       // 16-B pieces per row
  if (p >= 0) {
    const int s = p % L;
    for (int c = threadIdx.x; c < 4 * chunks; c += 64) {
      const int q = c % chunks;
      const int copy = (c / chunks) & 1;
      const bool is_v = c >= 2 * chunks;
      const uint4 x = *reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + size_t(b) * row_bytes + q * 16);
      uint8_t* dst = (is_v ? v_ring : k_ring) + (size_t(b) * 2 * L + s + copy * L) * row_bytes + q * 16;
      *reinterpret_cast<uint4*>(dst) = x;
    }
    if (threadIdx.x < 2) z_ring[size_t(b) * 2 * L + s + threadIdx.x * L] = z_new[b];
  }
  if (threadIdx.x == 0) {
    const bool done = p >= 0 && (p + 1) % m == 0 && (p + 1) / m - 1 < cap;
    plan[b] = done ? (p - m + 1) % L : 0;
    plan[B + b] = done ? (p + 1) / m - 1 : -1;
    const int q0 = max(0, p - L + 1);
    raw_pos0[b] = p >= 0 ? q0 - q0 % L : 0;
  }
}

}  // namespace

size_t csa_kv_append_workspace_size(int B) { return B <= 0 ? 0 : ((size_t(B) * 8 + 255) / 256) * 256; }

extern "C" csa_status_t csa_kv_cache_append(const void* k_new, const void* v_new, const float* z_new, int32_t io_dtype,
                                            const int32_t* pos, int32_t B, int32_t d, int32_t L_ring, void* k_ring,
                                            void* v_ring, float* z_ring, int32_t m, int32_t cap, int32_t ckv_dtype,
                                            void* ck, void* cv, float* ck_scale, float* cv_scale, int32_t* raw_pos0,
                                            void* ws, size_t ws_bytes, void* stream) {
  if (!k_new || !v_new || !z_new || !pos || !k_ring || !v_ring || !z_ring || !ck || !cv || !raw_pos0)
    return CSA_EINVAL;
  if (io_dtype != CSA_BF16 && io_dtype != CSA_F32) return CSA_EINVAL;
  if (!csa_dtype_ok(ckv_dtype)) return CSA_EINVAL;
  if (ckv_dtype == CSA_FP8_E4M3 && (!ck_scale || !cv_scale)) return CSA_EINVAL;
  if (d != kHeadDim || B < 0 || m < 1 || cap < 0 || L_ring < m) return CSA_EINVAL;
  if (long(B) * 2 * L_ring > 0x7FFFFFFFL) return CSA_ENOTSUP;
  if (B == 0) return CSA_OK;
  const size_t need = csa_kv_append_workspace_size(B);
  if (!ws || ws_bytes < need) return CSA_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* plan = static_cast<int32_t*>(ws);
  const int row_bytes = d * (io_dtype == CSA_F32 ? 4 : 2);
  hipLaunchKernelGGL(ring_append_kernel, dim3(unsigned(B)), dim3(64), 0, st, static_cast<const uint8_t*>(k_new),
                     static_cast<const uint8_t*>(v_new), z_new, pos, B, row_bytes, L_ring,
                     static_cast<uint8_t*>(k_ring), static_cast<uint8_t*>(v_ring), z_ring, m, cap, plan, raw_pos0);
  if (hipGetLastError() != hipSuccess) return CSA_EHIP;
  const hipError_t e = csa_cmp::launch_compress_append(io_dtype, ckv_dtype, k_ring, v_ring, z_ring, B, 2 * L_ring, m,
                                                       ck, cv, ck_scale, cv_scale, cap, plan, st);
  return e == hipSuccess ? CSA_OK : CSA_EHIP;
}
