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

size_t csa_kv_append_workspace_size(int) { return 0; }

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
