// Host-only entry points of the C ABI: workspace sizing, status text, version.
#include "common.hpp"

size_t csa_attn_workspace_size(long rows, int H, int n_list, bool invariant);
size_t csa_kv_append_workspace_size(int B);
size_t csa_indexer_topk_workspace_size(long rows, int T_q, int d_I, int cap);
size_t csa_topk_workspace_size(long rows, int cap);
size_t csa_attn_varlen_workspace_size(long n_rows, int n_seq, int H, int n_list, bool dense);
size_t csa_indexer_topk_varlen_workspace_size(long n_rows, int cap);

extern "C" size_t csa_workspace_size(int32_t op, int32_t B, int32_t T_q, int32_t H, int32_t d, int32_t n_keys) {
  if (B < 0 || T_q < 0 || n_keys < 0) return size_t(-1);
  switch (op) {
    case CSA_OP_TOPK:
      return csa_topk_workspace_size(long(B) * T_q, n_keys);
    case CSA_OP_INDEXER_TOPK:
      return csa_indexer_topk_workspace_size(long(B) * T_q, T_q, d, n_keys);
    case CSA_OP_SPARSE_ATTN:
    case CSA_OP_DENSE_ATTN:
    case CSA_OP_SPARSE_ATTN_BATCH_INVARIANT:
    case CSA_OP_DENSE_ATTN_BATCH_INVARIANT:
      if (d != kHeadDim || H < 16 || H > 128 || H % 16 != 0) return size_t(-1);
      return csa_attn_workspace_size(long(B) * T_q, H, n_keys,
                                     op == CSA_OP_SPARSE_ATTN_BATCH_INVARIANT || op == CSA_OP_DENSE_ATTN_BATCH_INVARIANT);
    case CSA_OP_KV_CACHE_APPEND:
      return csa_kv_append_workspace_size(B);
    case CSA_OP_INDEXER_TOPK_VARLEN:   // B = n_rows
      return csa_indexer_topk_varlen_workspace_size(B, n_keys);
    case CSA_OP_SPARSE_ATTN_VARLEN:    // B = n_rows, T_q = sequences
    case CSA_OP_DENSE_ATTN_VARLEN:
      if (d != kHeadDim || H < 16 || H > 128 || H % 16 != 0) return size_t(-1);
      return csa_attn_varlen_workspace_size(B, T_q, H, n_keys, op == CSA_OP_DENSE_ATTN_VARLEN);
    default:
      return size_t(-1);
  }
}

extern "C" const char* csa_status_str(int32_t status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_EINVAL: return "CSA_EINVAL: invalid argument";
    case CSA_ENOTSUP: return "CSA_ENOTSUP: unsupported combination";
    case CSA_EHIP: return "CSA_EHIP: HIP runtime error";
    case CSA_EWORKSPACE: return "CSA_EWORKSPACE: workspace missing or too small";
    case CSA_ESCRATCH: return "CSA_ESCRATCH: the call needs more than the allocation-free call's fixed scratch";
    default: return "unknown status";
  }
}

extern "C" int32_t csa_abi_version(void) { return 104; }
