/* csa.h -- C ABI of libcsa: compressed sparse attention (CSA) and heavily
 * compressed attention (HCA) on one AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V4 hybrid attention) as the public pages describe it:
 *   - CSA compresses every m tokens' key/value pairs into one entry, scores
 *     the entries against the query with a light FP4 "lightning indexer",
 *     keeps the top-k and attends only over those (blog.nickys.cn DeepSeek-V4
 *     post, section 三大架构改动 §1 CSA; "DeepSeek-V4 技术分析报告", §3 架构层);
 *   - HCA compresses every m' >> m tokens into one entry and attends densely
 *     over all entries (blog.nickys.cn, 三大架构改动 §2 HCA);
 *   - both add an uncompressed sliding-window branch so each token fully sees
 *     its nearest neighbours (sz-guanghua.com.cn ifanr repost, 百萬長上下文);
 *   - the indexer's query-key path is MXFP4 ("DeepSeek V4技术揭秘", §一);
 *   - the KV cache mixes BF16 and FP8 ("DeepSeek-V4 技术分析报告", 工程层).
 * The pooling rule and the indexer score formula are not given on the pages;
 * this library fixes them as documented on each call.
 *
 * Conventions for every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronizes; work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously.
 *   - Arrays are dense, row-major, last dimension innermost, unless a
 *     leading-dimension argument says otherwise.
 *   - head dimension d must be 128.
 *   - bf16 values are raw bit patterns (uint16); fp8 values are OCP E4M3FN
 *     codes (uint8; 0x7F/0xFF = NaN are never produced and must not be fed).
 *   - MXFP4 (OCP MX v1.0): E2M1 codes, two per byte, element 2i in the LOW
 *     nibble of byte i; one E8M0 scale byte per 32 consecutive elements
 *     (value 2^(e-127); 0xFF = NaN must not be fed).
 *   - Positions: query i of sequence b sits at absolute position
 *     q_pos0[b] + i.  Compressed entry e (block size m) covers positions
 *     [e*m, (e+1)*m) and is visible to position t iff e < floor((t+1)/m).
 *     Row r of a raw window buffer holds position raw_pos0[b] + r.
 *   - Argument errors return CSA_EINVAL (unsupported but well-formed
 *     combinations CSA_ENOTSUP) before anything is enqueued and leave every
 *     output untouched.  A HIP launch error returns CSA_EHIP.  Conditions
 *     that depend on device-resident data (positions) cannot be checked on
 *     the host; they are documented as preconditions per call.
 *   - Results are bitwise reproducible run to run: work splits depend only
 *     on the shape arguments and every reduction has a fixed order.
 *   - The library keeps no state beyond a mutex-guarded host record of which
 *     kernels have had their LDS limit raised on which device, and the fixed
 *     device scratch of csa_sparse_attn_noalloc; calls on different streams
 *     may overlap provided their outputs and workspaces do not alias.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_EINVAL = 1,     /* invalid argument (shape, pointer, enum)          */
  CSA_ENOTSUP = 2,    /* valid but unsupported combination               */
  CSA_EHIP = 3,       /* HIP runtime error while enqueueing               */
  CSA_EWORKSPACE = 4, /* workspace missing or smaller than required       */
  CSA_ESCRATCH = 5    /* beyond the fixed scratch of csa_sparse_attn_noalloc */
} csa_status_t;

typedef enum {
  CSA_BF16 = 0,       /* bf16 bit patterns                                 */
  CSA_F32 = 1,        /* IEEE fp32                                         */
  CSA_FP8_E4M3 = 2    /* OCP E4M3FN codes + one fp32 scale per entry       */
} csa_dtype_t;

typedef enum {
  CSA_OP_TOPK = 0,
  CSA_OP_SPARSE_ATTN = 1,
  CSA_OP_DENSE_ATTN = 2,
  CSA_OP_INDEXER_TOPK = 3,
  CSA_OP_SPARSE_ATTN_BATCH_INVARIANT = 4,
  CSA_OP_DENSE_ATTN_BATCH_INVARIANT = 5,
  CSA_OP_KV_CACHE_APPEND = 6,
  CSA_OP_INDEXER_TOPK_VARLEN = 7,
  CSA_OP_SPARSE_ATTN_VARLEN = 8,
  CSA_OP_DENSE_ATTN_VARLEN = 9
} csa_op_t;

/* ---------------------------------------------------------------------
 * csa_compress_kv -- pool each complete block of m tokens into one entry.
 *
 * Passage: every m tokens' key/value pairs become one entry, so the sequence
 * shrinks to 1/m (blog.nickys.cn, 三大架构改动 §1 CSA); HCA uses the same
 * operation with a far larger block m' (§2 HCA).
 * Pooling rule (fixed by this library): one scalar logit z per token, shared
 * by K and V; for block e, a_j = softmax(z[e*m .. e*m+m-1])_j and
 *   k_out[e] = sum_j a_j * k[e*m + j],  v_out[e] = sum_j a_j * v[e*m + j],
 * accumulated in fp32.  Storage: CSA_BF16 (round to nearest even),
 * CSA_F32, or CSA_FP8_E4M3 with per-entry scale = amax/448 (1 if amax == 0)
 * and code = RNE_e4m3(x / scale) saturated at +-448, separately for K and V.
 *
 *   k, v        [B, ld_in, d] in in_dtype (CSA_BF16 or CSA_F32); rows 0..L-1
 *               of each sequence are pooled
 *   logits      [B, ld_in] fp32
 *   L           tokens to pool per sequence; L % m == 0; L <= ld_in
 *   k_out,v_out [B, ld_out, d] in out_dtype; entries 0..L/m-1 are written
 *   k_scale_out, v_scale_out  [B, ld_out] fp32; required iff out_dtype is
 *               CSA_FP8_E4M3, ignored otherwise
 * Pointers may be offset by the caller to pool a tail (e.g. the block just
 * completed during decoding) into any entry slot.
 * ------------------------------------------------------------------- */
csa_status_t csa_compress_kv(const void* k, const void* v, int32_t in_dtype,
                             const float* logits, int32_t B, int32_t L, int32_t ld_in,
                             int32_t d, int32_t m, void* k_out, void* v_out,
                             float* k_scale_out, float* v_scale_out, int32_t ld_out,
                             int32_t out_dtype, void* stream);

/* ---------------------------------------------------------------------
 * csa_compress_kv_varlen -- the new entries of several sequences in one
 * launch (decode rows that complete a block and prefill chunks together).
 *
 * Passage: as csa_compress_kv.  Sequence b has n_b = cu_entries[b+1] -
 * cu_entries[b] new entries; its j-th (j < n_b) pools raw rows
 * row0[b] + j*m .. row0[b] + j*m + m - 1 of k[b], v[b], logits[b] into entry
 * entry0[b] + j of k_out[b], v_out[b] (and the scales), exactly as
 * csa_compress_kv pools a block (bit-identical results).
 *
 *   k, v, logits, in_dtype, d, m, k_out .. out_dtype   as csa_compress_kv
 *              ([B, ld_in, d], [B, ld_in], [B, ld_out, d], [B, ld_out])
 *   cu_entries [B+1] int32 (device): cu_entries[0] = 0, non-decreasing,
 *              cu_entries[B] = n_entries
 *   row0, entry0 [B] int32 (device)
 *   n_entries  all sequences' new entries (host value); 0 returns CSA_OK
 * Preconditions: row0[b] >= 0, row0[b] + n_b*m <= ld_in; entry0[b] >= 0,
 * entry0[b] + n_b <= ld_out.
 * ------------------------------------------------------------------- */
csa_status_t csa_compress_kv_varlen(const void* k, const void* v, int32_t in_dtype,
                                    const float* logits, int32_t B, int32_t ld_in, int32_t d,
                                    int32_t m, const int32_t* cu_entries, const int32_t* row0,
                                    const int32_t* entry0, int32_t n_entries, void* k_out,
                                    void* v_out, float* k_scale_out, float* v_scale_out,
                                    int32_t ld_out, int32_t out_dtype, void* stream);

/* ---------------------------------------------------------------------
 * csa_mxfp4_quantize -- real vectors to the indexer's MXFP4 operands.
 *
 * Passage: the indexer's query-key path is MXFP4 ("DeepSeek V4技术揭秘",
 * §一 基础设施; sz-guanghua.com.cn ifanr repost, 百萬長上下文, FP4 scores).
 * Conversion (OCP Microscaling v1.0, restated): per 32-element block,
 * X = floor(log2(max |x|)) - 2 clamped to [-127, 127] (-127 for an all-zero
 * block); code_i = E2M1 nearest to x_i / 2^X, ties to the even code,
 * magnitudes past 6 saturated, sign bit of x_i kept; e8m0 = X + 127.
 *
 *   x      [n_vec, d] in in_dtype (CSA_BF16 or CSA_F32), finite values
 *   codes  [n_vec, d/2] u8 (output): element 2i in the low nibble of byte i
 *   e8m0   [n_vec, d/32] u8 (output)
 * Limits: d a positive multiple of 32.  The outputs feed csa_indexer_scores,
 * csa_indexer_topk and csa_compress_indexer_topk as q_codes / q_e8m0 or
 * k_codes / k_e8m0 directly.
 * ------------------------------------------------------------------- */
csa_status_t csa_mxfp4_quantize(const void* x, int32_t in_dtype, int64_t n_vec, int32_t d,
                                uint8_t* codes, uint8_t* e8m0, void* stream);

/* ---------------------------------------------------------------------
 * csa_indexer_scores -- lightning-indexer relevance of every compressed entry.
 *
 * Passage: the indexer scores each query token against each compressed block
 * in FP4 (sz-guanghua.com.cn ifanr repost, 百萬長上下文); MXFP4 on the
 * indexer's query-key path ("DeepSeek V4技术揭秘", §一).
 * Score (fixed by this library):
 *   scores[b,i,e] = sum_h w[b,i,h] * max(0, q[b,i,h,:] . kx[b,e,:])
 * for e < nvis = floor((t+1)/m), t = q_pos0[b] + i; -inf for nvis <= e < cap.
 * Products of MXFP4 values are exact; sums are fp32.
 *
 *   q_codes [B, T_q, H_I, d_I/2] u8     q_e8m0 [B, T_q, H_I, d_I/32] u8
 *   w       [B, T_q, H_I] fp32
 *   k_codes [B, cap, d_I/2] u8          k_e8m0 [B, cap, d_I/32] u8
 *   q_pos0  [B] int32 (device)
 *   scores  [B, T_q, cap] fp32 (output)
 * Limits: H_I in {4, 8, 16}; d_I a multiple of 32, 32 <= d_I <= 512.
 * Precondition: nvis(t) <= cap (entries at or past cap are taken as absent).
 * ------------------------------------------------------------------- */
csa_status_t csa_indexer_scores(const uint8_t* q_codes, const uint8_t* q_e8m0,
                                const float* w, const uint8_t* k_codes,
                                const uint8_t* k_e8m0, const int32_t* q_pos0, int32_t B,
                                int32_t T_q, int32_t H_I, int32_t d_I, int32_t cap,
                                int32_t m, float* scores, void* stream);

/* ---------------------------------------------------------------------
 * csa_topk -- keep the k most relevant visible entries per query.
 *
 * Passage: keep the k compressed entries most relevant to the query
 * (blog.nickys.cn, 三大架构改动 §1 CSA).
 * Rule (fixed by this library): candidates are e < min(nvis(t), cap);
 * larger score first, equal scores (with -0 == +0) by lower index; the first
 * min(k, candidates) are written in ASCENDING index order, then -1 up to k.
 *
 *   scores [B, T_q, cap] fp32 (NaN must not occur)
 *   idx    [B, T_q, k] int32 (output)
 *   ws, ws_bytes  workspace of csa_workspace_size(CSA_OP_TOPK, ...) bytes
 *                 (may be NULL when that size is 0)
 * ------------------------------------------------------------------- */
csa_status_t csa_topk(const float* scores, const int32_t* q_pos0, int32_t B, int32_t T_q,
                      int32_t cap, int32_t m, int32_t k, int32_t* idx, void* ws,
                      size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_indexer_topk -- indexer scores and top-k selection in one call.
 *
 * Passages: as csa_indexer_scores and csa_topk (the indexer scores every
 * query token against every compressed block in FP4, sz-guanghua.com.cn
 * ifanr repost, 百萬長上下文; CSA keeps the most relevant k entries,
 * blog.nickys.cn, 三大架构改动 §1 CSA).
 * Result: idx equals, bit for bit, csa_topk(csa_indexer_scores(...)) on the
 * same arguments, for any input values.  In general the scoring pass stores
 * 16-bit order-preserving score keys (2 bytes per (query, entry) instead of
 * 4) and the selection re-scores only the entries whose 16-bit key ties the
 * k-th one, with the scoring pass's own arithmetic.  Decoding shapes score
 * and pre-select each 2048-entry slice in one pass (the fp32 scores go to
 * the workspace for the exact fallback), then select per row.
 *
 *   q_codes .. q_pos0, B .. m   as csa_indexer_scores (same layouts, limits
 *                               and preconditions)
 *   k         entries to keep; 1 <= k <= 32767 (larger: CSA_ENOTSUP)
 *   idx       [B, T_q, k] int32 (output), as csa_topk
 *   ws, ws_bytes  workspace of csa_workspace_size(CSA_OP_INDEXER_TOPK, B, T_q,
 *             0, d_I, cap) bytes (no initial contents needed): B*T_q*cap*2 in
 *             general; for decoding (T_q == 1, B <= 128, cap >= 8192,
 *             d_I <= 256) the fp32 scores plus per-slice candidate lists
 *             (about B*cap*8 bytes).
 *             Calls that share a workspace must be ordered on one stream.
 * ------------------------------------------------------------------- */
csa_status_t csa_indexer_topk(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                              const uint8_t* k_codes, const uint8_t* k_e8m0,
                              const int32_t* q_pos0, int32_t B, int32_t T_q, int32_t H_I,
                              int32_t d_I, int32_t cap, int32_t m, int32_t k, int32_t* idx,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_indexer_topk_varlen -- csa_indexer_topk over packed query rows of any
 * mix of sequences: decode rows and prefill chunks in one call.
 *
 * Passages: as csa_indexer_topk.  Sequence b's query rows are packed rows
 * cu_rows[b] .. cu_rows[b+1]-1, at positions q_pos0[b], q_pos0[b]+1, ...;
 * each row's selection is, bit for bit, the one csa_indexer_topk gives that
 * row in a call on its own sequence (any input values).
 *
 *   q_codes [n_rows, H_I, d_I/2] u8    q_e8m0 [n_rows, H_I, d_I/32] u8
 *   w       [n_rows, H_I] fp32
 *   k_codes [B, cap, d_I/2] u8         k_e8m0 [B, cap, d_I/32] u8
 *   cu_rows [B+1] int32 (device)       q_pos0 [B] int32 (device)
 *   idx     [n_rows, k] int32 (output), as csa_topk
 *   ws, ws_bytes  csa_workspace_size(CSA_OP_INDEXER_TOPK_VARLEN, n_rows, 0, 0,
 *                 0, cap) = n_rows*cap*2 bytes, no initial contents needed
 * Limits: as csa_indexer_topk; ceil(n_rows / (64/H_I)) + B <= 65535.
 * Preconditions: cu_rows[0] = 0, cu_rows non-decreasing, cu_rows[B] = n_rows;
 * nvis(t) <= cap for every row.  n_rows = 0 returns CSA_OK at once.
 * ------------------------------------------------------------------- */
csa_status_t csa_indexer_topk_varlen(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                                     const uint8_t* k_codes, const uint8_t* k_e8m0,
                                     const int32_t* cu_rows, const int32_t* q_pos0, int32_t B,
                                     int32_t n_rows, int32_t H_I, int32_t d_I, int32_t cap,
                                     int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                                     void* stream);

/* ---------------------------------------------------------------------
 * csa_compress_indexer_topk -- a CSA layer's compression and its indexer
 * top-k in one call.
 *
 * Passages: as csa_compress_kv (every m tokens' K/V become one entry,
 * blog.nickys.cn, 三大架构改动 §1 CSA) and csa_indexer_topk.
 * Result: exactly that of
 *   csa_compress_kv(k, v, in_dtype, logits, B, L, ld_in, d, m, k_out, v_out,
 *                   k_scale_out, v_scale_out, ld_out, out_dtype, stream);
 *   csa_indexer_topk(q_codes, ..., B, T_q, H_I, d_I, cap, m, k_sel, idx, ws,
 *                    ws_bytes, stream);
 * on the same arguments (B and m are shared: the layer's sequences and its
 * compression ratio).  The two parts are independent (the compression writes
 * the attention's entries, the indexer reads its own keys), so for decoding
 * shapes (those of the csa_indexer_topk decode path, with m < 32) the
 * compression runs inside the selection's launch on CUs the selection leaves
 * idle, saving a launch on the decode critical path; otherwise the two run
 * as two launches.
 *
 *   k .. out_dtype    as csa_compress_kv (without B, m)
 *   q_codes .. idx    as csa_indexer_topk (k_sel = its k)
 *   ws, ws_bytes      as csa_indexer_topk (same size)
 * Precondition: k_out, v_out and the scales overlap none of the indexer's
 * inputs, idx or the workspace.  Argument errors of either part are reported
 * before anything runs.
 * ------------------------------------------------------------------- */
csa_status_t csa_compress_indexer_topk(const void* k, const void* v, int32_t in_dtype,
                                       const float* logits, int32_t L, int32_t ld_in, int32_t d,
                                       void* k_out, void* v_out, float* k_scale_out,
                                       float* v_scale_out, int32_t ld_out, int32_t out_dtype,
                                       const uint8_t* q_codes, const uint8_t* q_e8m0,
                                       const float* w, const uint8_t* k_codes,
                                       const uint8_t* k_e8m0, const int32_t* q_pos0, int32_t B,
                                       int32_t T_q, int32_t H_I, int32_t d_I, int32_t cap,
                                       int32_t m, int32_t k_sel, int32_t* idx, void* ws,
                                       size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_sparse_attn -- attention over the selected entries plus the window.
 *
 * Passage: attention runs only over the k selected compressed entries, with a
 * few uncompressed sliding-window entries kept as well (blog.nickys.cn,
 * 三大架构改动 §1 CSA; "DeepSeek-V4 技术分析报告", 滑动窗口分支).
 * For each query (t) and head h, one softmax over the union (no de-duplication)
 *   { sm * q[h].ck[e] : e in idx[b,i,:], e >= 0 } U
 *   { sm * q[h].k_win[p - raw_pos0] : max(0, t-W+1) <= p <= t }
 * and out = sum p * value.  All H query heads share the single KV head.
 * An empty key set gives out = 0, lse = -inf.
 *
 *   q        [B, T_q, H, d] in io_dtype (CSA_BF16 or CSA_F32)
 *   ck, cv   [B, cap, d] compressed entries in ckv_dtype (BF16, F32 or
 *            FP8_E4M3 with ck_scale, cv_scale [B, cap] fp32)
 *   idx      [B, T_q, k] int32, -1 = empty slot (csa_topk output)
 *   k_win, v_win [B, L_raw, d] raw tokens in io_dtype
 *   raw_pos0 [B], q_pos0 [B] int32 (device)
 *   sm_scale logit scale (pass 1/sqrt(d) for the usual choice)
 *   out      [B, T_q, H, d] in io_dtype;  lse [B, T_q, H] fp32 or NULL
 *   ws       workspace of csa_workspace_size(CSA_OP_SPARSE_ATTN, B, T_q, H, d, k + W)
 *            bytes (no initial contents needed; may be NULL when that size is
 *            0).  Calls that share a workspace must be ordered on one stream.
 * Limits: H a multiple of 16 in [16, 128]; W >= 0; k >= 1.
 * Preconditions: idx entries are -1 or in [0, cap); the raw buffer covers
 * window(t) (rows outside [0, L_raw) are skipped).
 * ------------------------------------------------------------------- */
csa_status_t csa_sparse_attn(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                             const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                             int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                             const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                             const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q,
                             int32_t H, int32_t d, float sm_scale, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * hca_dense_attn -- attention over ALL visible compressed entries + window.
 *
 * Passage: HCA makes no sparse selection and attends densely over every
 * compressed entry (blog.nickys.cn, 三大架构改动 §2 HCA); the window branch as
 * for CSA (sz-guanghua.com.cn ifanr repost, 百萬長上下文).
 * Key set for query t: entries e < min(floor((t+1)/m_prime), cap) and
 * window(t); otherwise exactly as csa_sparse_attn.
 * ws: csa_workspace_size(CSA_OP_DENSE_ATTN, B, T_q, H, d, cap + W) bytes, same
 * contract as csa_sparse_attn.
 * ------------------------------------------------------------------- */
csa_status_t hca_dense_attn(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                            const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                            int32_t cap, int32_t m_prime, const void* k_win, const void* v_win,
                            const int32_t* raw_pos0, int32_t L_raw, const int32_t* q_pos0,
                            int32_t W, int32_t B, int32_t T_q, int32_t H, int32_t d,
                            float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------
 * csa_sparse_attn_noalloc -- csa_sparse_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, results (bit for bit) and limits as csa_sparse_attn,
 * without ws / ws_bytes: the split partials go to a fixed 32 MiB device array
 * inside the library (one per GPU, held until the process ends).  Nothing is
 * allocated or freed; the first call on a device looks up that device's
 * array address.  The array needs no initial contents.
 * Errors: a call whose csa_workspace_size(CSA_OP_SPARSE_ATTN, ...) exceeds
 * 32 MiB returns CSA_ESCRATCH before anything is enqueued (decode shapes need
 * a few MiB: 16 rows x 64 heads over 1152 keys take 4.8 MiB).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or host threads without ordering) race and
 * must not be issued.
 * ------------------------------------------------------------------- */
csa_status_t csa_sparse_attn_noalloc(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                     const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                     int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                                     const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                                     const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q,
                                     int32_t H, int32_t d, float sm_scale, void* out, float* lse,
                                     void* stream);

/* ---------------------------------------------------------------------
 * csa_sparse_attn_batch_invariant, hca_dense_attn_batch_invariant -- the
 * same attention as csa_sparse_attn / hca_dense_attn (same arguments, same
 * limits, same results to the same tolerance), with one more guarantee: the
 * bits of a query row's out and lse depend only on that row's inputs and on
 * n_keys (k + W, resp. cap + W), never on B, T_q or the other rows.  A row
 * computed in a batch of one and in a batch of many, or in prefill chunks of
 * any length, comes out bit-identical.
 *
 * The plain calls choose how many pieces to split each key list into from
 * the number of rows (to fill the chip) and, for many-query dense prefill, a
 * different kernel; each choice sums the softmax in another order.  These
 * calls fix the split at ceil(n_keys / 64) chunks of 64 keys cut into pieces
 * of max(2, ceil(chunks / 64)) chunks, and always use the split kernel: small
 * batches then run fewer, longer blocks than the plain calls and are slower.
 * Passage: the pages define the operation (see csa_sparse_attn); the
 * ordering guarantee is this library's.
 * ws: csa_workspace_size(CSA_OP_SPARSE_ATTN_BATCH_INVARIANT, ...) resp.
 * (CSA_OP_DENSE_ATTN_BATCH_INVARIANT, ...) with the same other arguments as
 * for the plain call.
 * ------------------------------------------------------------------- */
csa_status_t csa_sparse_attn_batch_invariant(
    const void* q, int32_t io_dtype, const void* ck, const void* cv, const float* ck_scale,
    const float* cv_scale, int32_t ckv_dtype, int32_t cap, const int32_t* idx, int32_t k,
    const void* k_win, const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
    const int32_t* q_pos0, int32_t W, int32_t B, int32_t T_q, int32_t H, int32_t d,
    float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);
csa_status_t hca_dense_attn_batch_invariant(
    const void* q, int32_t io_dtype, const void* ck, const void* cv, const float* ck_scale,
    const float* cv_scale, int32_t ckv_dtype, int32_t cap, int32_t m_prime, const void* k_win,
    const void* v_win, const int32_t* raw_pos0, int32_t L_raw, const int32_t* q_pos0, int32_t W,
    int32_t B, int32_t T_q, int32_t H, int32_t d, float sm_scale, void* out, float* lse,
    void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_sparse_attn_varlen, hca_dense_attn_varlen -- one call over the packed
 * query rows of several sequences: decode rows and prefill chunks together.
 *
 * Passage: the operation is csa_sparse_attn's / hca_dense_attn's.  Sequence
 * b's query rows are packed rows cu_rows[b] .. cu_rows[b+1]-1 at positions
 * q_pos0[b], q_pos0[b]+1, ...; each row's key set is the one those calls
 * give a query of that sequence at that position.
 * invariant != 0: the batch-invariant plan, so row r's bits equal those of
 * the *_batch_invariant call on its own sequence.  invariant == 0: the
 * kernels the plain calls would pick for a call of n_rows rows (bits may
 * depend on the batch); with bf16 queries, H in {32, 64, 128} and at least
 * 256 rows, the dense call runs the many-query kernel over tiles of each
 * sequence's rows, with the key lists of sequences of at most 8 / 4 / 2 rows
 * (H = 32 / 64 / 128) cut into pieces spread over the chip and merged after.
 *
 *   q        [n_rows, H, d] io_dtype;  out [n_rows, H, d];  lse [n_rows, H] or NULL
 *   idx      [n_rows, k] int32 (sparse)
 *   ck, cv, ck_scale, cv_scale, k_win, v_win, raw_pos0: per sequence, as for
 *            the plain calls ([B, cap, d], [B, L_raw, d], [B])
 *   cu_rows  [B+1] int32 (device): cu_rows[0] = 0, non-decreasing,
 *            cu_rows[B] = n_rows;  q_pos0 [B] int32 (device), >= 0
 *   ws       csa_workspace_size(CSA_OP_SPARSE_ATTN_VARLEN resp.
 *            CSA_OP_DENSE_ATTN_VARLEN, n_rows, B, H, d, n_keys) bytes (either
 *            mode), n_keys = k + W resp. cap + W
 * Limits as for the plain calls.  n_rows = 0 returns CSA_OK at once.
 * ------------------------------------------------------------------- */
csa_status_t csa_sparse_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                    const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                    int32_t cap, const int32_t* idx, int32_t k, const void* k_win,
                                    const void* v_win, const int32_t* raw_pos0, int32_t L_raw,
                                    const int32_t* cu_rows, const int32_t* q_pos0, int32_t n_rows,
                                    int32_t W, int32_t B, int32_t H, int32_t d, float sm_scale,
                                    int32_t invariant, void* out, float* lse, void* ws,
                                    size_t ws_bytes, void* stream);
csa_status_t hca_dense_attn_varlen(const void* q, int32_t io_dtype, const void* ck, const void* cv,
                                   const float* ck_scale, const float* cv_scale, int32_t ckv_dtype,
                                   int32_t cap, int32_t m_prime, const void* k_win, const void* v_win,
                                   const int32_t* raw_pos0, int32_t L_raw, const int32_t* cu_rows,
                                   const int32_t* q_pos0, int32_t n_rows, int32_t W, int32_t B,
                                   int32_t H, int32_t d, float sm_scale, int32_t invariant,
                                   void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_kv_cache_append -- one decode step's token into a layer's KV cache.
 *
 * Passage: the newest uncompressed tokens are kept in bf16 beside compressed
 * entries that may be fp8 (ferris DeepSeek-V4 analysis, 工程层, heterogeneous
 * KV cache); every m tokens' K/V become one entry (blog.nickys.cn, 三大架构改动
 * §1 CSA, §2 HCA).  The ring layout is this library's.
 *
 * For each sequence b with pos[b] >= 0 (its new token's position; < 0 = idle,
 * nothing written):
 *   - the token's K, V rows and logit are written to ring rows pos mod L_ring
 *     and pos mod L_ring + L_ring;
 *   - when pos + 1 is a multiple of m and entry (pos + 1)/m - 1 < cap, the m
 *     rows of the completed block are pooled into that entry exactly as
 *     csa_compress_kv pools a block (bit-identical results);
 *   - raw_pos0[b] is set so that the attention calls, given k_win = k_ring,
 *     v_win = v_ring, L_raw = 2 * L_ring, read the window of a query at pos
 *     from the ring: raw_pos0 = q0 - (q0 mod L_ring), q0 = max(0, pos-L_ring+1)
 *     (0 for idle sequences).  Valid for windows W <= L_ring.
 *
 *   k_new, v_new  [B, d] in io_dtype (CSA_BF16 or CSA_F32);  z_new [B] fp32
 *   pos           [B] int32 (device)
 *   k_ring, v_ring [B, 2*L_ring, d] io_dtype;  z_ring [B, 2*L_ring] fp32;
 *                 caller-owned, persistent across calls, no initial contents
 *   ck, cv        [B, cap, d] compressed cache in ckv_dtype (BF16, F32, or
 *                 FP8_E4M3 with ck_scale, cv_scale [B, cap])
 *   raw_pos0      [B] int32 output (device)
 *   ws, ws_bytes  unused (csa_workspace_size(CSA_OP_KV_CACHE_APPEND, ...) is 0);
 *                 may be NULL, 0.  Calls on one cache must be ordered on one
 *                 stream.
 * Limits: d = 128, m <= L_ring, B * 2 * L_ring < 2^31.
 * Preconditions: each sequence's positions advance by one per call (the
 * ring holds what earlier calls wrote).
 * ------------------------------------------------------------------- */
csa_status_t csa_kv_cache_append(const void* k_new, const void* v_new, const float* z_new,
                                 int32_t io_dtype, const int32_t* pos, int32_t B, int32_t d,
                                 int32_t L_ring, void* k_ring, void* v_ring, float* z_ring,
                                 int32_t m, int32_t cap, int32_t ckv_dtype, void* ck, void* cv,
                                 float* ck_scale, float* cv_scale, int32_t* raw_pos0, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * csa_mxfp4_quantize_appended -- the MXFP4 indexer key of each entry a
 * cache append has just completed.
 *
 * Passage: as csa_mxfp4_quantize.  For each sequence b whose token at pos[b]
 * completes a block by the rule of csa_kv_cache_append ((pos + 1) mod m = 0,
 * entry e = (pos + 1)/m - 1 < cap), vector e of x[b] is converted exactly as
 * csa_mxfp4_quantize converts it (bit-identical codes and scales) into
 * codes[b, e] and e8m0[b, e]; nothing else is written.  Together with a
 * csa_kv_cache_append on a ring of per-token indexer keys with fp32 entries,
 * this appends the indexer's MXFP4 key cache.
 *
 *   x      [B, cap, d] in_dtype (CSA_BF16 or CSA_F32): the pooled keys
 *   pos    [B] int32 (device), as passed to csa_kv_cache_append
 *   codes  [B, cap, d/2] uint8;  e8m0 [B, cap, d/32] uint8
 * Limits: d a positive multiple of 32.
 * ------------------------------------------------------------------- */
csa_status_t csa_mxfp4_quantize_appended(const void* x, int32_t in_dtype, const int32_t* pos,
                                         int32_t B, int32_t cap, int32_t m, int32_t d,
                                         uint8_t* codes, uint8_t* e8m0, void* stream);

/* ---------------------------------------------------------------------
 * csa_indexer_key_append -- one decode token's indexer key into the
 * indexer's ring and, when it completes a block, its MXFP4 key entry.
 *
 * Passage: as csa_kv_cache_append (per-entry keys pooled from the tokens'
 * keys) and csa_mxfp4_quantize (MXFP4 on the indexer path).  For each
 * sequence b with pos[b] >= 0 the key row and logit go to ring rows
 * pos mod L_ring and pos mod L_ring + L_ring; when pos + 1 is a multiple of m
 * and e = (pos + 1)/m - 1 < cap, the block is pooled (the K side of
 * csa_kv_cache_append with fp32 entries, bit for bit) and converted as
 * csa_mxfp4_quantize converts it into codes[b, e], e8m0[b, e].  The same
 * results as csa_kv_cache_append (fp32 entries) followed by
 * csa_mxfp4_quantize_appended, in one launch and without a V side.
 *
 *   k_new [B, d] io_dtype (CSA_BF16 or CSA_F32);  z_new [B] fp32;  pos [B]
 *   k_ring [B, 2*L_ring, d] io_dtype;  z_ring [B, 2*L_ring] fp32
 *   codes [B, cap, d/2], e8m0 [B, cap, d/32] uint8
 * Limits: d = 128; m < 32; m <= L_ring.
 * ------------------------------------------------------------------- */
csa_status_t csa_indexer_key_append(const void* k_new, const float* z_new, int32_t io_dtype,
                                    const int32_t* pos, int32_t B, int32_t d, int32_t L_ring,
                                    void* k_ring, float* z_ring, int32_t m, int32_t cap,
                                    uint8_t* codes, uint8_t* e8m0, void* stream);

/* ---------------------------------------------------------------------
 * csa_decode_append -- both cache appends of a CSA layer's decode token
 * (its K/V and its indexer key) in one launch.
 *
 * Passage: as csa_kv_cache_append and csa_indexer_key_append.  The results
 * are exactly those of
 *   csa_kv_cache_append(k_new, v_new, z_new, io_dtype, pos, B, d, L_ring,
 *                       k_ring, v_ring, z_ring, m, cap, ckv_dtype, ck, cv,
 *                       ck_scale, cv_scale, raw_pos0, NULL, 0, stream)
 * followed by
 *   csa_indexer_key_append(ki_new, zi_new, io_dtype, pos, B, d, Li_ring,
 *                          ki_ring, zi_ring, m, cap, codes, e8m0, stream),
 * bit for bit: the two appends touch disjoint buffers and run as the two
 * halves of one grid with the same code.  Arguments, layouts, ownership and
 * preconditions as in those two calls (the indexer keys have their own
 * logits zi_new [B], ring ki_ring [B, 2*Li_ring, d], zi_ring [B, 2*Li_ring]).
 * Limits: d = 128; m < 32; m <= L_ring, Li_ring; B * 2 * max(L_ring,
 * Li_ring) < 2^31.  Errors as those calls; nothing is enqueued on an
 * argument error.
 * ------------------------------------------------------------------- */
csa_status_t csa_decode_append(const void* k_new, const void* v_new, const float* z_new,
                               const void* ki_new, const float* zi_new, int32_t io_dtype,
                               const int32_t* pos, int32_t B, int32_t d, int32_t m, int32_t cap,
                               int32_t L_ring, void* k_ring, void* v_ring, float* z_ring,
                               int32_t ckv_dtype, void* ck, void* cv, float* ck_scale,
                               float* cv_scale, int32_t* raw_pos0, int32_t Li_ring, void* ki_ring,
                               float* zi_ring, uint8_t* codes, uint8_t* e8m0, void* stream);

/* Workspace bytes a call needs.  n_keys = k + W (CSA) or cap + W (HCA);
 * for CSA_OP_TOPK and CSA_OP_INDEXER_TOPK pass T_q and n_keys = cap (and, for
 * CSA_OP_INDEXER_TOPK, d = d_I).  Returns 0 when none is needed and
 * (size_t)-1 for invalid arguments. */
size_t csa_workspace_size(int32_t op, int32_t B, int32_t T_q, int32_t H, int32_t d,
                          int32_t n_keys);

/* Static text for a status code. */
const char* csa_status_str(int32_t status);

/* ABI version (major*100 + minor). */
int32_t csa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
