"""Python binding of libcsa (CSA / HCA compressed attention for MI355X, gfx950).

Argument marshalling only: every step runs in the HIP kernels of libcsa.so,
called through its C ABI (include/csa.h).  torch provides device memory and
the current stream.  There is no fallback: if the library is not built or no
GPU is present, the calls raise.

Tensor conventions
  bf16   torch.bfloat16 (or int16/uint16 holding the bit patterns)
  f32    torch.float32
  fp8    torch.uint8 / torch.float8_e4m3fn holding OCP E4M3FN codes
  MXFP4  torch.uint8: packed E2M1 codes (low nibble first) and E8M0 scales
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa.so")

CSA_OK, CSA_EINVAL, CSA_ENOTSUP, CSA_EHIP, CSA_EWORKSPACE, CSA_ESCRATCH = range(6)
CSA_BF16, CSA_F32, CSA_FP8_E4M3 = 0, 1, 2
CSA_OP_TOPK, CSA_OP_SPARSE_ATTN, CSA_OP_DENSE_ATTN, CSA_OP_INDEXER_TOPK = 0, 1, 2, 3
CSA_OP_SPARSE_ATTN_BATCH_INVARIANT, CSA_OP_DENSE_ATTN_BATCH_INVARIANT = 4, 5
CSA_OP_KV_CACHE_APPEND, CSA_OP_INDEXER_TOPK_VARLEN = 6, 7
CSA_OP_SPARSE_ATTN_VARLEN, CSA_OP_DENSE_ATTN_VARLEN = 8, 9
DTYPES = {"bf16": CSA_BF16, "f32": CSA_F32, "fp8": CSA_FP8_E4M3}

EXPORTS = ["csa_compress_kv", "csa_mxfp4_quantize", "csa_indexer_scores", "csa_indexer_topk",
           "csa_compress_indexer_topk", "csa_topk", "csa_sparse_attn", "hca_dense_attn",
           "csa_sparse_attn_batch_invariant", "hca_dense_attn_batch_invariant", "csa_kv_cache_append",
           "csa_mxfp4_quantize_appended", "csa_sparse_attn_varlen", "hca_dense_attn_varlen",
           "csa_indexer_key_append", "csa_sparse_attn_noalloc", "csa_compress_kv_varlen",
           "csa_indexer_topk_varlen", "csa_decode_append", "csa_workspace_size",
           "csa_status_str", "csa_abi_version"]

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t


class CsaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


def load(path=LIB_PATH):
    """Load libcsa.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m long_context_compressed_03_amd.build`")
    lib = ctypes.CDLL(path)
    lib.csa_compress_kv.argtypes = [_P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P]
    lib.csa_mxfp4_quantize.argtypes = [_P, _I, ctypes.c_int64, _I, _P, _P, _P]
    lib.csa_indexer_scores.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]
    lib.csa_indexer_topk.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _S,
                                     _P]
    lib.csa_compress_indexer_topk.argtypes = [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _I, _I,
                                              _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P,
                                              _P, _S, _P]
    lib.csa_topk.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _S, _P]
    for fn in ["csa_sparse_attn", "csa_sparse_attn_batch_invariant"]:
        getattr(lib, fn).argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _I,
                                     _I, _I, _I, _I, _F, _P, _P, _P, _S, _P]
    for fn in ["hca_dense_attn", "hca_dense_attn_batch_invariant"]:
        getattr(lib, fn).argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _I, _P, _I,
                                     _I, _I, _I, _I, _F, _P, _P, _P, _S, _P]
    lib.csa_kv_cache_append.argtypes = [_P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P,
                                        _P, _P, _P, _P, _S, _P]
    lib.csa_mxfp4_quantize_appended.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P]
    lib.csa_sparse_attn_varlen.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P,
                                           _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _S, _P]
    lib.hca_dense_attn_varlen.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P,
                                          _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _S, _P]
    lib.csa_indexer_key_append.argtypes = [_P, _P, _I, _P, _I, _I, _I, _P, _P, _I, _I, _P, _P, _P]
    lib.csa_decode_append.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P,
                                      _P, _P, _I, _P, _P, _P, _P, _P]
    lib.csa_sparse_attn_noalloc.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _I,
                                            _I, _I, _I, _I, _F, _P, _P, _P]
    lib.csa_compress_kv_varlen.argtypes = [_P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _I,
                                           _I, _P]
    lib.csa_indexer_topk_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                            _S, _P]
    for fn in ["csa_compress_kv_varlen", "csa_indexer_topk_varlen", "csa_indexer_key_append", "csa_sparse_attn_noalloc", "csa_sparse_attn_varlen", "hca_dense_attn_varlen",
               "csa_mxfp4_quantize_appended", "csa_kv_cache_append", "csa_compress_kv", "csa_mxfp4_quantize", "csa_indexer_scores", "csa_indexer_topk",
               "csa_compress_indexer_topk", "csa_topk", "csa_sparse_attn", "hca_dense_attn",
               "csa_sparse_attn_batch_invariant", "hca_dense_attn_batch_invariant"]:
        getattr(lib, fn).restype = _I
    lib.csa_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.csa_workspace_size.restype = _S
    lib.csa_status_str.argtypes = [_I]
    lib.csa_status_str.restype = ctypes.c_char_p
    lib.csa_abi_version.argtypes = []
    lib.csa_abi_version.restype = _I
    _lib = lib
    return lib


def status_str(status):
    return load().csa_status_str(int(status)).decode()


def _check(fn, status):
    if status != CSA_OK:
        raise CsaError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt_of(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return CSA_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------- calls --

def _compress_ptrs(k, v, logits, m, k_out, v_out, k_scale_out, v_scale_out, L, row0, entry0):
    """Pointer arguments of a compression call (rows row0.., entries entry0..)."""
    B, ld_in, d = k.shape
    ld_out = k_out.shape[1]
    L = ld_in - row0 if L is None else L
    if row0 < 0 or entry0 < 0 or row0 + L > ld_in or entry0 + L // max(m, 1) > ld_out:
        raise ValueError("row or entry range outside the buffers")

    def off(t, n):
        return None if t is None else ctypes.c_void_p(_ptr(t).value + n * t.element_size())
    return dict(B=B, L=L, ld_in=ld_in, d=d, ld_out=ld_out, in_dt=_dt_of(k), out_dt=_dt_of(k_out),
                k=off(k, row0 * d), v=off(v, row0 * d), logits=off(logits, row0),
                k_out=off(k_out, entry0 * d), v_out=off(v_out, entry0 * d),
                k_scale=off(k_scale_out, entry0), v_scale=off(v_scale_out, entry0))


def csa_compress_kv(k, v, logits, m, k_out, v_out, k_scale_out=None, v_scale_out=None, L=None,
                    row0=0, entry0=0, stream=None):
    """Pool every complete block of m rows of k/v [B, ld_in, 128] into k_out/v_out [B, ld_out, 128].

    Rows row0 .. row0+L-1 of each sequence are pooled into entries entry0 .. entry0+L/m-1
    (default: all ld_in rows into entries from 0).  Output storage type follows k_out's
    dtype (bf16, f32, or uint8 = fp8 with per-entry scales in k_scale_out/v_scale_out
    [B, ld_out]).
    """
    c = _compress_ptrs(k, v, logits, m, k_out, v_out, k_scale_out, v_scale_out, L, row0, entry0)
    st = load().csa_compress_kv(c["k"], c["v"], c["in_dt"], c["logits"], c["B"], c["L"], c["ld_in"], c["d"],
                                m, c["k_out"], c["v_out"], c["k_scale"], c["v_scale"], c["ld_out"],
                                c["out_dt"], _stream(stream))
    _check("csa_compress_kv", st)


def csa_compress_indexer_topk(k, v, logits, k_out, v_out, k_scale_out, v_scale_out, q_codes, q_e8m0, w,
                              k_codes, k_e8m0, q_pos0, m, k_sel, idx=None, L=None, row0=0, entry0=0,
                              stream=None):
    """csa_compress_kv(k, v, logits, m, k_out, ...) and csa_indexer_topk(q_codes, ..., m, k_sel) in one call.

    The compression's sequences are the indexer's (k.shape[0] == q_codes.shape[0]); returns idx.
    """
    B, T_q, H_I, half = q_codes.shape
    cap = k_codes.shape[1]
    c = _compress_ptrs(k, v, logits, m, k_out, v_out, k_scale_out, v_scale_out, L, row0, entry0)
    if c["B"] != B:
        raise ValueError("the compression and the indexer must cover the same sequences")
    if idx is None:
        idx = torch.empty((B, T_q, k_sel), dtype=torch.int32, device=q_codes.device)
    lib = load()
    ws = _workspace(q_codes.device, lib.csa_workspace_size(CSA_OP_INDEXER_TOPK, B, T_q, 0, 2 * half, cap))
    st = lib.csa_compress_indexer_topk(c["k"], c["v"], c["in_dt"], c["logits"], c["L"], c["ld_in"], c["d"],
                                       c["k_out"], c["v_out"], c["k_scale"], c["v_scale"], c["ld_out"],
                                       c["out_dt"], _ptr(q_codes), _ptr(q_e8m0), _ptr(w), _ptr(k_codes),
                                       _ptr(k_e8m0), _ptr(q_pos0), B, T_q, H_I, 2 * half, cap, m, k_sel,
                                       _ptr(idx), _ws_ptr(ws), _ws_len(ws), _stream(stream))
    _check("csa_compress_indexer_topk", st)
    return idx


def csa_mxfp4_quantize(x, codes=None, e8m0=None, stream=None):
    """Real vectors x [..., d] (bf16 or fp32, d a multiple of 32) -> MXFP4 (codes [..., d/2] u8,
    e8m0 [..., d/32] u8), the layout the indexer calls take."""
    d = x.shape[-1]
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (d // 2,), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty(lead + (d // 32,), dtype=torch.uint8, device=x.device)
    if not x.is_contiguous() or not codes.is_contiguous() or not e8m0.is_contiguous():
        raise ValueError("contiguous tensors expected")
    n_vec = x.numel() // d if d else 0
    st = load().csa_mxfp4_quantize(_ptr(x), _dt_of(x), n_vec, d, _ptr(codes), _ptr(e8m0), _stream(stream))
    _check("csa_mxfp4_quantize", st)
    return codes, e8m0


def csa_indexer_scores(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, m, scores=None, stream=None):
    """Indexer scores [B, T_q, cap] fp32 for MXFP4 queries [B,T_q,H_I,d_I/2] and keys [B,cap,d_I/2]."""
    B, T_q, H_I, half = q_codes.shape
    cap = k_codes.shape[1]
    if scores is None:
        scores = torch.empty((B, T_q, cap), dtype=torch.float32, device=q_codes.device)
    st = load().csa_indexer_scores(_ptr(q_codes), _ptr(q_e8m0), _ptr(w), _ptr(k_codes),
                                   _ptr(k_e8m0), _ptr(q_pos0), B, T_q, H_I, 2 * half, cap, m,
                                   _ptr(scores), _stream(stream))
    _check("csa_indexer_scores", st)
    return scores


def csa_topk(scores, q_pos0, m, k, idx=None, stream=None):
    """Top-k visible entries per query row: idx [B, T_q, k] int32, ascending, -1 padded."""
    B, T_q, cap = scores.shape
    if idx is None:
        idx = torch.empty((B, T_q, k), dtype=torch.int32, device=scores.device)
    ws = _workspace(scores.device, load().csa_workspace_size(CSA_OP_TOPK, B, T_q, 0, 128, cap))
    st = load().csa_topk(_ptr(scores), _ptr(q_pos0), B, T_q, cap, m, k, _ptr(idx), _ws_ptr(ws),
                         _ws_len(ws), _stream(stream))
    _check("csa_topk", st)
    return idx


def csa_indexer_topk(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, m, k, idx=None, stream=None):
    """Fused indexer + top-k: idx [B, T_q, k] int32, identical to csa_topk(csa_indexer_scores(...))."""
    B, T_q, H_I, half = q_codes.shape
    cap = k_codes.shape[1]
    if idx is None:
        idx = torch.empty((B, T_q, k), dtype=torch.int32, device=q_codes.device)
    lib = load()
    ws = _workspace(q_codes.device, lib.csa_workspace_size(CSA_OP_INDEXER_TOPK, B, T_q, 0, 2 * half, cap))
    st = lib.csa_indexer_topk(_ptr(q_codes), _ptr(q_e8m0), _ptr(w), _ptr(k_codes), _ptr(k_e8m0),
                              _ptr(q_pos0), B, T_q, H_I, 2 * half, cap, m, k, _ptr(idx), _ws_ptr(ws),
                              _ws_len(ws), _stream(stream))
    _check("csa_indexer_topk", st)
    return idx


def csa_indexer_topk_varlen(q_codes, q_e8m0, w, k_codes, k_e8m0, cu_rows, q_pos0, m, k, idx=None,
                            stream=None):
    """Indexer top-k over packed query rows of B sequences: q_codes [n_rows, H_I, d_I/2],
    k_codes [B, cap, d_I/2], cu_rows [B+1] (sequence b owns rows cu_rows[b] ..
    cu_rows[b+1]-1, at positions q_pos0[b], q_pos0[b]+1, ...).  idx [n_rows, k] int32."""
    n_rows, H_I, half = q_codes.shape
    B, cap = k_codes.shape[0], k_codes.shape[1]
    if cu_rows.numel() != B + 1 or q_pos0.numel() != B:
        raise ValueError("cu_rows holds B + 1 offsets and q_pos0 B positions")
    if idx is None:
        idx = torch.empty((n_rows, k), dtype=torch.int32, device=q_codes.device)
    lib = load()
    ws = _workspace(q_codes.device, lib.csa_workspace_size(CSA_OP_INDEXER_TOPK_VARLEN, n_rows, 0, 0, 0, cap))
    st = lib.csa_indexer_topk_varlen(_ptr(q_codes), _ptr(q_e8m0), _ptr(w), _ptr(k_codes), _ptr(k_e8m0),
                                     _ptr(cu_rows), _ptr(q_pos0), B, n_rows, H_I, 2 * half, cap, m, k, _ptr(idx),
                                     _ws_ptr(ws), _ws_len(ws), _stream(stream))
    _check("csa_indexer_topk_varlen", st)
    return idx


def csa_compress_kv_varlen(k, v, logits, m, k_out, v_out, cu_entries, row0, entry0, n_entries,
                           k_scale_out=None, v_scale_out=None, stream=None):
    """New entries of B sequences in one launch: k, v [B, ld_in, 128], logits [B, ld_in];
    sequence b's j-th new entry (j < cu_entries[b+1] - cu_entries[b]) pools rows
    row0[b] + j*m .. into entry entry0[b] + j of k_out, v_out [B, ld_out, 128]."""
    B, ld_in, d = k.shape
    if cu_entries.numel() != B + 1 or row0.numel() != B or entry0.numel() != B:
        raise ValueError("cu_entries holds B + 1 offsets, row0 and entry0 B values")
    st = load().csa_compress_kv_varlen(_ptr(k), _ptr(v), _dt_of(k), _ptr(logits), B, ld_in, d, m, _ptr(cu_entries),
                                       _ptr(row0), _ptr(entry0), int(n_entries), _ptr(k_out), _ptr(v_out),
                                       _ptr(k_scale_out), _ptr(v_scale_out), k_out.shape[1], _dt_of(k_out),
                                       _stream(stream))
    _check("csa_compress_kv_varlen", st)


_WS = {}


def _workspace(device, nbytes):
    """Scratch for split partial results, cached per device and grown on demand."""
    if nbytes == ctypes.c_size_t(-1).value:
        raise CsaError("csa_workspace_size", CSA_EINVAL)
    if nbytes == 0:
        return None
    key = (device.type, device.index)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def _ws_ptr(ws):
    return None if ws is None else ctypes.c_void_p(ws.data_ptr())


def _ws_len(ws):
    return 0 if ws is None else ws.numel()


def _attn_common(q, ck, ck_scale, out, lse):
    B, T_q, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    return B, T_q, H, d, out


def csa_sparse_attn(q, ck, cv, idx, k_win, v_win, raw_pos0, q_pos0, W, ck_scale=None,
                    cv_scale=None, sm_scale=None, out=None, lse=None, stream=None,
                    batch_invariant=False):
    """CSA attention over idx-selected compressed entries plus window(t).

    batch_invariant=True calls csa_sparse_attn_batch_invariant: a row's bits then
    do not depend on the batch around it."""
    B, T_q, H, d, out = _attn_common(q, ck, ck_scale, out, lse)
    k = idx.shape[-1]
    cap = ck.shape[1]
    sm = d ** -0.5 if sm_scale is None else sm_scale
    lib = load()
    name = "csa_sparse_attn_batch_invariant" if batch_invariant else "csa_sparse_attn"
    op = CSA_OP_SPARSE_ATTN_BATCH_INVARIANT if batch_invariant else CSA_OP_SPARSE_ATTN
    ws = _workspace(q.device, lib.csa_workspace_size(op, B, T_q, H, d, k + W))
    st = getattr(lib, name)(_ptr(q), _dt_of(q), _ptr(ck), _ptr(cv), _ptr(ck_scale),
                             _ptr(cv_scale), _dt_of(ck), cap, _ptr(idx), k, _ptr(k_win),
                             _ptr(v_win), _ptr(raw_pos0), k_win.shape[1], _ptr(q_pos0), W, B,
                             T_q, H, d, sm, _ptr(out), _ptr(lse), _ws_ptr(ws), _ws_len(ws),
                             _stream(stream))
    _check(name, st)
    return out


def csa_sparse_attn_noalloc(q, ck, cv, idx, k_win, v_win, raw_pos0, q_pos0, W, out, ck_scale=None,
                            cv_scale=None, sm_scale=None, lse=None, stream=None):
    """csa_sparse_attn for callers that cannot allocate: the caller passes `out` (and `lse`), and
    the split partials go to the library's fixed per-GPU scratch.  Calls that may overlap on one
    GPU must not be issued (they share that scratch)."""
    B, T_q, H, d = q.shape
    k = idx.shape[-1]
    sm = d ** -0.5 if sm_scale is None else sm_scale
    st = load().csa_sparse_attn_noalloc(_ptr(q), _dt_of(q), _ptr(ck), _ptr(cv), _ptr(ck_scale), _ptr(cv_scale),
                                        _dt_of(ck), ck.shape[1], _ptr(idx), k, _ptr(k_win), _ptr(v_win),
                                        _ptr(raw_pos0), k_win.shape[1], _ptr(q_pos0), W, B, T_q, H, d, sm,
                                        _ptr(out), _ptr(lse), _stream(stream))
    _check("csa_sparse_attn_noalloc", st)
    return out


def hca_dense_attn(q, ck, cv, m_prime, k_win, v_win, raw_pos0, q_pos0, W, ck_scale=None,
                   cv_scale=None, sm_scale=None, out=None, lse=None, stream=None,
                   batch_invariant=False):
    """HCA attention over all visible compressed entries plus window(t).

    batch_invariant=True calls hca_dense_attn_batch_invariant."""
    B, T_q, H, d, out = _attn_common(q, ck, ck_scale, out, lse)
    cap = ck.shape[1]
    sm = d ** -0.5 if sm_scale is None else sm_scale
    lib = load()
    name = "hca_dense_attn_batch_invariant" if batch_invariant else "hca_dense_attn"
    op = CSA_OP_DENSE_ATTN_BATCH_INVARIANT if batch_invariant else CSA_OP_DENSE_ATTN
    ws = _workspace(q.device, lib.csa_workspace_size(op, B, T_q, H, d, cap + W))
    st = getattr(lib, name)(_ptr(q), _dt_of(q), _ptr(ck), _ptr(cv), _ptr(ck_scale),
                            _ptr(cv_scale), _dt_of(ck), cap, m_prime, _ptr(k_win), _ptr(v_win),
                            _ptr(raw_pos0), k_win.shape[1], _ptr(q_pos0), W, B, T_q, H, d, sm,
                            _ptr(out), _ptr(lse), _ws_ptr(ws), _ws_len(ws), _stream(stream))
    _check(name, st)
    return out


def csa_sparse_attn_batch_invariant(*args, **kwargs):
    """csa_sparse_attn whose row results do not depend on the batch around them."""
    return csa_sparse_attn(*args, batch_invariant=True, **kwargs)


def hca_dense_attn_batch_invariant(*args, **kwargs):
    """hca_dense_attn whose row results do not depend on the batch around them."""
    return hca_dense_attn(*args, batch_invariant=True, **kwargs)


def csa_kv_cache_append(k_new, v_new, z_new, pos, k_ring, v_ring, z_ring, m, ck, cv, ck_scale=None,
                        cv_scale=None, raw_pos0=None, stream=None):
    """Append one token per sequence (k_new, v_new [B, d]; z_new [B]; pos [B] int32, < 0 = idle)
    to a ring (k_ring, v_ring [B, 2L, d]; z_ring [B, 2L]) and, when a block of m completes,
    its pooled entry to the compressed cache ck, cv [B, cap, d].  Returns raw_pos0 [B] int32:
    the window base for the attention calls over the ring (L_raw = 2L)."""
    B, d = k_new.shape
    L2 = k_ring.shape[1]
    if L2 % 2:
        raise ValueError("the ring holds 2 * L_ring rows per sequence")
    if raw_pos0 is None:
        raw_pos0 = torch.empty(B, dtype=torch.int32, device=k_new.device)
    lib = load()
    ws = _workspace(k_new.device, lib.csa_workspace_size(CSA_OP_KV_CACHE_APPEND, B, 0, 0, 0, 0))
    st = lib.csa_kv_cache_append(_ptr(k_new), _ptr(v_new), _ptr(z_new), _dt_of(k_new), _ptr(pos), B, d,
                                 L2 // 2, _ptr(k_ring), _ptr(v_ring), _ptr(z_ring), m, ck.shape[1],
                                 _dt_of(ck), _ptr(ck), _ptr(cv), _ptr(ck_scale), _ptr(cv_scale),
                                 _ptr(raw_pos0), _ws_ptr(ws), _ws_len(ws), _stream(stream))
    _check("csa_kv_cache_append", st)
    return raw_pos0


def csa_mxfp4_quantize_appended(x, pos, m, codes, e8m0, stream=None):
    """MXFP4-convert, for each sequence whose token at pos completes a block of m, the
    entry it completes: x [B, cap, d] (bf16 or f32) into codes [B, cap, d/2] and
    e8m0 [B, cap, d/32] (uint8), bit-identical to csa_mxfp4_quantize."""
    B, cap, d = x.shape
    st = load().csa_mxfp4_quantize_appended(_ptr(x), _dt_of(x), _ptr(pos), B, cap, m, d, _ptr(codes),
                                            _ptr(e8m0), _stream(stream))
    _check("csa_mxfp4_quantize_appended", st)


def _varlen(name, op, q, ck, cv, mid, n_keys, k_win, v_win, raw_pos0, cu_rows, q_pos0, W, ck_scale,
            cv_scale, sm_scale, invariant, out, lse, stream):
    n_rows, H, d = q.shape
    B, cap = ck.shape[0], ck.shape[1]
    if cu_rows.numel() != B + 1 or q_pos0.numel() != B:
        raise ValueError("cu_rows holds B + 1 offsets and q_pos0 B positions (B = ck.shape[0])")
    if out is None:
        out = torch.empty_like(q)
    sm = d ** -0.5 if sm_scale is None else sm_scale
    lib = load()
    ws = _workspace(q.device, lib.csa_workspace_size(op, n_rows, B, H, d, n_keys))
    st = getattr(lib, name)(_ptr(q), _dt_of(q), _ptr(ck), _ptr(cv), _ptr(ck_scale), _ptr(cv_scale),
                            _dt_of(ck), cap, *mid, _ptr(k_win), _ptr(v_win), _ptr(raw_pos0),
                            k_win.shape[1], _ptr(cu_rows), _ptr(q_pos0), n_rows, W, B, H, d, sm,
                            int(bool(invariant)), _ptr(out), _ptr(lse), _ws_ptr(ws), _ws_len(ws), _stream(stream))
    _check(name, st)
    return out


def csa_sparse_attn_varlen(q, ck, cv, idx, k_win, v_win, raw_pos0, cu_rows, q_pos0, W, ck_scale=None,
                           cv_scale=None, sm_scale=None, invariant=True, out=None, lse=None, stream=None):
    """CSA attention over the packed query rows of B sequences: q [n_rows, H, d], idx
    [n_rows, k]; sequence b owns rows cu_rows[b] .. cu_rows[b+1]-1 at positions q_pos0[b],
    q_pos0[b]+1, ...  invariant: each row's bits equal the batch-invariant call's on its own
    sequence; otherwise the plain calls' kernels for a call of n_rows rows."""
    k = idx.shape[-1]
    return _varlen("csa_sparse_attn_varlen", CSA_OP_SPARSE_ATTN_VARLEN, q, ck, cv, (_ptr(idx), k), k + W, k_win,
                   v_win, raw_pos0, cu_rows, q_pos0, W, ck_scale, cv_scale, sm_scale, invariant, out, lse, stream)


def hca_dense_attn_varlen(q, ck, cv, m_prime, k_win, v_win, raw_pos0, cu_rows, q_pos0, W, ck_scale=None,
                          cv_scale=None, sm_scale=None, invariant=True, out=None, lse=None, stream=None):
    """HCA attention over the packed query rows of B sequences (as csa_sparse_attn_varlen)."""
    return _varlen("hca_dense_attn_varlen", CSA_OP_DENSE_ATTN_VARLEN, q, ck, cv, (m_prime,), ck.shape[1] + W,
                   k_win, v_win, raw_pos0, cu_rows, q_pos0, W, ck_scale, cv_scale, sm_scale, invariant, out, lse,
                   stream)


def csa_decode_append(k_new, v_new, z_new, ki_new, zi_new, pos, k_ring, v_ring, z_ring, m, ck, cv,
                      ki_ring, zi_ring, codes, e8m0, ck_scale=None, cv_scale=None, raw_pos0=None, stream=None):
    """Both appends of a CSA layer's decode token in one launch: exactly csa_kv_cache_append
    (k_new, v_new, z_new into the K/V ring and cache ck, cv) followed by csa_indexer_key_append
    (ki_new, zi_new into the indexer ring ki_ring, zi_ring and the MXFP4 keys codes, e8m0).
    Returns raw_pos0 [B] int32."""
    B, d = k_new.shape
    L2, Li2 = k_ring.shape[1], ki_ring.shape[1]
    if L2 % 2 or Li2 % 2:
        raise ValueError("a ring holds 2 * L_ring rows per sequence")
    if raw_pos0 is None:
        raw_pos0 = torch.empty(B, dtype=torch.int32, device=k_new.device)
    st = load().csa_decode_append(_ptr(k_new), _ptr(v_new), _ptr(z_new), _ptr(ki_new), _ptr(zi_new),
                                  _dt_of(k_new), _ptr(pos), B, d, m, ck.shape[1], L2 // 2, _ptr(k_ring),
                                  _ptr(v_ring), _ptr(z_ring), _dt_of(ck), _ptr(ck), _ptr(cv), _ptr(ck_scale),
                                  _ptr(cv_scale), _ptr(raw_pos0), Li2 // 2, _ptr(ki_ring), _ptr(zi_ring),
                                  _ptr(codes), _ptr(e8m0), _stream(stream))
    _check("csa_decode_append", st)
    return raw_pos0


def csa_indexer_key_append(k_new, z_new, pos, k_ring, z_ring, m, codes, e8m0, stream=None):
    """Append one indexer key per sequence (k_new [B, d], z_new [B], pos [B]) to its ring
    (k_ring [B, 2L, d], z_ring [B, 2L]) and write the MXFP4 entry of a block it completes
    into codes [B, cap, d/2] and e8m0 [B, cap, d/32]."""
    B, d = k_new.shape
    L2 = k_ring.shape[1]
    if L2 % 2:
        raise ValueError("the ring holds 2 * L_ring rows per sequence")
    st = load().csa_indexer_key_append(_ptr(k_new), _ptr(z_new), _dt_of(k_new), _ptr(pos), B, d, L2 // 2,
                                       _ptr(k_ring), _ptr(z_ring), m, codes.shape[1], _ptr(codes), _ptr(e8m0),
                                       _stream(stream))
    _check("csa_indexer_key_append", st)
