"""Python binding of libdsa.so (include/dsa.h): argument marshalling only.

Every function takes torch tensors on the GPU, checks their dtype/shape/contiguity, and calls
the C entry point of the same name on the current HIP stream. All computation runs in the
library's kernels; there is no fallback of any kind: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_E4M3, DSA_F32, DSA_BF16 = 0, 1, 2
PATHS = {
    0: "none", 1: "indexer_generic", 2: "indexer_scan_mfma", 3: "indexer_prefill_mfma", 4: "indexer_topk_fused",
    10: "topk_copy", 11: "topk_radix", 12: "topk_radix_reg", 13: "topk_radix_staged", 20: "mla_generic", 21: "mla_mfma", 22: "mla_mfma_split",
    30: "mha_mfma", 31: "mha_mfma_masked", 40: "cache_write", 41: "quantize", 42: "project",
}

EXPORTS = [
    "dsa_status_string", "dsa_last_error", "dsa_last_path",
    "dsa_indexer_scores", "dsa_topk_workspace_size", "dsa_topk",
    "dsa_indexer_topk_workspace_size", "dsa_indexer_topk",
    "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
    "dsa_sparse_mla_decode_noalloc",
    "dsa_dense_mla_workspace_size", "dsa_dense_mla_prefill",
    "dsa_expanded_mha_workspace_size", "dsa_expanded_mha_prefill",
    "dsa_indexer_cache_write", "dsa_latent_cache_write", "dsa_e4m3_quantize",
    "dsa_indexer_key_project", "dsa_indexer_query_project", "dsa_indexer_projection_workspace_size",
]


class DSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libdsa.so (raises if it has not been built) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() or "
                           "python -m sparse_attention_06_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_status_string.argtypes = [i32]
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_path.restype = i32
    lib.dsa_last_path.argtypes = []
    lib.dsa_indexer_scores.restype = i32
    lib.dsa_indexer_scores.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       vp, i64, vp]
    lib.dsa_topk_workspace_size.restype = sz
    lib.dsa_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_topk.restype = i32
    lib.dsa_topk.argtypes = [vp, i64, vp, i32, i32, i32, vp, i64, vp, sz, vp]
    lib.dsa_indexer_topk_workspace_size.restype = sz
    lib.dsa_indexer_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_indexer_topk.restype = i32
    lib.dsa_indexer_topk.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     vp, i64, i32, vp, i64, vp, sz, vp]
    lib.dsa_sparse_mla_workspace_size.restype = sz
    lib.dsa_sparse_mla_workspace_size.argtypes = [i32, i32, i32, i32]
    attn = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp,
            sz, vp]
    lib.dsa_sparse_mla_decode.restype = i32
    lib.dsa_sparse_mla_decode.argtypes = attn
    lib.dsa_sparse_mla_prefill.restype = i32
    lib.dsa_sparse_mla_prefill.argtypes = attn
    lib.dsa_sparse_mla_decode_noalloc.restype = i32
    lib.dsa_sparse_mla_decode_noalloc.argtypes = attn[:-3] + [vp]
    lib.dsa_dense_mla_workspace_size.restype = sz
    lib.dsa_dense_mla_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_dense_mla_prefill.restype = i32
    lib.dsa_dense_mla_prefill.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                          i32, f32, vp, vp, vp, sz, vp]
    lib.dsa_expanded_mha_workspace_size.restype = sz
    lib.dsa_expanded_mha_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_expanded_mha_prefill.restype = i32
    lib.dsa_expanded_mha_prefill.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, i64, i32, i32, i32, i32, i32,
                                             f32, vp, vp, vp, sz, vp]
    lib.dsa_indexer_cache_write.restype = i32
    lib.dsa_indexer_cache_write.argtypes = [vp, i32, i32, i32, vp, vp, i32, vp, i64, i32, i32, vp, vp, vp]
    lib.dsa_latent_cache_write.restype = i32
    lib.dsa_latent_cache_write.argtypes = [vp, i32, i32, vp, vp, i32, vp, i64, i32, i32, vp, vp]
    lib.dsa_e4m3_quantize.restype = i32
    lib.dsa_e4m3_quantize.argtypes = [vp, i64, vp, vp]
    lib.dsa_indexer_key_project.restype = i32
    lib.dsa_indexer_key_project.argtypes = [vp, vp, i32, i32, i32, vp, vp, i32, vp, i64, i32, i32, vp, vp, vp, sz,
                                            vp]
    lib.dsa_indexer_query_project.restype = i32
    lib.dsa_indexer_query_project.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.dsa_indexer_projection_workspace_size.restype = sz
    lib.dsa_indexer_projection_workspace_size.argtypes = [i32, i32]
    _lib = lib
    return lib


def last_path() -> str:
    return PATHS.get(load().dsa_last_path(), "unknown")


def _check(fn, status):
    if status != DSA_OK:
        lib = load()
        raise DSAError(fn, lib.dsa_status_string(status).decode(), lib.dsa_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, dim=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims (got {t.dim()})")


def _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq):
    """The query-row descriptor: rows = n_seq * q_per_seq in groups per sequence (q_seq None), or
    row r of sequence q_seq[r] (q_per_seq must then be 1)."""
    _need(q_pos, "q_pos", torch.int32, 1)
    if q_pos.numel() != rows:
        raise ValueError(f"q_pos has {q_pos.numel()} entries for {rows} rows")
    if q_seq is None:
        if rows != n_seq * q_per_seq:
            raise ValueError("rows must equal n_seq * q_per_seq (or pass q_seq)")
    else:
        _need(q_seq, "q_seq", torch.int32, 1)
        if q_seq.numel() != rows or q_per_seq != 1:
            raise ValueError("q_seq needs one entry per row and q_per_seq = 1")


def indexer_scores(q, w, k_cache, k_scale, page_table, q_pos, n_seq, q_per_seq, max_ctx, scores=None,
                   stream=None, q_seq=None):
    """q [rows, Hi, Di] uint8 (E4M3 bytes) or float32; w [rows, Hi] f32; k_cache [P, page, Di];
    k_scale [P, page] f32 or None; page_table [n_seq, ld_pt] i32; q_pos [rows] i32.
    Returns scores [rows, max_ctx] f32 (entries j > q_pos[r] are -inf or unspecified)."""
    dtype = DSA_E4M3 if q.dtype == torch.uint8 else DSA_F32
    _need(q, "q", q.dtype, 3)
    _need(k_cache, "k_cache", q.dtype, 3)
    _need(w, "w", torch.float32, 2)
    _need(page_table, "page_table", torch.int32, 2)
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32)
    rows, Hi, Di = q.shape
    _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq)
    if scores is None:
        scores = torch.empty(rows, max_ctx, dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, 2)
    st = load().dsa_indexer_scores(_p(q), _p(w), _p(k_cache), _p(k_scale), _p(page_table), page_table.shape[1],
                                   k_cache.shape[1], k_cache.shape[0], _p(q_seq), _p(q_pos), rows, n_seq, q_per_seq,
                                   max_ctx, Hi, Di, dtype, _p(scores), scores.shape[1], _stream(stream))
    _check("dsa_indexer_scores", st)
    return scores


def topk_workspace_size(rows, max_ctx, k) -> int:
    return int(load().dsa_topk_workspace_size(rows, max_ctx, k))


def topk(scores, q_pos, max_ctx, k, idx=None, ws=None, stream=None):
    """Top-k positions per row, ascending, -1 padded: idx [rows, k] int32. `ws` (uint8, at least
    topk_workspace_size bytes) is allocated here when needed and not given."""
    _need(scores, "scores", torch.float32, 2)
    _need(q_pos, "q_pos", torch.int32, 1)
    rows = scores.shape[0]
    if idx is None:
        idx = torch.empty(rows, k, dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, 2)
    need = topk_workspace_size(rows, max_ctx, k) if rows > 0 else 0
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    st = load().dsa_topk(_p(scores), scores.shape[1], _p(q_pos), rows, max_ctx, k, _p(idx), idx.shape[1], _p(ws),
                         0 if ws is None else ws.numel(), _stream(stream))
    _check("dsa_topk", st)
    return idx


def indexer_topk_workspace_size(rows, max_ctx, k) -> int:
    return int(load().dsa_indexer_topk_workspace_size(rows, max_ctx, k))


def indexer_topk(q, w, k_cache, k_scale, page_table, q_pos, n_seq, q_per_seq, max_ctx, k, scores=None, idx=None,
                 ws=None, stream=None, q_seq=None):
    """indexer_scores then topk in one call (the top-k's first radix pass counted during the scan).
    `ws` (uint8, at least indexer_topk_workspace_size bytes) must be zero-filled before its first
    use and is left so by every successful call; a zeroed one is allocated here when not given.
    Returns (scores, idx)."""
    dtype = DSA_E4M3 if q.dtype == torch.uint8 else DSA_F32
    _need(q, "q", q.dtype, 3)
    _need(k_cache, "k_cache", q.dtype, 3)
    _need(w, "w", torch.float32, 2)
    _need(page_table, "page_table", torch.int32, 2)
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32)
    rows, Hi, Di = q.shape
    _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq)
    if scores is None:
        scores = torch.empty(rows, max_ctx, dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, 2)
    if idx is None:
        idx = torch.empty(rows, k, dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32, 2)
    if ws is None and rows > 0:
        ws = torch.zeros(indexer_topk_workspace_size(rows, max_ctx, k), dtype=torch.uint8, device=q.device)
    st = load().dsa_indexer_topk(_p(q), _p(w), _p(k_cache), _p(k_scale), _p(page_table), page_table.shape[1],
                                 k_cache.shape[1], k_cache.shape[0], _p(q_seq), _p(q_pos), rows, n_seq, q_per_seq,
                                 max_ctx, Hi, Di, dtype, _p(scores), scores.shape[1], k, _p(idx), idx.shape[1], _p(ws),
                                 0 if ws is None else ws.numel(), _stream(stream))
    _check("dsa_indexer_topk", st)
    return scores, idx


def sparse_mla_workspace_size(rows, H, Dv, k) -> int:
    return int(load().dsa_sparse_mla_workspace_size(rows, H, Dv, k))


def _attn_common(q, kv_cache, page_table, q_pos, out, lse, Dv):
    _need(q, "q", torch.uint16 if q.dtype == torch.uint16 else torch.bfloat16, 3)
    _need(kv_cache, "kv_cache", kv_cache.dtype, 3)
    if kv_cache.dtype not in (torch.bfloat16, torch.uint16):
        raise ValueError("kv_cache must be bf16 (or its uint16 bits)")
    _need(page_table, "page_table", torch.int32, 2)
    _need(q_pos, "q_pos", torch.int32, 1)
    rows, H, _ = q.shape
    if out is None:
        out = torch.empty(rows, H, Dv, dtype=torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.uint16):
        raise ValueError("out must be bf16")
    _need(out, "out", out.dtype, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    return out


def _sparse(fn_name, q, kv_cache, page_table, q_pos, n_seq, q_per_seq, idx, Dqk, Dv, v_col0, sm_scale,
            out=None, lse=None, ws=None, stream=None, q_seq=None):
    out = _attn_common(q, kv_cache, page_table, q_pos, out, lse, Dv)
    _need(idx, "idx", torch.int32, 2)
    rows, H, _ = q.shape
    _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq)
    k = idx.shape[1]
    lib = load()
    need = lib.dsa_sparse_mla_workspace_size(rows, H, Dv, k) if fn_name == "dsa_sparse_mla_decode" else 0
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    fn = getattr(lib, fn_name)
    st = fn(_p(q), _p(kv_cache), _p(page_table), page_table.shape[1], kv_cache.shape[1], kv_cache.shape[0],
            _p(q_seq), _p(q_pos), rows, n_seq, q_per_seq, _p(idx), idx.shape[1], k, H, Dqk, Dv, kv_cache.shape[2], v_col0,
            float(sm_scale), _p(out), _p(lse), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
            _stream(stream))
    _check(fn_name, st)
    return out


def sparse_mla_decode(*args, **kw):
    return _sparse("dsa_sparse_mla_decode", *args, **kw)


def sparse_mla_prefill(*args, **kw):
    return _sparse("dsa_sparse_mla_prefill", *args, **kw)


def sparse_mla_decode_noalloc(q, kv_cache, page_table, q_pos, n_seq, q_per_seq, idx, Dqk, Dv, v_col0, sm_scale,
                              out, lse=None, stream=None, q_seq=None):
    """dsa_sparse_mla_decode without a workspace argument: the library's own device scratch is
    used, and nothing is allocated here either (out, and lse if wanted, are the caller's)."""
    if out is None:
        raise ValueError("sparse_mla_decode_noalloc needs the caller's out tensor")
    _attn_common(q, kv_cache, page_table, q_pos, out, lse, Dv)
    _need(idx, "idx", torch.int32, 2)
    rows, H, _ = q.shape
    _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq)
    st = load().dsa_sparse_mla_decode_noalloc(
        _p(q), _p(kv_cache), _p(page_table), page_table.shape[1], kv_cache.shape[1], kv_cache.shape[0], _p(q_seq),
        _p(q_pos), rows, n_seq, q_per_seq, _p(idx), idx.shape[1], idx.shape[1], H, Dqk, Dv, kv_cache.shape[2], v_col0,
        float(sm_scale), _p(out), _p(lse), _stream(stream))
    _check("dsa_sparse_mla_decode_noalloc", st)
    return out


def dense_mla_prefill(q, kv_cache, page_table, q_pos, n_seq, q_per_seq, max_ctx, Dqk, Dv, v_col0, sm_scale,
                      out=None, lse=None, stream=None, q_seq=None):
    out = _attn_common(q, kv_cache, page_table, q_pos, out, lse, Dv)
    rows, H, _ = q.shape
    _check_rows(rows, q_pos, n_seq, q_per_seq, q_seq)
    st = load().dsa_dense_mla_prefill(_p(q), _p(kv_cache), _p(page_table), page_table.shape[1], kv_cache.shape[1],
                                      kv_cache.shape[0], _p(q_seq), _p(q_pos), rows, n_seq, q_per_seq, max_ctx, H,
                                      Dqk, Dv,
                                      kv_cache.shape[2], v_col0, float(sm_scale), _p(out), _p(lse), None, 0,
                                      _stream(stream))
    _check("dsa_dense_mla_prefill", st)
    return out


def expanded_mha_workspace_size(rows, max_ctx, k) -> int:
    return int(load().dsa_expanded_mha_workspace_size(rows, max_ctx, k))


def expanded_mha_prefill(q, k_nope, k_rope, v, q_pos, n_seq, q_per_seq, sm_scale, idx=None, out=None, lse=None,
                         ws=None, stream=None):
    """Expanded multi-head attention (the dense fallback for short prefill), dense causal, or over
    the idx sets when idx is given (the masked MHA mode). q [rows, H, 192] bf16; k_nope
    [n_seq, H, max_ctx, 128] bf16; k_rope [n_seq, max_ctx, 64] bf16; v [n_seq, H, max_ctx, 128] bf16;
    q_pos [rows] i32; idx [rows, k] i32 or None. Returns out [rows, H, 128] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_nope, "k_nope", torch.bfloat16, 4)
    _need(k_rope, "k_rope", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 4)
    _need(q_pos, "q_pos", torch.int32, 1)
    rows, H, Dq = q.shape
    max_ctx = k_nope.shape[2]
    if (k_nope.shape[0] != n_seq or v.shape[0] != n_seq or k_rope.shape[0] != n_seq or k_nope.shape[1] != H
            or v.shape[1] != H or v.shape[2] != max_ctx or k_rope.shape[1] != max_ctx):
        raise ValueError("inconsistent expanded attention shapes")
    if rows != n_seq * q_per_seq or q_pos.numel() != rows:
        raise ValueError("rows must equal n_seq * q_per_seq")
    Dn, Dr, Dv = k_nope.shape[3], k_rope.shape[2], v.shape[3]
    if out is None:
        out = torch.empty(rows, H, Dv, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    k, ld_idx = 0, 0
    if idx is not None:
        _need(idx, "idx", torch.int32, 2)
        k, ld_idx = idx.shape[1], idx.shape[1]
        need = expanded_mha_workspace_size(rows, max_ctx, k)
        if ws is None and need:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = load().dsa_expanded_mha_prefill(_p(q), _p(k_nope), _p(k_rope), _p(v), max_ctx, _p(q_pos), n_seq, q_per_seq,
                                         _p(idx), ld_idx, k, H, Dn, Dr, Dv, float(sm_scale), _p(out), _p(lse),
                                         _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("dsa_expanded_mha_prefill", st)
    return out


def indexer_cache_write(k, seq, pos, page_table, k_cache, k_scale, stream=None):
    """Quantise indexer keys per token (s = max|k|/448, codes E4M3(k/s)) into the paged cache.
    k [n_tok, 128] float32 or bfloat16; seq, pos [n_tok] int32; page_table [n_seq, ld_pt] int32;
    k_cache [P, page, 128] uint8 and k_scale [P, page] float32, written in place."""
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("k must be float32 or bfloat16")
    _need(k, "k", k.dtype, 2)
    for t, n in ((seq, "seq"), (pos, "pos")):
        _need(t, n, torch.int32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(k_cache, "k_cache", torch.uint8, 3)
    _need(k_scale, "k_scale", torch.float32, 2)
    if seq.numel() != k.shape[0] or pos.numel() != k.shape[0]:
        raise ValueError("seq and pos need one entry per key row")
    st = load().dsa_indexer_cache_write(_p(k), DSA_F32 if k.dtype == torch.float32 else DSA_BF16, k.shape[0], k.shape[1],
                                        _p(seq), _p(pos), page_table.shape[0], _p(page_table), page_table.shape[1],
                                        k_cache.shape[1], k_cache.shape[0], _p(k_cache), _p(k_scale), _stream(stream))
    _check("dsa_indexer_cache_write", st)


def latent_cache_write(rows, seq, pos, page_table, kv_cache, stream=None):
    """Place latent rows [n_tok, kv_dim] bf16 into the paged cache [P, page, kv_dim] in place."""
    _need(rows, "rows", torch.bfloat16, 2)
    for t, n in ((seq, "seq"), (pos, "pos")):
        _need(t, n, torch.int32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    if kv_cache.shape[2] != rows.shape[1]:
        raise ValueError("rows and kv_cache widths differ")
    if seq.numel() != rows.shape[0] or pos.numel() != rows.shape[0]:
        raise ValueError("seq and pos need one entry per row")
    st = load().dsa_latent_cache_write(_p(rows), rows.shape[0], rows.shape[1], _p(seq), _p(pos), page_table.shape[0],
                                       _p(page_table), page_table.shape[1], kv_cache.shape[1], kv_cache.shape[0],
                                       _p(kv_cache), _stream(stream))
    _check("dsa_latent_cache_write", st)


def e4m3_quantize(x, out=None, stream=None):
    """float32 tensor -> E4M3 codes (uint8, same shape), no scale."""
    _need(x, "x", torch.float32)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _need(out, "out", torch.uint8)
    st = load().dsa_e4m3_quantize(_p(x), x.numel(), _p(out), _stream(stream))
    _check("dsa_e4m3_quantize", st)
    return out


def indexer_projection_workspace_size(rows, d) -> int:
    return int(load().dsa_indexer_projection_workspace_size(rows, d))


def _proj_ws(rows, d, ws, device):
    if ws is False:
        return None   # no workspace: the unsplit launch
    if ws is None:
        need = indexer_projection_workspace_size(rows, d)
        ws = torch.empty(need, dtype=torch.uint8, device=device) if need else None
    return ws


def indexer_key_project(h, w_k, seq, pos, page_table, k_cache, k_scale, ws=None, stream=None):
    """Keys k = h w_k^T (h [n_tok, d] bf16, w_k [128, d] bf16, the [out, in] layout of a linear
    layer), quantised per token into the paged key cache (k_cache [P, page, 128] uint8, k_scale
    [P, page] f32) at the tokens' (seq, pos) (int32 [n_tok]). ws: uint8 workspace (allocated here
    when None; False runs the unsplit launch)."""
    _need(h, "h", torch.bfloat16, 2)
    _need(w_k, "w_k", torch.bfloat16, 2)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(k_cache, "k_cache", torch.uint8, 3)
    _need(k_scale, "k_scale", torch.float32, 2)
    n_tok, d = h.shape
    if w_k.shape[1] != d or seq.numel() != n_tok or pos.numel() != n_tok:
        raise ValueError("inconsistent key projection shapes")
    ws = _proj_ws(n_tok, d, ws, h.device)
    st = load().dsa_indexer_key_project(_p(h), _p(w_k), n_tok, d, w_k.shape[0], _p(seq), _p(pos), page_table.shape[0],
                                        _p(page_table), page_table.shape[1], k_cache.shape[1], k_cache.shape[0],
                                        _p(k_cache), _p(k_scale), _p(ws), 0 if ws is None else ws.numel(),
                                        _stream(stream))
    _check("dsa_indexer_key_project", st)


def indexer_query_project(c_q, w_q, h, w_w, Hi, Di, q8=None, w=None, ws=None, stream=None):
    """Indexer queries q8 = E4M3(c_q w_q^T) [rows, Hi, Di] (uint8 codes, no scale) and head weights
    w = h w_w^T [rows, Hi] f32. c_q [rows, d_cq], w_q [Hi * Di, d_cq], h [rows, d], w_w [Hi, d], all
    bf16. Returns (q8, w)."""
    for t, name in ((c_q, "c_q"), (w_q, "w_q"), (h, "h"), (w_w, "w_w")):
        _need(t, name, torch.bfloat16, 2)
    rows, d_cq = c_q.shape
    d = h.shape[1]
    if h.shape[0] != rows or w_q.shape != (Hi * Di, d_cq) or w_w.shape != (Hi, d):
        raise ValueError("inconsistent query projection shapes")
    if q8 is None:
        q8 = torch.empty(rows, Hi, Di, dtype=torch.uint8, device=c_q.device)
    if w is None:
        w = torch.empty(rows, Hi, dtype=torch.float32, device=c_q.device)
    _need(q8, "q8", torch.uint8, 3)
    _need(w, "w", torch.float32, 2)
    ws = _proj_ws(rows, d, ws, c_q.device)
    st = load().dsa_indexer_query_project(_p(c_q), _p(w_q), _p(h), _p(w_w), rows, d_cq, d, Hi, Di, _p(q8), _p(w),
                                          _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check("dsa_indexer_query_project", st)
    return q8, w
