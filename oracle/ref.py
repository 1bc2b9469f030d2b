"""ctypes wrapper of the C oracle (``liboracle.so``), built with plain gcc.

TEST INFRASTRUCTURE ONLY (tests, smoke check, the benchmark's CPU baseline). Arrays are
numpy; every call can split rows over host threads (ctypes drops the GIL during a call).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3 = 0
F32 = 1
BF16 = 2

_lib = None
_lock = threading.Lock()


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, so every double operation is IEEE)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build_oracle(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_e4m3_to_double.restype = dbl
            lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
            lib.oracle_bf16_to_double.restype = dbl
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_indexer_scores.restype = i32
            lib.oracle_indexer_scores.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32,
                                                  i32, i32, i32, vp, i64, i32, i32]
            lib.oracle_topk.restype = i32
            lib.oracle_topk.argtypes = [vp, i64, vp, i32, i32, vp, i64, i32, i32]
            lib.oracle_sparse_mla.restype = i32
            lib.oracle_sparse_mla.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, vp, i64, i32,
                                              i32, i32, i32, i32, i32, dbl, vp, vp, i32, i32]
            lib.oracle_dense_mla.restype = i32
            lib.oracle_dense_mla.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, i32, dbl, vp, vp, i32, i32]
            lib.oracle_e4m3_from_float.restype = ctypes.c_uint8
            lib.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
            lib.oracle_e4m3_quantize.restype = i32
            lib.oracle_e4m3_quantize.argtypes = [vp, i64, vp]
            lib.oracle_indexer_cache_write.restype = i32
            lib.oracle_indexer_cache_write.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, i64, i32, i32, vp, vp, vp]
            lib.oracle_latent_cache_write.restype = i32
            lib.oracle_latent_cache_write.argtypes = [vp, i32, vp, vp, i32, i32, vp, i64, i32, i32, vp, vp]
            lib.oracle_indexer_key_project.restype = i32
            lib.oracle_indexer_key_project.argtypes = [vp, vp, i32, i32, i32, vp, vp, i32, vp, i64, i32, i32, vp,
                                                       vp, vp, vp]
            lib.oracle_indexer_query_project.restype = i32
            lib.oracle_indexer_query_project.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
            lib.oracle_mha.restype = i32
            lib.oracle_mha.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, vp, i64, i32, i32, i32, i32, i32,
                                       dbl, vp, vp, i32, i32]
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _run_rows(fn, rows, threads, row_subset=None):
    """Call fn(row_begin, row_end) over [0, rows) (or over the given sorted row subset)
    split across `threads` host threads; raise on a nonzero return code."""
    if row_subset is not None:
        spans = [(int(r), int(r) + 1) for r in row_subset]
    else:
        threads = max(1, min(threads, rows)) if rows > 0 else 1
        step = (rows + threads - 1) // threads if rows > 0 else 0
        spans = [(b, min(rows, b + step)) for b in range(0, rows, step)] if rows > 0 else []
    errors = []

    def work(chunk):
        for b, e in chunk:
            rc = fn(b, e)
            if rc != 0:
                errors.append(rc)

    n = max(1, min(threads, len(spans)))
    chunks = [spans[i::n] for i in range(n)]
    ts = [threading.Thread(target=work, args=(c,)) for c in chunks]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errors:
        raise ValueError(f"oracle call failed with code {errors[0]}")


def e4m3_to_double(code: int) -> float:
    return _load().oracle_e4m3_to_double(code)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _seq(q_seq, nrows):
    """The per-row sequence ids as a C array (None: rows in groups of q_per_seq per sequence)."""
    if q_seq is None:
        return None
    q_seq = _c(q_seq, np.int32)
    assert q_seq.shape == (nrows,)
    return q_seq


def indexer_scores(q, w, k_cache, k_scale, page_table, page_size, q_pos, n_seq, q_per_seq, fmt,
                   ld_scores, scores=None, threads=1, rows=None, q_seq=None):
    """Scores [rows, ld_scores] float32 (rows = q.shape[0]); entries j > q_pos[r] are left as given
    (NaN in a fresh array). `rows` optionally restricts the computed rows. q_seq: per-row
    sequence ids (q_per_seq must then be 1), or None for n_seq * q_per_seq rows in groups."""
    lib = _load()
    qdt = np.uint8 if fmt == E4M3 else np.float32
    q = _c(q, qdt)
    k_cache = _c(k_cache, qdt)
    w = _c(w, np.float32)
    pt = _c(page_table, np.int32)
    q_pos = _c(q_pos, np.int32)
    ks = None if k_scale is None else _c(k_scale, np.float32)
    nrows = q.shape[0]
    qs = _seq(q_seq, nrows)
    Hi, Di = q.shape[-2], q.shape[-1]
    num_pages = k_cache.shape[0]
    if scores is None:
        scores = np.full((nrows, ld_scores), np.nan, dtype=np.float32)

    def fn(b, e):
        return lib.oracle_indexer_scores(_ptr(q), _ptr(w), _ptr(k_cache), _ptr(ks), _ptr(pt), pt.shape[1],
                                         page_size, num_pages, _ptr(qs), _ptr(q_pos), nrows, n_seq, q_per_seq, Hi,
                                         Di, fmt, _ptr(scores), ld_scores, b, e)

    _run_rows(fn, nrows, threads, rows)
    return scores


def topk(scores, q_pos, k, threads=1, rows=None, idx=None):
    lib = _load()
    scores = _c(scores, np.float32)
    q_pos = _c(q_pos, np.int32)
    nrows = scores.shape[0]
    if idx is None:
        idx = np.full((nrows, k), -2, dtype=np.int32)

    def fn(b, e):
        return lib.oracle_topk(_ptr(scores), scores.shape[1], _ptr(q_pos), nrows, k, _ptr(idx), k, b, e)

    _run_rows(fn, nrows, threads, rows)
    return idx


def sparse_mla(q, kv_cache, page_table, page_size, q_pos, n_seq, q_per_seq, idx, Dqk, Dv, v_col0,
               sm_scale, threads=1, rows=None, with_lse=True, q_seq=None):
    """q: uint16 (bf16 bits) [rows, H, Dqk]; kv_cache: uint16 [P, page, kv_dim];
    returns (out float32 [rows, H, Dv], lse float32 [rows, H])."""
    lib = _load()
    q = _c(q, np.uint16)
    kv = _c(kv_cache, np.uint16)
    pt = _c(page_table, np.int32)
    q_pos = _c(q_pos, np.int32)
    idx = _c(idx, np.int32)
    nrows, H = q.shape[0], q.shape[1]
    qs = _seq(q_seq, nrows)
    kv_dim = kv.shape[-1]
    num_pages = kv.shape[0]
    out = np.full((nrows, H, Dv), np.nan, dtype=np.float32)
    lse = np.full((nrows, H), np.nan, dtype=np.float32) if with_lse else None

    def fn(b, e):
        return lib.oracle_sparse_mla(_ptr(q), _ptr(kv), _ptr(pt), pt.shape[1], page_size, num_pages,
                                     _ptr(qs), _ptr(q_pos), nrows, n_seq, q_per_seq, _ptr(idx), idx.shape[1],
                                     idx.shape[1],
                                     H, Dqk, Dv, kv_dim, v_col0, float(sm_scale), _ptr(out), _ptr(lse), b, e)

    _run_rows(fn, nrows, threads, rows)
    return out, lse


def dense_mla(q, kv_cache, page_table, page_size, q_pos, n_seq, q_per_seq, Dqk, Dv, v_col0, sm_scale,
              threads=1, rows=None, with_lse=True, q_seq=None):
    lib = _load()
    q = _c(q, np.uint16)
    kv = _c(kv_cache, np.uint16)
    pt = _c(page_table, np.int32)
    q_pos = _c(q_pos, np.int32)
    nrows, H = q.shape[0], q.shape[1]
    qs = _seq(q_seq, nrows)
    kv_dim = kv.shape[-1]
    num_pages = kv.shape[0]
    out = np.full((nrows, H, Dv), np.nan, dtype=np.float32)
    lse = np.full((nrows, H), np.nan, dtype=np.float32) if with_lse else None

    def fn(b, e):
        return lib.oracle_dense_mla(_ptr(q), _ptr(kv), _ptr(pt), pt.shape[1], page_size, num_pages,
                                    _ptr(qs), _ptr(q_pos), nrows, n_seq, q_per_seq, H, Dqk, Dv, kv_dim, v_col0,
                                    float(sm_scale), _ptr(out), _ptr(lse), b, e)

    _run_rows(fn, nrows, threads, rows)
    return out, lse


def mha(q, k_nope, k_rope, v, q_pos, n_seq, q_per_seq, idx, sm_scale, threads=1, rows=None, with_lse=True):
    """Expanded multi-head attention (the short-prefill fallback), dense causal when idx is None,
    else restricted to the idx entries (as a set). q: uint16 (bf16 bits) [rows, H, Dn+Dr];
    k_nope [n_seq, H, ld_kv, Dn]; k_rope [n_seq, ld_kv, Dr]; v [n_seq, H, ld_kv, Dv].
    Returns (out float32 [rows, H, Dv], lse float32 [rows, H])."""
    lib = _load()
    q = _c(q, np.uint16)
    kn = _c(k_nope, np.uint16)
    kr = _c(k_rope, np.uint16)
    v = _c(v, np.uint16)
    q_pos = _c(q_pos, np.int32)
    idx = None if idx is None else _c(idx, np.int32)
    nrows, H = q.shape[0], q.shape[1]
    Dn, Dr, Dv, ld_kv = kn.shape[3], kr.shape[2], v.shape[3], kn.shape[2]
    if q.shape[2] != Dn + Dr or kr.shape[1] != ld_kv or v.shape[2] != ld_kv or v.shape[1] != H or kn.shape[1] != H:
        raise ValueError("inconsistent expanded attention shapes")
    out = np.full((nrows, H, Dv), np.nan, dtype=np.float32)
    lse = np.full((nrows, H), np.nan, dtype=np.float32) if with_lse else None
    k = 0 if idx is None else idx.shape[1]

    def fn(b, e):
        return lib.oracle_mha(_ptr(q), _ptr(kn), _ptr(kr), _ptr(v), ld_kv, _ptr(q_pos), n_seq, q_per_seq,
                              _ptr(idx), k, k, H, Dn, Dr, Dv, float(sm_scale), _ptr(out), _ptr(lse), b, e)

    _run_rows(fn, nrows, threads, rows)
    return out, lse


def e4m3_from_float(x: float) -> int:
    return int(_load().oracle_e4m3_from_float(float(x)))


def e4m3_quantize(x):
    """float32 array -> E4M3 codes (uint8), no scale."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    if _load().oracle_e4m3_quantize(_ptr(x), x.size, _ptr(out)) != 0:
        raise ValueError("oracle call failed")
    return out


def indexer_cache_write(k, seq, pos, page_table, page_size, k_cache, k_scale):
    """k: float32 [n_tok, Di] or uint16 bf16 bits [n_tok, Di]; writes into k_cache (uint8
    [P, page, Di]) and k_scale (float32 [P, page]) in place; returns the skipped-token count."""
    fmt = F32 if k.dtype == np.float32 else BF16
    k = _c(k, np.float32 if fmt == F32 else np.uint16)
    seq, pos, pt = _c(seq, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    assert k_cache.flags.c_contiguous and k_scale.flags.c_contiguous
    skipped = ctypes.c_int(0)
    rc = _load().oracle_indexer_cache_write(_ptr(k), fmt, k.shape[1], _ptr(seq), _ptr(pos), k.shape[0], pt.shape[0], _ptr(pt),
                                            pt.shape[1], page_size, k_cache.shape[0], _ptr(k_cache), _ptr(k_scale),
                                            ctypes.byref(skipped))
    if rc != 0:
        raise ValueError(f"oracle call failed with code {rc}")
    return skipped.value


def latent_cache_write(rows, seq, pos, page_table, page_size, kv_cache):
    """rows: uint16 [n_tok, kv_dim]; writes into kv_cache (uint16 [P, page, kv_dim]) in place."""
    rows = _c(rows, np.uint16)
    seq, pos, pt = _c(seq, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    assert kv_cache.flags.c_contiguous
    skipped = ctypes.c_int(0)
    rc = _load().oracle_latent_cache_write(_ptr(rows), rows.shape[1], _ptr(seq), _ptr(pos), rows.shape[0], pt.shape[0], _ptr(pt),
                                           pt.shape[1], page_size, kv_cache.shape[0], _ptr(kv_cache),
                                           ctypes.byref(skipped))
    if rc != 0:
        raise ValueError(f"oracle call failed with code {rc}")
    return skipped.value


def indexer_key_project(h, w_k, seq, pos, page_table, page_size, k_cache, k_scale, threads=1):
    """k = h w_k^T (h uint16 bf16 bits [n_tok, d], w_k [Di, d]) quantised per token into k_cache
    (uint8 [P, page, Di]) / k_scale (float32 [P, page]) in place. Returns (k float32 [n_tok, Di]
    before quantisation, skipped-token count)."""
    h, w_k = _c(h, np.uint16), _c(w_k, np.uint16)
    seq, pos, pt = _c(seq, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    n_tok, d = h.shape
    Di = w_k.shape[0]
    assert k_cache.flags.c_contiguous and k_scale.flags.c_contiguous
    k = np.empty((n_tok, Di), np.float32)
    skipped = ctypes.c_int(0)
    rc = _load().oracle_indexer_key_project(_ptr(h), _ptr(w_k), n_tok, d, Di, _ptr(seq), _ptr(pos), pt.shape[0],
                                            _ptr(pt), pt.shape[1], page_size, k_cache.shape[0], _ptr(k_cache),
                                            _ptr(k_scale), _ptr(k), ctypes.byref(skipped))
    if rc != 0:
        raise ValueError(f"oracle call failed with code {rc}")
    return k, skipped.value


def indexer_query_project(c_q, w_q, h, w_w, Hi, Di, threads=1):
    """q8 = E4M3(c_q w_q^T) [rows, Hi, Di] and w = h w_w^T [rows, Hi] (float32); also q before its
    coding [rows, Hi, Di]. Rows are split over `threads` host threads."""
    c_q, w_q, h, w_w = (_c(x, np.uint16) for x in (c_q, w_q, h, w_w))
    rows, d_cq = c_q.shape
    d = h.shape[1]
    q8 = np.empty((rows, Hi, Di), np.uint8)
    w = np.empty((rows, Hi), np.float32)
    q = np.empty((rows, Hi, Di), np.float32)
    lib = _load()

    def fn(b, e):
        n = e - b
        return lib.oracle_indexer_query_project(_ptr(c_q[b:e]), _ptr(w_q), _ptr(h[b:e]), _ptr(w_w), n, d_cq, d, Hi, Di,
                                                q8[b:e].ctypes.data_as(ctypes.c_void_p),
                                                w[b:e].ctypes.data_as(ctypes.c_void_p),
                                                q[b:e].ctypes.data_as(ctypes.c_void_p))

    _run_rows(fn, rows, threads)
    return q8, w, q
