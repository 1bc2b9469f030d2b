"""CPU-side checks of the C ABI: the library loads, exports every entry point that
include/dsa.h declares, and rejects bad host arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from sparse_attention_06_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.lib_path()):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    return dsa.load()


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ["dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
              "dsa_dense_mla_prefill"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(dsa.lib_path())
    for n in _declared():
        assert hasattr(raw, n), f"{n} declared in include/dsa.h but not exported"
    assert sorted(dsa.EXPORTS) == _declared()


def test_status_strings(lib):
    assert lib.dsa_status_string(0) == b"DSA_OK"
    assert lib.dsa_status_string(3) == b"DSA_ERR_WORKSPACE"


NULL = None


def test_indexer_rejects_null_and_bad_dims(lib):
    st = lib.dsa_indexer_scores(NULL, NULL, NULL, NULL, NULL, 1, 64, 1, NULL, NULL, 1, 1, 1, 64, 64, 128, 0, NULL, 64, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG
    assert b"non-NULL" in lib.dsa_last_error()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    st = lib.dsa_indexer_scores(fake, fake, fake, NULL, fake, 1, 64, 1, NULL, fake, 1, 1, 1, 64, 64, 128, 7, fake, 64, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG and b"dtype" in lib.dsa_last_error()
    st = lib.dsa_indexer_scores(fake, fake, fake, NULL, fake, 1, 64, 1, NULL, fake, 1, 1, 1, 128, 64, 128, 0, fake, 64, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG    # ld_pt too small for max_ctx = 128
    st = lib.dsa_indexer_scores(fake, fake, fake, NULL, fake, 2, 64, 1, NULL, fake, 1, 1, 1, 128, 64, 128, 0, fake, 64, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG    # ld_scores < max_ctx
    mis = ctypes.c_void_p(0x1004)
    st = lib.dsa_indexer_scores(mis, fake, fake, NULL, fake, 2, 64, 1, NULL, fake, 1, 1, 1, 128, 64, 128, 0, fake, 128, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG and b"aligned" in lib.dsa_last_error()


def test_topk_rejects_bad_k(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.dsa_topk(fake, 64, fake, 4, 64, 0, fake, 64, NULL, 0, NULL) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(fake, 64, fake, 4, 64, 32, fake, 16, NULL, 0, NULL) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_workspace_size(128, 16384, 2048) == 0


def test_fused_indexer_topk_workspace_and_arguments(lib):
    """The fused call sizes its workspace from the rows' chunks (per-chunk counts, the merge's counts
    for rows over one chunk, then the two-stage top-k's own workspace) and rejects a missing or
    small workspace and bad k before any launch."""
    size = lib.dsa_indexer_topk_workspace_size
    one = size(128, 16384, 2048)
    assert one == 256 + 128 * 2048 * 4                       # one chunk: counts only
    long_rows = size(4, 131072, 2048)
    assert long_rows == 256 + 4 * (8 + 1) * 2048 * 4 + lib.dsa_topk_workspace_size(4, 131072, 2048)
    assert size(0, 16384, 2048) == 0
    fake = ctypes.c_void_p(0x1000)
    args = (fake, fake, fake, fake, fake, 256, 64, 256, NULL, fake, 128, 64, 2, 16384, 64, 128, 0, fake, 16384)
    assert lib.dsa_indexer_topk(*args, 2048, fake, 2048, NULL, 0, NULL) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_indexer_topk(*args, 2048, fake, 2048, fake, one - 1, NULL) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_indexer_topk(*args, 0, fake, 2048, fake, one, NULL) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_topk(*args, 2048, fake, 1024, fake, one, NULL) == dsa.DSA_ERR_INVALID_ARG


def test_attention_rejects_unsupported_and_inconsistent(lib):
    fake = ctypes.c_void_p(0x1000)
    # v_col0 + Dv beyond the row
    st = lib.dsa_sparse_mla_decode(fake, fake, fake, 1, 64, 1, NULL, fake, 1, 1, 1, fake, 8, 8, 128, 576, 512, 576, 65,
                                   ctypes.c_float(0.1), fake, NULL, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG
    # a shape no kernel handles is reported, never substituted
    st = lib.dsa_sparse_mla_decode(fake, fake, fake, 1, 64, 1, NULL, fake, 1, 1, 1, fake, 8, 8, 4, 2048, 64, 2048, 0,
                                   ctypes.c_float(0.1), fake, NULL, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    # the tuned decode path needs its split workspace for small batches
    need = lib.dsa_sparse_mla_workspace_size(4, 128, 512, 2048)
    assert need > 0
    st = lib.dsa_sparse_mla_decode(fake, fake, fake, 64, 64, 64, NULL, fake, 4, 4, 1, fake, 2048, 2048, 128, 576, 512,
                                   576, 0,
                                   ctypes.c_float(0.1), fake, NULL, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_WORKSPACE
    st = lib.dsa_dense_mla_prefill(fake, fake, fake, 1, 64, 1, NULL, fake, 4, 1, 4, 0, 128, 576, 512, 576, 0,
                                   ctypes.c_float(0.1), fake, NULL, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG    # max_ctx = 0


def test_row_descriptor_checks(lib):
    """rows must equal n_seq * q_per_seq without q_seq; with q_seq, q_per_seq must be 1 and rows need
    a sequence; the binding rejects a q_seq of the wrong length."""
    fake = ctypes.c_void_p(0x1000)
    args = (fake, fake, fake, NULL, fake, 1, 64, 1)
    tail = (64, 64, 128, 0, fake, 64, NULL)
    assert lib.dsa_indexer_scores(*args, NULL, fake, 5, 2, 2, *tail) == dsa.DSA_ERR_INVALID_ARG
    assert b"n_seq * q_per_seq" in lib.dsa_last_error()
    assert lib.dsa_indexer_scores(*args, fake, fake, 4, 2, 2, *tail) == dsa.DSA_ERR_INVALID_ARG
    assert b"q_per_seq must be 1" in lib.dsa_last_error()
    assert lib.dsa_indexer_scores(*args, fake, fake, 4, 0, 1, *tail) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(*args, fake, fake, 0, 3, 1, *tail) == dsa.DSA_OK      # no rows: nothing to do
    st = lib.dsa_sparse_mla_prefill(fake, fake, fake, 1, 64, 1, fake, fake, 3, 2, 2, fake, 8, 8, 128, 576, 512, 576,
                                    0, ctypes.c_float(0.1), fake, NULL, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_INVALID_ARG


def _attention_splits(rows, k, nk=32):
    """The decode split rule restated: double while fewer than 256 workgroups and each split keeps
    at least 4 tiles of nk keys."""
    s = 1
    while rows * s < 256 and k // (s * 2) >= 4 * nk:
        s *= 2
    return s


def _align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("rows,k", [(1, 2048), (4, 2048), (16, 2048), (64, 2048), (128, 2048), (130, 256), (255, 2048),
                                    (256, 2048), (3, 128), (5, 100)])
def test_attention_split_workspace_follows_the_split_rule(lib, rows, k):
    """Workspace bytes of the decode split: fp16 partials [units, 128, 512] and (max, sum) pairs
    [units, 128], each part 256-byte aligned, for units = rows x splits; none without a split."""
    s = _attention_splits(rows, k)
    want = 0 if s == 1 else _align256(rows * s * 128 * 512 * 2) + _align256(rows * s * 128 * 8)
    assert lib.dsa_sparse_mla_workspace_size(rows, 128, 512, k) == want


def _projection_ws(M, N, K):
    """The projection split-K plan restated: split only when 128-row tiles give fewer than 512
    workgroups; then deal K blocks of 64 so that about 1024 32-row workgroups run, at most 16 ways."""
    n_tiles = (N + 127) // 128
    tiles = (M + 31) // 32 * n_tiles
    kb = K // 64
    if (M + 127) // 128 * n_tiles >= 512 or kb < 2:
        return 0
    want = min(1024 // tiles, kb, 16)
    if want < 2:
        return 0
    per = (kb + want - 1) // want
    kz = (kb + per - 1) // per
    return kz * M * N * 4 if kz > 1 else 0


@pytest.mark.parametrize("rows,d", [(1, 7168), (128, 7168), (600, 7168), (3900, 7168), (4096, 7168), (16384, 7168),
                                    (65536, 7168), (131072, 7168), (300, 128), (37, 64)])
def test_projection_workspace_follows_the_split_plan(lib, rows, d):
    """The projection workspace covers the split-K partials of both calls' GEMMs (keys: N = 128;
    head weights: N = 64)."""
    want = max(_projection_ws(rows, 128, d), _projection_ws(rows, 64, d))
    assert lib.dsa_indexer_projection_workspace_size(rows, d) == want


def test_projection_rejects_oversized_reduction_dims(lib):
    """d and d_cq above 65536 are reported as unsupported before any launch."""
    fake = ctypes.c_void_p(0x1000)
    st = lib.dsa_indexer_key_project(fake, fake, 4, 65536 + 64, 128, fake, fake, 1, fake, 1, 64, 1, fake, fake, NULL, 0,
                                     NULL)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    st = lib.dsa_indexer_query_project(fake, fake, fake, fake, 4, 65536 + 64, 128, 64, 128, fake, fake, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    st = lib.dsa_indexer_query_project(fake, fake, fake, fake, 4, 128, 65536 + 64, 64, 128, fake, fake, NULL, 0, NULL)
    assert st == dsa.DSA_ERR_UNSUPPORTED
