"""The fused indexer -> top-k call (dsa_indexer_topk) on the GPU.

The scan counts each row's valid scores by the top-k's first radix digit and the top-k starts
from those counts. Checks: the scores against the oracle (as for dsa_indexer_scores); the index
sets against the oracle's top-k of the oracle's scores (sets equal outside the tie band, as for
the separate calls); and the index lists bit for bit against dsa_topk on the same scores, whose
own parity with the oracle is exact. Repeated calls on one workspace (the histogram is left
zero by each call), rows of both unit widths (two MTP rows per scan unit, or one), rows no
longer than k, rows whose scores all tie (zero head weights) or are all <= 0 with signed zeros
(negative head weights), rows over one 16384-position chunk (whose chunk stages either pass on
the keys at or above the row's threshold first digit or select their own top k), and the
full-size decode batches.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_scores, check_topk_sets, gpu_inputs
from sparse_attention_06_amd import dsa

pytestmark = pytest.mark.gpu


def _fused(w, d, ws, k=None):
    return dsa.indexer_topk(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], w.n_seq, w.q_per_seq,
                            w.max_ctx, k or w.topk, ws=ws)


def _nh(max_ctx):
    # histograms per row in the workspace: one per 16384-position chunk, plus the merge's
    c = (max_ctx + 16383) // 16384
    return c + (1 if c > 1 else 0)


def _hist_part_zero(ws, hists):
    base = (-ws.data_ptr()) % 256
    return bool((ws[base: base + hists * 2048 * 4] == 0).all())


@pytest.mark.parametrize("qps,q_pos,max_ctx", [
    (2, [4999, 4998, 3000, 3001, 100, 2047], 5000),
    (1, [4095, 0, 2048, 3333, 64], 4096),
    (2, [16383, 16383, 9000, 9001], 16384),
    (1, [40000, 16384, 16383, 30000, 2047], 40001),   # rows over one chunk: two-stage top-k
    (2, [40000, 39999, 20000, 16385], 40001),          # two rows per scan unit over several chunks
    (3, [2999, 3000, 3001, 100, 2500, 2600], 3002),  # three rows per sequence: one row per scan unit
])
def test_fused_indexer_topk_matches_oracle(oracle_lib, qps, q_pos, max_ctx):
    print(f"case: fused indexer+topk qps={qps} q_pos={q_pos}", flush=True)
    n_seq = len(q_pos) // qps
    w = workloads.make_random(n_seq, qps, q_pos, max_ctx, H=2, Dqk=16, Dv=8, seed=57 + qps, permute_pages=True,
                              extra_pages=3)
    if qps == 2:
        w.iw[2:4] = 0.0                     # one unit: every score 0, all keys tie
        if w.rows > 4:
            w.iw[4] = -np.abs(w.iw[4])      # scores <= 0: -0 and +0 rank equal
    d = gpu_inputs(w)
    rows = w.rows
    ws = torch.zeros(dsa.indexer_topk_workspace_size(rows, max_ctx, w.topk), dtype=torch.uint8, device="cuda")
    results = []
    for _ in range(3):                      # the workspace is reused: each call re-zeroes its histogram
        s, idx = _fused(w, d, ws)
        torch.cuda.synchronize()
        assert dsa.last_path() == "indexer_topk_fused"
        assert _hist_part_zero(ws, rows * _nh(max_ctx))
        results.append((s.cpu().numpy(), idx.cpu().numpy()))
    for s_i, idx_i in results[1:]:
        for r in range(rows):               # entries past q_pos[r] are unspecified
            n = int(w.q_pos[r]) + 1
            np.testing.assert_array_equal(s_i[r, :n].view(np.uint32), results[0][0][r, :n].view(np.uint32))
        np.testing.assert_array_equal(idx_i, results[0][1])
    s_gpu, idx_gpu = results[0]
    ref_s = oracle.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, w.page_size, w.q_pos, w.n_seq,
                                  w.q_per_seq, w.fmt, w.max_ctx, threads=8)
    check_scores(s_gpu, ref_s, w.q_pos)
    check_topk_sets(idx_gpu, oracle.topk(ref_s, w.q_pos, w.topk, threads=8), ref_s, w.q_pos, w.topk)
    sep = dsa.topk(torch.from_numpy(s_gpu).cuda(), d["q_pos"], max_ctx, w.topk).cpu().numpy()
    np.testing.assert_array_equal(idx_gpu, sep)
    if qps == 2:
        # all-tie unit: the k smallest positions; non-positive row: equal to the separate top-k
        for r in (2, 3):
            n = int(w.q_pos[r]) + 1
            np.testing.assert_array_equal(idx_gpu[r, :min(n, w.topk)], np.arange(min(n, w.topk)))


@pytest.mark.parametrize("name", ["decode_mtp_b64_16k", "decode_b16_4k", "decode_b4_128k"])
def test_fused_full_size_equals_separate_calls(oracle_lib, name):
    """Full-size decode batches: index lists bit for bit equal to the separate calls (128K rows: the
    counts are per 16384-position chunk and the two-stage top-k's chunk stage starts from them)."""
    print(f"case: fused full size {name}", flush=True)
    w = getattr(workloads, "make_" + name)()
    d = gpu_inputs(w)
    ws = torch.zeros(dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        s, idx = _fused(w, d, ws)
    torch.cuda.synchronize()
    assert dsa.last_path() == "indexer_topk_fused"
    assert _hist_part_zero(ws, w.rows * _nh(w.max_ctx))
    s_sep = dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], w.n_seq,
                               w.q_per_seq, w.max_ctx)
    idx_sep = dsa.topk(s_sep, d["q_pos"], w.max_ctx, w.topk)
    torch.cuda.synchronize()
    s_h, s_sep_h = s.cpu().numpy().view(np.uint32), s_sep.cpu().numpy().view(np.uint32)
    for r in range(w.rows):                 # entries past q_pos[r] are unspecified
        n = int(w.q_pos[r]) + 1
        np.testing.assert_array_equal(s_h[r, :n], s_sep_h[r, :n])
    assert torch.equal(idx, idx_sep)
    # sampled rows against the oracle
    rows = sorted({0, w.rows - 1, w.rows // 2})
    ref_s = oracle.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, w.page_size, w.q_pos, w.n_seq,
                                  w.q_per_seq, w.fmt, w.max_ctx, threads=8, rows=rows)
    check_scores(s.cpu().numpy(), ref_s, w.q_pos, rows=rows)
    ref_idx = oracle.topk(ref_s[rows], w.q_pos[rows], w.topk, threads=8)
    check_topk_sets(idx.cpu().numpy()[rows], ref_idx, ref_s[rows], w.q_pos[rows], w.topk)


def test_fused_ragged_long_rows_equal_separate_calls(oracle_lib):
    """The 128K-context decode size with ragged lengths (16385, 20000, 70000, 131072): most rows
    end in a short 16384-position chunk or have empty ones, whose chunk stage keeps every key and
    adds all its counts to the merge's histogram. Index lists bit for bit equal to the separate
    calls and to the oracle's top-k of the same scores (exact), on one workspace used twice."""
    print("case: fused ragged long rows", flush=True)
    q_pos = [16384, 19999, 69999, 131071]
    w = workloads.make_random(4, 1, q_pos, 131072, H=2, Dqk=16, Dv=8, seed=93, permute_pages=True, extra_pages=5)
    d = gpu_inputs(w)
    ws = torch.zeros(dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        s, idx = _fused(w, d, ws)
        torch.cuda.synchronize()
        assert dsa.last_path() == "indexer_topk_fused"
        assert _hist_part_zero(ws, w.rows * _nh(w.max_ctx))
        runs.append(idx.cpu().numpy())
    np.testing.assert_array_equal(runs[0], runs[1])
    s_sep = dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], w.n_seq,
                               w.q_per_seq, w.max_ctx)
    idx_sep = dsa.topk(s_sep, d["q_pos"], w.max_ctx, w.topk)
    torch.cuda.synchronize()
    s_h = s.cpu().numpy()
    for r in range(w.rows):
        n = int(w.q_pos[r]) + 1
        np.testing.assert_array_equal(s_h[r, :n].view(np.uint32), s_sep.cpu().numpy()[r, :n].view(np.uint32))
    np.testing.assert_array_equal(runs[0], idx_sep.cpu().numpy())
    np.testing.assert_array_equal(runs[0], oracle.topk(s_h, w.q_pos, w.topk, threads=8))


def test_fused_long_rows_row_threshold_and_own_selection(oracle_lib):
    """Rows over 16384 positions whose chunks take both chunk-stage forms: a chunk passes on its
    keys at or above the row's threshold first digit when there are at most k of them, else it
    selects its own top k. Row 0: random scores. Row 1: the first chunk's key scales times 1000,
    so the row's top k lies in that chunk (which selects its own) and the other chunks pass on
    nothing. Row 2: zero head weights, every score ties (every chunk selects its own; the k
    smallest positions win). Row 3: no longer than k (every key kept). Index lists bit for bit
    equal to the separate calls and to the oracle's top-k of the same scores."""
    print("case: fused long rows, row threshold and own selection", flush=True)
    q_pos = [131071, 100000, 70000, 2047]
    w = workloads.make_random(4, 1, q_pos, 131072, H=2, Dqk=16, Dv=8, seed=95, permute_pages=True, extra_pages=2)
    pages = w.page_table[1, : 16384 // w.page_size]
    w.iks[pages] *= 1000.0
    w.iw[2] = 0.0
    d = gpu_inputs(w)
    ws = torch.zeros(dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        s, idx = _fused(w, d, ws)
        torch.cuda.synchronize()
        assert dsa.last_path() == "indexer_topk_fused"
        assert _hist_part_zero(ws, w.rows * _nh(w.max_ctx))
        runs.append(idx.cpu().numpy())
    np.testing.assert_array_equal(runs[0], runs[1])
    s_h = s.cpu().numpy()
    idx_sep = dsa.topk(s, d["q_pos"], w.max_ctx, w.topk).cpu().numpy()
    np.testing.assert_array_equal(runs[0], idx_sep)
    np.testing.assert_array_equal(runs[0], oracle.topk(s_h, w.q_pos, w.topk, threads=8))
    assert (runs[0][1] < 16384).all()                                   # row 1: all from the first chunk
    np.testing.assert_array_equal(runs[0][2], np.arange(w.topk))         # row 2: ties, smallest positions
    np.testing.assert_array_equal(runs[0][3], np.arange(w.topk))         # row 3: every key


def test_fused_long_rows_many_chunk_workgroups(oracle_lib):
    """64 rows (32 units of two MTP rows) over up to 131072 positions: 512 chunk-stage workgroups,
    so the chunk stage and the merge take the two-per-CU variants, with the row-threshold filter.
    One unit has zero head weights (every score ties). Index lists bit for bit equal to the
    separate calls; three rows against the oracle's top-k of the same scores."""
    print("case: fused long rows, 512 chunk-stage workgroups", flush=True)
    lens = [131072, 100000, 40000, 16385, 2048, 70001, 131072, 65536]
    q_pos = []
    for u in range(32):
        n = lens[u % len(lens)]
        q_pos += [n - 1, n - 2]
    w = workloads.make_random(32, 2, q_pos, 131072, H=2, Dqk=16, Dv=8, seed=97, permute_pages=True)
    w.iw[12:14] = 0.0
    d = gpu_inputs(w)
    ws = torch.zeros(dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        s, idx = _fused(w, d, ws)
        torch.cuda.synchronize()
        assert dsa.last_path() == "indexer_topk_fused"
        assert _hist_part_zero(ws, w.rows * _nh(w.max_ctx))
        runs.append(idx.cpu().numpy())
    np.testing.assert_array_equal(runs[0], runs[1])
    idx_sep = dsa.topk(s, d["q_pos"], w.max_ctx, w.topk).cpu().numpy()
    np.testing.assert_array_equal(runs[0], idx_sep)
    rows = [0, 13, 63]
    s_h = s.cpu().numpy()
    np.testing.assert_array_equal(runs[0][rows], oracle.topk(s_h[rows], w.q_pos[rows], w.topk, threads=8))
    np.testing.assert_array_equal(runs[0][12], np.arange(w.topk))


def test_fused_rejects_small_workspace():
    w = workloads.make_random(1, 2, [300, 301], 320, H=2, Dqk=16, Dv=8, seed=3)
    d = gpu_inputs(w)
    need = dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk)
    with pytest.raises(dsa.DSAError, match="WORKSPACE"):
        _fused(w, d, torch.zeros(need - 1, dtype=torch.uint8, device="cuda"))
