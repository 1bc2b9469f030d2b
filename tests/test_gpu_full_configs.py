"""Full-size workloads, run exactly as the benchmark runs them (the same entry points, buffers and
launch configuration, via bench.DecodeStep), checked against the oracle.

Rows checked per workload: every row of the decode workloads (16 x 4K, 64 x 2 x 16K, 4 x 128K);
for the prefill blocks (8192 rows over 8K positions, 4096 rows over 128K positions) a sample of
the first and last rows, rows at t = k-2 .. k+1 where they exist, and seeded random rows. The
oracle runs on a compact copy of the sampled rows (each row its own one-row sequence with its
original page-table row), so its arrays stay small.

Per sampled row: indexer scores within 1e-5 * max|I| of the oracle, top-k sets equal outside the
tie band, and attention (run on the GPU with the oracle's index sets written into those rows,
then the full-size call repeated) within 2e-2 max abs / 5e-3 relative RMS."""
import os

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from helpers import check_attn, check_scores, check_topk_sets

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


def _sample_rows(w, n, seed):
    rows = w.rows
    if n is None or n >= rows:
        return np.arange(rows)
    pick = {0, rows - 1}
    for t in range(w.topk - 2, w.topk + 2):
        hit = np.nonzero(w.q_pos == t)[0]
        if hit.size:
            pick.add(int(hit[0]))
    rng = np.random.default_rng(seed)
    while len(pick) < n:
        pick.add(int(rng.integers(0, rows)))
    return np.array(sorted(pick))


def _subset(w, rows):
    seq = rows // w.q_per_seq
    return {"iq": w.iq[rows], "iw": w.iw[rows], "q": w.q[rows], "q_pos": w.q_pos[rows],
            "pt": np.ascontiguousarray(w.page_table[seq])}


@pytest.mark.parametrize("name,nsample", [
    ("decode_b16_4k", None),
    ("decode_mtp_b64_16k", None),
    ("decode_b4_128k", None),
    ("prefill_8k", 128),
    ("prefill_chunk_128k", 64),
])
def test_full_size_workload(oracle_lib, name, nsample):
    print(f"case: full-size {name}", flush=True)
    w = workloads.MAKERS[name]()
    step = bench.DecodeStep(w, copies=1)
    step.run(0)
    torch.cuda.synchronize()
    d = step.copies[0]
    rows = _sample_rows(w, nsample, seed=0xD5A0)
    sub = _subset(w, rows)
    ns = len(rows)
    rows_t = torch.from_numpy(rows).cuda()

    # indexer
    ref_s = oracle.indexer_scores(sub["iq"], sub["iw"], w.ik, w.iks, sub["pt"], w.page_size, sub["q_pos"], ns, 1,
                                  w.fmt, w.max_ctx, threads=THREADS)
    check_scores(d["scores"].index_select(0, rows_t).cpu().numpy(), ref_s, sub["q_pos"])

    # top-k
    ref_idx = oracle.topk(ref_s, sub["q_pos"], w.topk, threads=THREADS)
    check_topk_sets(d["idx"].index_select(0, rows_t).cpu().numpy(), ref_idx, ref_s, sub["q_pos"], w.topk)

    # attention on the oracle's index sets, through the same full-size call
    d["idx"][rows_t] = torch.from_numpy(ref_idx).cuda()
    step.call_mla(0, step.stream)
    torch.cuda.synchronize()
    ref_o, _ = oracle.sparse_mla(sub["q"], w.kv, sub["pt"], w.page_size, sub["q_pos"], ns, 1, ref_idx, w.Dqk, w.Dv,
                                 w.v_col0, w.sm_scale, threads=THREADS)
    check_attn(d["out"].index_select(0, rows_t).float().cpu().numpy(), ref_o)


@pytest.mark.parametrize("T", [1024, 2048])
def test_crossover_dense_fallbacks(oracle_lib, T):
    """The prefill blocks the crossover sweep runs against the dense fallbacks (T = 1024 and 2048,
    both no longer than k = 2048, so dense causal attention is exact DSA: [Handbook] k = min(L,
    2048)), through the calls the sweep times (bench.CrossoverCase). Sampled rows of the absorbed
    dense fallback against the oracle's dense attention and its sparse attention over the full
    set; sampled rows of the expanded multi-head fallback against the oracle's expanded attention."""
    print(f"case: crossover dense fallbacks T={T}", flush=True)
    c = bench.CrossoverCase(T, keep_host=True)
    w = c.w
    c.dense()
    c.expanded()
    torch.cuda.synchronize()
    rows = _sample_rows(w, 16, seed=0xD5A0 + T)
    rows_t = torch.from_numpy(rows).cuda()
    got = c.out.index_select(0, rows_t).float().cpu().numpy()
    sub = _subset(w, rows)
    ns = len(rows)
    ref_d, _ = oracle.dense_mla(sub["q"], w.kv, sub["pt"], w.page_size, sub["q_pos"], ns, 1, w.Dqk, w.Dv, w.v_col0,
                                w.sm_scale, threads=THREADS)
    check_attn(got, ref_d)
    full = np.full((ns, w.topk), -1, np.int32)
    for i, t in enumerate(sub["q_pos"]):
        full[i, : t + 1] = np.arange(t + 1)
    ref_s, _ = oracle.sparse_mla(sub["q"], w.kv, sub["pt"], w.page_size, sub["q_pos"], ns, 1, full, w.Dqk, w.Dv,
                                 w.v_col0, w.sm_scale, threads=THREADS)
    np.testing.assert_array_equal(ref_s, ref_d)   # exact inside the oracle when k >= t + 1
    # expanded fallback: the sampled rows' queries against the whole sequence's keys and values
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    ref_x, _ = oracle.mha(bits(c.xq.index_select(0, rows_t)), bits(c.xkn), bits(c.xkr), bits(c.xv), sub["q_pos"], 1,
                          ns, None, c.scale, threads=THREADS)
    check_attn(c.xout.index_select(0, rows_t).float().cpu().numpy(), ref_x)
