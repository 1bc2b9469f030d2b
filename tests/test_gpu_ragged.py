"""Ragged batches through the per-row query descriptor (q_seq) on the GPU, against the oracle.

One call holds rows of three sequences with different row counts, interleaved: a decode request
(1 row), an MTP-style request (3 rows) and a 300-row prefill chunk, each over its own paged
caches (permuted pages). Checked through the C ABI: the indexer (scan path and, with 32-token
pages, the query x key tile path) and the fused indexer + top-k against the oracle's scores and
top-k; the sparse attention (decode and prefill entry points) and the dense fallback against the
oracle on the decode rows and sampled chunk rows; the uniform layout given as per-row ids gives
the same attention bit for bit; and a row whose sequence id lies outside the page table touches
nothing and leaves the other rows unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_attn, check_scores, check_topk_sets, gpu_inputs
from sparse_attention_06_amd import dsa

pytestmark = pytest.mark.gpu

THREADS = 8


def _ragged():
    """Caches of 3 sequences (make_random's), and 304 query rows: sequence 0 one decode row at
    2999, sequence 1 three rows at 2497..2499, sequence 2 a chunk at 2000..2299; interleaved."""
    lens = [3000, 2500, 2300]
    w = workloads.make_random(3, 1, [x - 1 for x in lens], 3000, seed=211, permute_pages=True, extra_pages=4)
    seq = np.array([0] + [1] * 3 + [2] * 300, np.int32)
    pos = np.concatenate([[2999], np.arange(2497, 2500), np.arange(2000, 2300)]).astype(np.int32)
    order = np.random.default_rng(5).permutation(seq.size)
    seq, pos = seq[order], pos[order]
    g = torch.Generator()
    g.manual_seed(212)
    n = seq.size
    w.iq = workloads.e4m3_bits(torch.randn(n, 64, 128, generator=g))
    w.iw = (torch.randn(n, 64, generator=g) / 8.0).numpy()
    w.q = workloads.bf16_bits(torch.randn(n, 128, 576, generator=g))
    w.q_pos = pos
    w.q_per_seq = 1
    return w, seq


def _sample(seq, pos):
    rows = [i for i in range(seq.size) if seq[i] != 2]                      # decode and MTP rows
    chunk = np.nonzero(seq == 2)[0]
    rows += [int(chunk[np.argmin(pos[chunk])]), int(chunk[np.argmax(pos[chunk])])]
    rows += [int(x) for x in np.random.default_rng(7).choice(chunk, 10, replace=False)]
    return np.array(sorted(set(rows)))


def test_ragged_indexer_topk_and_attention(oracle_lib):
    print("case: ragged batch (1 + 3 + 300 rows), indexer, top-k, attention", flush=True)
    w, seq = _ragged()
    d = gpu_inputs(w)
    qs = torch.from_numpy(seq).cuda()
    n = seq.size
    s = dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx, q_seq=qs)
    assert dsa.last_path() == "indexer_scan_mfma"
    ref_s = oracle.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, 64, w.q_pos, 3, 1, w.fmt, w.max_ctx,
                                  threads=THREADS, q_seq=seq)
    s_h = s.cpu().numpy()
    check_scores(s_h, ref_s, w.q_pos)
    ref_idx = oracle.topk(ref_s, w.q_pos, 2048, threads=THREADS)
    idx = dsa.topk(s, d["q_pos"], w.max_ctx, 2048)
    check_topk_sets(idx.cpu().numpy(), ref_idx, ref_s, w.q_pos, 2048)
    # the fused call: same scores and index lists as the separate calls
    s_f, idx_f = dsa.indexer_topk(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx,
                                  2048, q_seq=qs)
    assert dsa.last_path() == "indexer_topk_fused" and torch.equal(idx_f, idx)
    for r in range(n):
        t = int(w.q_pos[r]) + 1
        np.testing.assert_array_equal(s_f.cpu().numpy()[r, :t].view(np.uint32), s_h[r, :t].view(np.uint32))

    rows = _sample(seq, w.q_pos)
    d_idx = torch.from_numpy(ref_idx).cuda()
    ref_o, ref_lse = oracle.sparse_mla(w.q, w.kv, w.page_table, 64, w.q_pos, 3, 1, ref_idx, w.Dqk, w.Dv, w.v_col0,
                                       w.sm_scale, threads=THREADS, rows=rows, q_seq=seq)
    for fn in (dsa.sparse_mla_decode, dsa.sparse_mla_prefill):
        lse = torch.empty(n, 128, dtype=torch.float32, device="cuda")
        out = fn(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 1, d_idx, w.Dqk, w.Dv, w.v_col0, w.sm_scale,
                 lse=lse, q_seq=qs)
        assert dsa.last_path().startswith("mla_mfma")
        check_attn(out.float().cpu().numpy()[rows], ref_o[rows])
        np.testing.assert_allclose(lse.cpu().numpy()[rows], ref_lse[rows], rtol=0, atol=1e-4)
    dense = dsa.dense_mla_prefill(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx, w.Dqk, w.Dv,
                                  w.v_col0, w.sm_scale, q_seq=qs)
    ref_d, _ = oracle.dense_mla(w.q, w.kv, w.page_table, 64, w.q_pos, 3, 1, w.Dqk, w.Dv, w.v_col0, w.sm_scale,
                                threads=THREADS, rows=rows, q_seq=seq)
    check_attn(dense.float().cpu().numpy()[rows], ref_d[rows])


def test_ragged_indexer_tile_path_other_page_size(oracle_lib):
    """32-token pages take the query x key tile kernel, whose waves pair consecutive rows: pairs
    that straddle two sequences are scanned one row at a time."""
    print("case: ragged batch, 32-token pages", flush=True)
    w, seq = _ragged()
    d = gpu_inputs(w)
    P = d["ik"].shape[0]
    ik32 = d["ik"].reshape(2 * P, 32, 128).contiguous()
    iks32 = d["iks"].reshape(2 * P, 32).contiguous()
    pt = d["page_table"].long()
    pt32 = torch.stack([2 * pt, 2 * pt + 1], dim=2).reshape(pt.shape[0], -1).to(torch.int32).contiguous()
    s = dsa.indexer_scores(d["iq"], d["iw"], ik32, iks32, pt32, d["q_pos"], 3, 1, w.max_ctx,
                           q_seq=torch.from_numpy(seq).cuda())
    assert dsa.last_path() == "indexer_prefill_mfma"
    ref_s = oracle.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, 64, w.q_pos, 3, 1, w.fmt, w.max_ctx,
                                  threads=THREADS, q_seq=seq)
    check_scores(s.cpu().numpy(), ref_s, w.q_pos)


def test_uniform_layout_as_per_row_ids_is_bit_identical(oracle_lib):
    """The uniform layout (2 rows per request) written out as per-row sequence ids gives the same
    attention outputs bit for bit, and the same index lists."""
    print("case: uniform layout as per-row ids", flush=True)
    q_pos = [3000, 3001, 1500, 1501, 2047, 2048]
    w = workloads.make_random(3, 2, q_pos, 3002, seed=221, permute_pages=True, extra_pages=2)
    d = gpu_inputs(w)
    qs = torch.arange(6, dtype=torch.int32, device="cuda") // 2
    s1, i1 = dsa.indexer_topk(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 2, w.max_ctx, 2048)
    s2, i2 = dsa.indexer_topk(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx, 2048,
                              q_seq=qs)
    assert torch.equal(i1, i2)
    args = (w.Dqk, w.Dv, w.v_col0, w.sm_scale)
    o1 = dsa.sparse_mla_decode(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 2, i1, *args)
    o2 = dsa.sparse_mla_decode(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 1, i1, *args, q_seq=qs)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_row_with_sequence_outside_the_table(oracle_lib):
    """A row whose sequence id lies outside [0, n_seq): the kernels bound-check it (no page-table
    access), its attention is over an empty set (zeros), and the other rows are unchanged."""
    print("case: row with an out-of-range sequence id", flush=True)
    q_pos = [1200, 900, 500]
    w = workloads.make_random(3, 1, q_pos, 1201, seed=231, permute_pages=True)
    d = gpu_inputs(w)
    good = torch.arange(3, dtype=torch.int32, device="cuda")
    bad = good.clone()
    bad[1] = 7
    s_good = dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx,
                                q_seq=good)
    s_bad = dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], 3, 1, w.max_ctx,
                               q_seq=bad)
    for r in (0, 2):
        t = q_pos[r] + 1
        assert torch.equal(s_good[r, :t], s_bad[r, :t])
    idx = dsa.topk(s_good, d["q_pos"], w.max_ctx, 2048)
    args = (w.Dqk, w.Dv, w.v_col0, w.sm_scale)
    o_good = dsa.sparse_mla_prefill(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 1, idx, *args, q_seq=good)
    o_bad = dsa.sparse_mla_prefill(d["q"], d["kv"], d["page_table"], d["q_pos"], 3, 1, idx, *args, q_seq=bad)
    torch.cuda.synchronize()
    assert torch.equal(o_good[0].view(torch.int16), o_bad[0].view(torch.int16))
    assert torch.equal(o_good[2].view(torch.int16), o_bad[2].view(torch.int16))
    assert (o_bad[1].float() == 0).all()
