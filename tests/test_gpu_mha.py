"""Expanded multi-head attention (the short-prefill fallback) on the GPU against the oracle.

Dense causal and masked (index-set) modes; ragged query blocks (rows not a multiple of the
256-row workgroup block), a context that is not a multiple of the 32-position tile, rows that see
nothing, index lists with repeats, padding and invisible entries; and a full-size 128-head case
on sampled rows. Tolerances as for the absorbed attention (helpers.check_attn); lse within 1e-3.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import check_attn
from sparse_attention_06_amd import dsa

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(seed, n_seq, q_per_seq, H, max_ctx, q_pos, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rows = n_seq * q_per_seq
    q = torch.randn(rows, H, 192, generator=g, device=device).to(torch.bfloat16)
    kn = torch.randn(n_seq, H, max_ctx, 128, generator=g, device=device).to(torch.bfloat16)
    kr = torch.randn(n_seq, max_ctx, 64, generator=g, device=device).to(torch.bfloat16)
    v = torch.randn(n_seq, H, max_ctx, 128, generator=g, device=device).to(torch.bfloat16)
    return q, kn, kr, v, torch.from_numpy(np.asarray(q_pos, np.int32)).to(device)


def _rand_idx(q_pos, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((len(q_pos), k), -1, np.int32)
    for r, t in enumerate(q_pos):
        if t < 0:
            continue
        m = min(k, t + 1)
        sel = rng.choice(t + 1, m, replace=False)
        idx[r, :m] = sel
        if m >= 4 and r % 3 == 0:
            idx[r, m - 1] = sel[0]           # a repeat
        if m < k:
            idx[r, m] = t + 5                # invisible: ignored
    return idx


def _check(q, kn, kr, v, qp, n_seq, qps, idx, scale, rows=None):
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
    idx_d = None if idx is None else torch.from_numpy(idx).cuda()
    out = dsa.expanded_mha_prefill(q, kn, kr, v, qp, n_seq, qps, scale, idx=idx_d, lse=lse)
    torch.cuda.synchronize()
    assert dsa.last_path() == ("mha_mfma" if idx is None else "mha_mfma_masked")
    ref_o, ref_l = oracle.mha(_bits(q), _bits(kn), _bits(kr), _bits(v), qp.cpu().numpy(), n_seq, qps, idx, scale,
                              threads=THREADS, rows=rows)
    sel = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    check_attn(out.float().cpu().numpy()[sel], ref_o[sel])
    got_l, want_l = lse.cpu().numpy()[sel], ref_l[sel]
    fin = np.isfinite(want_l)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    np.testing.assert_allclose(got_l[fin], want_l[fin], rtol=0, atol=1e-3)


@pytest.mark.parametrize("masked", [False, True])
def test_mha_ragged_blocks_and_tail(oracle_lib, masked):
    # 2 sequences x 300 rows (a full 256-row block and a 44-row one), 333 positions (ragged tile)
    n_seq, qps, H, T = 2, 300, 3, 333
    rng = np.random.default_rng(7)
    q_pos = np.concatenate([np.sort(rng.integers(0, T, qps)) for _ in range(n_seq)]).astype(np.int32)
    q_pos[0], q_pos[1], q_pos[qps - 1] = 0, 31, T - 1
    print(f"case: mha ragged masked={masked}", flush=True)
    q, kn, kr, v, qp = _case(1, n_seq, qps, H, T, q_pos)
    idx = _rand_idx(q_pos, 64, 2) if masked else None
    _check(q, kn, kr, v, qp, n_seq, qps, idx, 1 / math.sqrt(192))


def test_mha_prefill_block_masked_and_empty_rows(oracle_lib):
    # one sequence, positions 0..T-1 (prefill): rows with t < k keep every position; a row with an
    # empty index set and a row at a negative position see nothing (out 0, lse -inf)
    T, H, k = 700, 2, 96
    q_pos = np.arange(T, dtype=np.int32)
    q_pos[5] = -1
    print("case: mha prefill masked", flush=True)
    q, kn, kr, v, qp = _case(3, 1, T, H, T, q_pos)
    idx = _rand_idx(q_pos, k, 4)
    idx[9] = -1
    _check(q, kn, kr, v, qp, 1, T, idx, 0.11)
    _check(q, kn, kr, v, qp, 1, T, None, 0.11)


def test_mha_full_index_sets_equal_dense(oracle_lib):
    # masked mode with every visible position listed equals the dense causal result bit for bit
    T, H = 300, 2
    q_pos = np.arange(T, dtype=np.int32)
    q, kn, kr, v, qp = _case(5, 1, T, H, T, q_pos)
    idx = np.full((T, T), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t, -1, -1)
    dense = dsa.expanded_mha_prefill(q, kn, kr, v, qp, 1, T, 0.07)
    full = dsa.expanded_mha_prefill(q, kn, kr, v, qp, 1, T, 0.07, idx=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), full.view(torch.int16))


@pytest.mark.parametrize("masked", [False, True])
def test_mha_full_size_sampled_rows(oracle_lib, masked):
    # 128 heads, one 4096-position prefill block; the oracle checks 12 sampled rows
    T, H, k = 4096, 128, 2048
    q_pos = np.arange(T, dtype=np.int32)
    print(f"case: mha full size masked={masked}", flush=True)
    q, kn, kr, v, qp = _case(9, 1, T, H, T, q_pos)
    idx = _rand_idx(q_pos, k, 10) if masked else None
    rows = [0, 1, 255, 256, 2046, 2047, 2048, 2049, 3000, 4094, 4095, 777]
    _check(q, kn, kr, v, qp, 1, T, idx, 1 / math.sqrt(192), rows=sorted(rows))


def test_mha_rejects_other_shapes_and_missing_workspace():
    q, kn, kr, v, qp = _case(11, 1, 8, 2, 40, np.arange(8))
    with pytest.raises(dsa.DSAError, match="UNSUPPORTED"):
        dsa.expanded_mha_prefill(q, kn[..., :64].contiguous(), kr, v, qp, 1, 8, 0.1)
    idx = torch.zeros(8, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DSAError, match="WORKSPACE"):
        dsa.expanded_mha_prefill(q, kn, kr, v, qp, 1, 8, 0.1, idx=idx, ws=torch.empty(4, dtype=torch.uint8, device="cuda"))
