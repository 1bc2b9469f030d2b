"""Pins of the CPU oracle against facts fixed independently of it (CPU only).

Each test checks the oracle against something other than itself: the worked example printed
on the DSA blog page, library routines (torch's FP8/bf16 decoders, torch.topk, numpy einsum,
torch's float64 scaled_dot_product_attention), closed forms and brute force. The cases are
chosen so that a plausible slip (a dropped ReLU, a sign, a transposed operand, a wrong tie
rule, a missing scale, an off-by-one in causality) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoders


def test_e4m3_decode_matches_torch_for_all_codes(oracle_lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle_lib.e4m3_to_double(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), (c, got, ref[c])


def test_e4m3_spec_values(oracle_lib):
    # OCP E4M3FN: bias 7, max normal 448, min subnormal 2^-9, S.1111.111 = NaN
    d = oracle_lib.e4m3_to_double
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x80) == 0.0 and math.copysign(1, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))


def test_bf16_decode_matches_torch(oracle_lib):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        got = oracle_lib.bf16_to_double(int(b))
        assert (math.isnan(got) and math.isnan(r)) or got == r


# ---------------------------------------------------------------- indexer helpers


def _one_page_table(n_seq, pages_per_seq):
    return np.arange(n_seq * pages_per_seq, dtype=np.int32).reshape(n_seq, pages_per_seq)


def _worked_inputs(coeff, head_w, heads, dims, extra_head=None):
    """Query at 0-based position 7 of one sequence; keys k_j = coeff_j * e_1."""
    T = len(coeff)
    q = np.zeros((1, heads, dims), np.float32)
    q[0, :, 0] = 1.0
    w = np.full((1, heads), head_w, np.float32)
    k = np.zeros((1, 64, dims), np.float32)   # one 64-token page
    k[0, :T, 0] = coeff
    if extra_head is not None:   # (head, weight, {pos: value}) on component 1
        h, wv, comps = extra_head
        q[0, h, :] = 0.0
        q[0, h, 1] = 1.0
        w[0, h] = wv
        for p, v in comps.items():
            k[0, p, 1] = v
    return q, w, k, np.array([T - 1], np.int32)


def _select(oracle_lib, q, w, k, q_pos, kk, fmt=1, k_scale=None):
    pt = _one_page_table(1, k.shape[0])
    s = oracle_lib.indexer_scores(q, w, k, k_scale, pt, 64, q_pos, 1, len(q_pos), fmt, 64 * k.shape[0])
    idx = oracle_lib.topk(s, q_pos, kk)
    return s, idx


def test_worked_example_from_golden(oracle_lib):
    g = _golden()
    q, w, k, q_pos = _worked_inputs(g["key_coeff_by_position_1based"], g["head_weight"], g["heads"], g["dims"])
    s, idx = _select(oracle_lib, q, w, k, q_pos, g["k"])
    # the construction gives I_8j = c_j exactly (4 * 1/4 * c_j)
    np.testing.assert_array_equal(s[0, :8], np.float32(g["key_coeff_by_position_1based"]))
    assert [int(i) + 1 for i in idx[0]] == g["expected_1based"]


def test_worked_example_relu_not_abs(oracle_lib):
    g = _golden()
    c = list(g["key_coeff_by_position_1based"])
    c[0] = -5.0   # largest magnitude, but ReLU clips it to 0
    q, w, k, q_pos = _worked_inputs(c, g["head_weight"], g["heads"], g["dims"])
    s, idx = _select(oracle_lib, q, w, k, q_pos, g["k"])
    assert s[0, 0] == 0.0
    assert [int(i) + 1 for i in idx[0]] == [2, 5, 8]


def test_worked_example_negative_head_weight_demotes(oracle_lib):
    g = _golden()
    c = g["key_coeff_by_position_1based"]
    # head 3 looks at component 1, weight -1; only position 5 (1-based) has that component
    q, w, k, q_pos = _worked_inputs(c, g["head_weight"], g["heads"], g["dims"], extra_head=(3, -1.0, {4: 1.0}))
    s, idx = _select(oracle_lib, q, w, k, q_pos, g["k"])
    expect = [0.75 * x for x in c]
    expect[4] -= 1.0
    np.testing.assert_allclose(s[0, :8], expect, rtol=1e-6)
    assert [int(i) + 1 for i in idx[0]] == [2, 7, 8]


def test_worked_example_causality_excludes_future(oracle_lib):
    # the same query at position 8 (1-based) must not see a huge score at position 9
    g = _golden()
    c = list(g["key_coeff_by_position_1based"]) + [100.0]
    q, w, k, _ = _worked_inputs(c, g["head_weight"], g["heads"], g["dims"])
    s, idx = _select(oracle_lib, q, w, k, np.array([7], np.int32), g["k"])
    assert [int(i) + 1 for i in idx[0]] == [2, 5, 8]


def _np_scores(q, w, keys_by_pos, q_pos, q_per_seq, seq_keys):
    out = {}
    for r in range(q.shape[0]):
        s = r // q_per_seq
        K = seq_keys[s][: q_pos[r] + 1]                                      # [t+1, Di]
        dots = np.einsum("hd,jd->hj", q[r].astype(np.float64), K)            # [Hi, t+1]
        out[r] = np.einsum("h,hj->j", w[r].astype(np.float64), np.maximum(dots, 0.0))
    return out


def test_indexer_f32_matches_numpy_einsum_with_permuted_pages(oracle_lib):
    rng = np.random.default_rng(1)
    n_seq, qps, Hi, Di, ps = 2, 3, 5, 12, 64
    pps = 3
    P = n_seq * pps + 2
    perm = rng.permutation(P)[: n_seq * pps].astype(np.int32).reshape(n_seq, pps)
    k_cache = rng.standard_normal((P, ps, Di)).astype(np.float32)
    q = rng.standard_normal((n_seq * qps, Hi, Di)).astype(np.float32)
    w = rng.standard_normal((n_seq * qps, Hi)).astype(np.float32)
    q_pos = np.array([0, 70, 191, 5, 64, 150], np.int32)
    s = oracle_lib.indexer_scores(q, w, k_cache, None, perm, ps, q_pos, n_seq, qps, 1, 192)
    seq_keys = [np.concatenate([k_cache[perm[b, p]] for p in range(pps)]).astype(np.float64) for b in range(n_seq)]
    ref = _np_scores(q, w, None, q_pos, qps, seq_keys)
    for r, v in ref.items():
        np.testing.assert_allclose(s[r, : q_pos[r] + 1], v.astype(np.float32), rtol=2e-6, atol=1e-6)
        assert np.isnan(s[r, q_pos[r] + 1:]).all()      # nothing written past the visible prefix


def test_indexer_e4m3_matches_torch_decode_and_einsum(oracle_lib):
    w = workloads.make_random(1, 2, [100, 127], 128, Hi=8, Di=32, H=2, Dqk=16, Dv=8, seed=7)
    s = oracle_lib.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, 64, w.q_pos, 1, 2, 0, 128)
    dec = lambda b: torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    keys = dec(w.ik).reshape(-1, 32) * w.iks.reshape(-1, 1).astype(np.float64)
    qd = dec(w.iq)
    ref = _np_scores(qd, w.iw, None, w.q_pos, 2, [keys])
    for r, v in ref.items():
        np.testing.assert_allclose(s[r, : w.q_pos[r] + 1], v.astype(np.float32), rtol=1e-6, atol=1e-7)


def test_indexer_key_scale_homogeneity_exact(oracle_lib):
    # ReLU is positively homogeneous: scaling one key's scale by 4 scales its score by exactly 4
    w = workloads.make_random(1, 1, [63], 64, Hi=8, Di=32, H=2, Dqk=16, Dv=8, seed=9)
    s1 = oracle_lib.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, 64, w.q_pos, 1, 1, 0, 64)
    ks = w.iks.copy()
    ks[0, 10] *= 4.0
    s2 = oracle_lib.indexer_scores(w.iq, w.iw, w.ik, ks, w.page_table, 64, w.q_pos, 1, 1, 0, 64)
    assert s2[0, 10] == np.float32(4.0) * s1[0, 10]
    others = [j for j in range(64) if j != 10]
    np.testing.assert_array_equal(s2[0, others], s1[0, others])


# ---------------------------------------------------------------- top-k


def _rank_key(v, j):
    return (-v, j)


def test_topk_brute_force_small_rows_with_ties(oracle_lib):
    rng = np.random.default_rng(2)
    values = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 13))
        sc = rng.choice(values, size=n).astype(np.float32)
        row = np.full((1, 16), np.nan, np.float32)
        row[0, :n] = sc
        idx = oracle_lib.topk(row, np.array([n - 1], np.int32), k)[0]
        m = min(k, n)
        # brute force: the unique m-subset whose members all outrank (value desc, position asc)
        # every non-member
        winners = []
        for sub in itertools.combinations(range(n), m):
            rest = [j for j in range(n) if j not in sub]
            if all(_rank_key(float(sc[a]), a) < _rank_key(float(sc[b]), b) for a in sub for b in rest):
                winners.append(sub)
        assert len(winners) == 1
        assert list(idx[:m]) == list(winners[0])
        assert list(idx[m:]) == [-1] * (k - m)


def test_topk_values_match_torch_topk(oracle_lib):
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((3, 5000)).astype(np.float32)
    q_pos = np.array([4999, 3000, 100], np.int32)
    idx = oracle_lib.topk(sc, q_pos, 512)
    for r in range(3):
        n = q_pos[r] + 1
        m = min(512, n)
        ref = torch.topk(torch.from_numpy(sc[r, :n]), m).values.numpy()
        got = np.sort(sc[r, idx[r, :m]])[::-1]
        np.testing.assert_array_equal(got, ref)
        assert (np.diff(idx[r, :m]) > 0).all()       # ascending, no duplicates


def test_topk_short_prefix_keeps_everything(oracle_lib):
    sc = np.random.default_rng(4).standard_normal((2, 64)).astype(np.float32)
    idx = oracle_lib.topk(sc, np.array([9, 0], np.int32), 32)
    assert list(idx[0, :10]) == list(range(10)) and (idx[0, 10:] == -1).all()
    assert idx[1, 0] == 0 and (idx[1, 1:] == -1).all()


def test_topk_signed_zero_ties_by_position(oracle_lib):
    sc = np.array([[0.0, -0.0, 0.0, -0.0, -1.0, 0.0]], np.float32)
    idx = oracle_lib.topk(sc, np.array([5], np.int32), 3)
    assert list(idx[0]) == [0, 1, 2]


# ---------------------------------------------------------------- attention


def _bf16(x):
    return workloads.bf16_bits(torch.as_tensor(x, dtype=torch.float32))


def _dec_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _attn_case(seed=5, rows=4, H=3, Dqk=16, Dv=8, kv_dim=24, v_col0=8, T=100):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((rows, H, Dqk)))
    kv = _bf16(rng.standard_normal((2, 64, kv_dim)))
    pt = np.array([[1, 0]], np.int32)         # non-identity paging
    q_pos = np.array(sorted(rng.integers(0, T, rows)), np.int32)
    return q, kv, pt, q_pos


def _rows_of(kv, pt, n):
    flat = kv.reshape(-1, kv.shape[-1])
    return np.stack([flat[pt[0, p // 64] * 64 + p % 64] for p in range(n)])


def test_sparse_attention_matches_torch_sdpa_with_mask(oracle_lib):
    q, kv, pt, q_pos = _attn_case()
    rows, H, Dqk = q.shape
    Dv, v0, T = 8, 8, 128
    rng = np.random.default_rng(6)
    k = 12
    idx = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        m = min(k, q_pos[r] + 1)
        idx[r, :m] = np.sort(rng.choice(q_pos[r] + 1, m, replace=False))
    scale = 0.37
    out, lse = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, idx, Dqk, Dv, v0, scale)
    allrows = _dec_bf16(_rows_of(kv, pt, T))                          # [T, kv_dim]
    K, V = allrows[:, :Dqk], allrows[:, v0: v0 + Dv]
    Q = _dec_bf16(q)                                                  # [rows, H, Dqk]
    mask = torch.zeros(rows, T, dtype=torch.bool)
    for r in range(rows):
        for j in idx[r]:
            if j >= 0:
                mask[r, j] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1), K.expand(H, T, Dqk), V.expand(H, T, Dv),
        attn_mask=mask.unsqueeze(0).expand(H, rows, T), scale=scale).transpose(0, 1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-6, atol=1e-6)
    logits = scale * torch.einsum("rhd,jd->rhj", Q, K)
    ref_lse = torch.logsumexp(logits.masked_fill(~mask.unsqueeze(1), -math.inf), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-6, atol=1e-6)


def test_dense_attention_matches_torch_sdpa_causal(oracle_lib):
    q, kv, pt, q_pos = _attn_case(seed=8)
    rows, H, Dqk = q.shape
    out, lse = oracle_lib.dense_mla(q, kv, pt, 64, q_pos, 1, rows, Dqk, 8, 8, 0.25)
    T = 128
    allrows = _dec_bf16(_rows_of(kv, pt, T))
    K, V = allrows[:, :Dqk], allrows[:, 8:16]
    Q = _dec_bf16(q)
    mask = torch.arange(T).unsqueeze(0) <= torch.from_numpy(q_pos).long().unsqueeze(1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1), K.expand(H, T, Dqk), V.expand(H, T, 8),
        attn_mask=mask.unsqueeze(0).expand(H, rows, T), scale=0.25).transpose(0, 1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-6, atol=1e-6)


def test_sparse_with_full_set_equals_dense_bitwise(oracle_lib):
    # k >= t: DSA is dense causal attention (the handbook's k = min(L, 2048))
    q, kv, pt, q_pos = _attn_case(seed=10)
    rows, H, Dqk = q.shape
    k = 128
    idx = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        idx[r, : q_pos[r] + 1] = np.arange(q_pos[r] + 1)
    o1, l1 = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, idx, Dqk, 8, 8, 0.3)
    o2, l2 = oracle_lib.dense_mla(q, kv, pt, 64, q_pos, 1, rows, Dqk, 8, 8, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_sparse_single_position_returns_its_value_row(oracle_lib):
    q, kv, pt, q_pos = _attn_case(seed=11)
    rows, H, Dqk = q.shape
    idx = np.full((rows, 4), -1, np.int32)
    idx[:, 0] = q_pos // 2
    out, lse = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, idx, Dqk, 8, 8, 0.5)
    allrows = _dec_bf16(_rows_of(kv, pt, 128)).numpy()
    Q = _dec_bf16(q).numpy()
    for r in range(rows):
        j = idx[r, 0]
        np.testing.assert_array_equal(out[r], np.broadcast_to(allrows[j, 8:16].astype(np.float32), (H, 8)))
        np.testing.assert_allclose(lse[r], 0.5 * Q[r] @ allrows[j, :Dqk], rtol=1e-6)


def test_sparse_zero_query_averages_values(oracle_lib):
    q, kv, pt, q_pos = _attn_case(seed=12)
    q[:] = 0
    rows, H, Dqk = q.shape
    idx = np.full((rows, 6), -1, np.int32)
    for r in range(rows):
        m = min(6, q_pos[r] + 1)
        idx[r, :m] = np.arange(q_pos[r] + 1 - m, q_pos[r] + 1)
    out, lse = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, idx, Dqk, 8, 8, 1.0)
    allrows = _dec_bf16(_rows_of(kv, pt, 128)).numpy()
    for r in range(rows):
        sel = idx[r][idx[r] >= 0]
        np.testing.assert_allclose(out[r], np.broadcast_to(allrows[sel, 8:16].mean(0), (H, 8)), rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(lse[r], math.log(len(sel)), rtol=1e-6)


def test_sparse_ignores_padding_and_invisible_entries(oracle_lib):
    q, kv, pt, q_pos = _attn_case(seed=13)
    rows, H, Dqk = q.shape
    base = np.full((rows, 5), -1, np.int32)
    noisy = np.full((rows, 8), -1, np.int32)
    for r in range(rows):
        sel = np.arange(min(3, q_pos[r] + 1))
        base[r, : len(sel)] = sel
        noisy[r, : len(sel)] = sel
        noisy[r, 5] = q_pos[r] + 1          # a future position is not visible
        noisy[r, 6] = -7
    o1, l1 = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, base, Dqk, 8, 8, 0.3)
    o2, l2 = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, noisy, Dqk, 8, 8, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_sparse_repeated_and_shuffled_entries_are_a_set(oracle_lib):
    """S_t is a set ([DSA-blog] "Sparse Attention": the mask is 0 exactly on S_t): a list that
    repeats positions, in any order and with holes, gives the masked softmax of its distinct
    positions -- torch's float64 SDPA under the boolean mask -- and equals the deduplicated
    ascending list bit for bit. Counting a repeat twice would weight that row double."""
    q, kv, pt, q_pos = _attn_case(seed=15)
    rows, H, Dqk = q.shape
    Dv, v0, T, k = 8, 8, 128, 16
    rng = np.random.default_rng(16)
    rep = np.full((rows, k), -1, np.int32)
    ded = np.full((rows, k), -1, np.int32)
    mask = torch.zeros(rows, T, dtype=torch.bool)
    for r in range(rows):
        m = min(5, q_pos[r] + 1)
        sel = np.sort(rng.choice(q_pos[r] + 1, m, replace=False))
        lst = np.concatenate([sel, sel[: max(1, m // 2)], sel[:1], [-1, q_pos[r] + 3]])
        rng.shuffle(lst)
        rep[r, : len(lst)] = lst
        ded[r, :m] = sel
        mask[r, torch.from_numpy(sel).long()] = True
    assert any(len(set(x[x >= 0].tolist())) < int((x >= 0).sum()) for x in rep)
    o1, l1 = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, rep, Dqk, Dv, v0, 0.41)
    o2, l2 = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, ded, Dqk, Dv, v0, 0.41)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    allrows = _dec_bf16(_rows_of(kv, pt, T))
    K, V = allrows[:, :Dqk], allrows[:, v0: v0 + Dv]
    ref = torch.nn.functional.scaled_dot_product_attention(
        _dec_bf16(q).transpose(0, 1), K.expand(H, T, Dqk), V.expand(H, T, Dv),
        attn_mask=mask.unsqueeze(0).expand(H, rows, T), scale=0.41).transpose(0, 1)
    np.testing.assert_allclose(o1, ref.numpy(), rtol=1e-6, atol=1e-6)


def test_sparse_empty_set(oracle_lib):
    q, kv, pt, q_pos = _attn_case(seed=14)
    rows, H, Dqk = q.shape
    idx = np.full((rows, 4), -1, np.int32)
    out, lse = oracle_lib.sparse_mla(q, kv, pt, 64, q_pos, 1, rows, idx, Dqk, 8, 8, 0.3)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_tiny_workload_end_to_end_invariants(oracle_lib):
    """The tiny prefill workload: every row with t + 1 <= k reproduces dense attention, and the
    selected sets obey the score order."""
    w = workloads.make_tiny()
    s = oracle_lib.indexer_scores(w.iq, w.iw, w.ik, None, w.page_table, 64, w.q_pos, 1, w.rows, 1, w.max_ctx)
    idx = oracle_lib.topk(s, w.q_pos, w.topk)
    out, lse = oracle_lib.sparse_mla(w.q, w.kv, w.page_table, 64, w.q_pos, 1, w.rows, idx, w.Dqk, w.Dv, w.v_col0, w.sm_scale)
    dout, dlse = oracle_lib.dense_mla(w.q, w.kv, w.page_table, 64, w.q_pos, 1, w.rows, w.Dqk, w.Dv, w.v_col0, w.sm_scale)
    short = w.q_pos + 1 <= w.topk
    np.testing.assert_array_equal(out[short], dout[short])
    assert not np.allclose(out[~short], dout[~short])   # sparse differs once the prefix exceeds k
    for r in range(w.rows):
        n = w.q_pos[r] + 1
        sel = idx[r][idx[r] >= 0]
        assert len(sel) == min(n, w.topk)
        if n > w.topk:
            rest = np.setdiff1d(np.arange(n), sel)
            assert s[r, sel].min() >= s[r, rest].max()


# ---------------------------------------------------------------- expanded attention (fallback)


def _mha_case(seed=11, n_seq=2, q_per_seq=3, H=4, Dn=16, Dr=8, Dv=12, T=70):
    rng = np.random.default_rng(seed)
    rows = n_seq * q_per_seq
    q = _bf16(rng.standard_normal((rows, H, Dn + Dr)))
    kn = _bf16(rng.standard_normal((n_seq, H, T, Dn)))
    kr = _bf16(rng.standard_normal((n_seq, T, Dr)))
    v = _bf16(rng.standard_normal((n_seq, H, T, Dv)))
    q_pos = np.concatenate([np.sort(rng.choice(T, q_per_seq, replace=False)) for _ in range(n_seq)]).astype(np.int32)
    return q, kn, kr, v, q_pos


def test_mha_matches_torch_sdpa_per_head_keys(oracle_lib):
    # per-head keys = [nope | shared rope]: torch's float64 attention with the causal mask, and with
    # a random position set (the masked MHA mode)
    q, kn, kr, v, q_pos = _mha_case()
    n_seq, H, T, Dn = kn.shape
    rows, Dv, Dr = q.shape[0], v.shape[3], kr.shape[2]
    qps = rows // n_seq
    rng = np.random.default_rng(3)
    idx = np.full((rows, 9), -1, np.int32)
    for r in range(rows):
        m = min(9, q_pos[r] + 1)
        idx[r, :m] = rng.choice(q_pos[r] + 1, m, replace=False)   # unsorted on purpose
    scale = 0.29
    for use_idx in (False, True):
        out, lse = oracle_lib.mha(q, kn, kr, v, q_pos, n_seq, qps, idx if use_idx else None, scale)
        for r in range(rows):
            s = r // qps
            K = torch.cat([_dec_bf16(kn[s]), _dec_bf16(kr[s]).unsqueeze(0).expand(H, T, Dr)], dim=-1)
            V = _dec_bf16(v[s])
            mask = torch.arange(T) <= int(q_pos[r])
            if use_idx:
                sel = torch.zeros(T, dtype=torch.bool)
                sel[[j for j in idx[r] if j >= 0]] = True
                mask &= sel
            Q = _dec_bf16(q[r]).unsqueeze(1)                              # [H, 1, Dn+Dr]
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q, K, V, attn_mask=mask.view(1, 1, T).expand(H, 1, T), scale=scale)[:, 0]
            np.testing.assert_allclose(out[r], ref.numpy(), rtol=1e-6, atol=1e-6)
            logits = scale * (K @ Q.transpose(1, 2))[:, :, 0]
            ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
            np.testing.assert_allclose(lse[r], ref_lse.numpy(), rtol=1e-6, atol=1e-6)


def test_expanded_equals_absorbed_mla(oracle_lib):
    # [Handbook] cost model: the expanded pair (per-head k = c W_UK, v = c W_UV) and the absorbed
    # pair (q W_UK^T against the latent row, output times W_UV) are the same attention. With
    # W_UK, W_UV made of signed unit columns on distinct latent dims, every product is exact in
    # bf16, so the absorbed oracle (pinned above) and the expanded one must agree to rounding.
    rng = np.random.default_rng(21)
    H, DC, Dn, Dr, Dv, T, rows = 3, 48, 16, 8, 12, 64, 5
    lat = rng.standard_normal((T, DC))
    rope = rng.standard_normal((T, Dr))
    qn = rng.standard_normal((rows, H, Dn))
    qr = rng.standard_normal((rows, H, Dr))
    lat, rope, qn, qr = (_dec_bf16(_bf16(x)).numpy() for x in (lat, rope, qn, qr))
    WUK = np.zeros((H, DC, Dn))
    WUV = np.zeros((H, DC, Dv))
    for h in range(H):
        for d, c in enumerate(rng.choice(DC, Dn, replace=False)):
            WUK[h, c, d] = rng.choice([-1.0, 1.0])
        for d, c in enumerate(rng.choice(DC, Dv, replace=False)):
            WUV[h, c, d] = rng.choice([-1.0, 1.0])
    q_pos = np.sort(rng.choice(T, rows, replace=False)).astype(np.int32)
    idx = np.full((rows, 20), -1, np.int32)
    for r in range(rows):
        m = min(20, q_pos[r] + 1)
        idx[r, :m] = np.sort(rng.choice(q_pos[r] + 1, m, replace=False))
    scale = 1.0 / math.sqrt(Dn + Dr)
    # expanded operands
    q_exp = _bf16(np.concatenate([qn, qr], axis=-1))
    kn = _bf16(np.einsum("jc,hcd->hjd", lat, WUK)[None])
    kr = _bf16(rope[None])
    v = _bf16(np.einsum("jc,hcd->hjd", lat, WUV)[None])
    # absorbed operands: one latent row [c | rope] per position, q_abs = [qn W_UK^T | qr]
    q_abs = _bf16(np.concatenate([np.einsum("rhd,hcd->rhc", qn, WUK), qr], axis=-1))
    kv = _bf16(np.concatenate([lat, rope], axis=-1).reshape(1, T, DC + Dr))
    pt = np.zeros((1, 1), np.int32)
    for use_idx in (False, True):
        if use_idx:
            o_abs, lse_abs = oracle_lib.sparse_mla(q_abs, kv, pt, T, q_pos, 1, rows, idx, DC + Dr, DC, 0, scale)
        else:
            o_abs, lse_abs = oracle_lib.dense_mla(q_abs, kv, pt, T, q_pos, 1, rows, DC + Dr, DC, 0, scale)
        o_exp, lse_exp = oracle_lib.mha(q_exp, kn, kr, v, q_pos, 1, rows, idx if use_idx else None, scale)
        np.testing.assert_allclose(o_exp, np.einsum("rhc,hcd->rhd", o_abs.astype(np.float64), WUV),
                                   rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(lse_exp, lse_abs, rtol=1e-6, atol=1e-6)


def test_mha_full_index_set_equals_dense_bitwise(oracle_lib):
    q, kn, kr, v, q_pos = _mha_case(seed=13)
    rows = q.shape[0]
    n_seq = kn.shape[0]
    T = kn.shape[2]
    idx = np.full((rows, T + 3), -1, np.int32)
    for r in range(rows):
        idx[r, :q_pos[r] + 1] = np.arange(q_pos[r], -1, -1)      # every visible position, reversed
        idx[r, q_pos[r] + 1: q_pos[r] + 3] = 0                    # repeats count once
    dense = oracle_lib.mha(q, kn, kr, v, q_pos, n_seq, rows // n_seq, None, 0.2)
    full = oracle_lib.mha(q, kn, kr, v, q_pos, n_seq, rows // n_seq, idx, 0.2)
    assert np.array_equal(dense[0], full[0]) and np.array_equal(dense[1], full[1])


def test_mha_single_position_and_empty_set(oracle_lib):
    q, kn, kr, v, q_pos = _mha_case(seed=17, n_seq=1, q_per_seq=4)
    rows = q.shape[0]
    idx = np.full((rows, 3), -1, np.int32)
    idx[:, 0] = q_pos // 2
    idx[:, 1] = q_pos + 1                   # invisible: ignored
    out, lse = oracle_lib.mha(q, kn, kr, v, q_pos, 1, rows, idx, 0.5)
    for r in range(rows):
        np.testing.assert_array_equal(out[r], _dec_bf16(v[0, :, q_pos[r] // 2]).numpy().astype(np.float32))
    idx[:] = -1
    out, lse = oracle_lib.mha(q, kn, kr, v, q_pos, 1, rows, idx, 0.5)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- FP8 quantisation, cache writes


def _e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    return {c: float(vals[c]) for c in range(256) if not math.isnan(vals[c])}


def test_e4m3_encode_round_trips_every_code(oracle_lib):
    for c, v in _e4m3_values().items():
        got = oracle_lib.e4m3_from_float(v)
        if v == 0.0:   # +0 and -0 both decode to zero; the sign bit follows the input's sign
            assert got == (0x80 if math.copysign(1, v) < 0 else 0x00)
        else:
            assert got == c, (hex(c), v, hex(got))


def test_e4m3_encode_ties_to_even_and_saturates(oracle_lib):
    vals = sorted((v, c) for c, v in _e4m3_values().items() if v > 0)
    for (v0, c0), (v1, c1) in zip(vals, vals[1:]):
        mid = np.float32((v0 + v1) / 2)           # exactly representable: one more mantissa bit
        assert float(mid) == (v0 + v1) / 2
        want = c0 if (c0 & 1) == 0 else c1
        assert oracle_lib.e4m3_from_float(float(mid)) == want, (v0, v1)
        assert oracle_lib.e4m3_from_float(-float(mid)) == (want | 0x80)
        assert oracle_lib.e4m3_from_float(float(np.nextafter(mid, np.float32(0)))) == c0
        assert oracle_lib.e4m3_from_float(float(np.nextafter(mid, np.float32(1e9)))) == c1
    for big in (448.0, 448.0001, 463.9, 464.0, 480.0, 1e6, 3.0e38):
        assert oracle_lib.e4m3_from_float(big) == 0x7E
        assert oracle_lib.e4m3_from_float(-big) == 0xFE


def test_e4m3_quantize_matches_torch_in_range(oracle_lib):
    rng = np.random.default_rng(31)
    mag = np.exp2(rng.uniform(-12, 8.8, 200000)).astype(np.float32)
    x = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = oracle_lib.e4m3_quantize(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_indexer_cache_write_matches_torch_quantiser_and_pages(oracle_lib):
    # the per-token quantiser against an independent torch statement of it (s = max|k|/448 and
    # k/s in float32, torch's E4M3 rounding), written through a permuted page table; rows of
    # other positions stay untouched and a token without a valid page is skipped
    rng = np.random.default_rng(33)
    n_seq, pages, Di = 2, 3, 128
    pt = rng.permutation(n_seq * pages + 1)[: n_seq * pages].astype(np.int32).reshape(n_seq, pages)
    P = n_seq * pages + 1
    n_tok = 50
    seq = rng.integers(0, n_seq, n_tok).astype(np.int32)
    pos = rng.choice(pages * 64, n_tok, replace=False).astype(np.int32)
    k = (rng.standard_normal((n_tok, Di)) * np.exp2(rng.uniform(-8, 8, (n_tok, 1)))).astype(np.float32)
    k[3] = 0.0                                        # a zero key: scale 0, codes 0
    pos_bad = pos.copy()
    pos_bad[7] = pages * 64 + 5                       # past the page table: skipped
    cache = np.full((P, 64, Di), 0xAB, np.uint8)
    scale = np.full((P, 64), -1.0, np.float32)
    skipped = oracle_lib.indexer_cache_write(k, seq, pos_bad, pt, 64, cache, scale)
    assert skipped == 1
    kt = torch.from_numpy(k)
    s = kt.abs().amax(dim=1) / 448.0
    ref = torch.where(s[:, None] > 0, kt / torch.where(s > 0, s, torch.ones_like(s))[:, None], torch.zeros_like(kt))
    ref8 = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    written = set()
    for t in range(n_tok):
        if t == 7:
            continue
        r = pt[seq[t], pos[t] // 64] * 64 + pos[t] % 64
        written.add(int(r))
        np.testing.assert_array_equal(cache.reshape(-1, Di)[r], ref8[t])
        assert scale.reshape(-1)[r] == s[t].item()
    for r in range(P * 64):
        if r not in written:
            assert (cache.reshape(-1, Di)[r] == 0xAB).all() and scale.reshape(-1)[r] == -1.0
    # bf16 input: the same as float input of the bf16 values
    kb = workloads.bf16_bits(kt)
    c2 = np.zeros_like(cache)
    s2 = np.zeros_like(scale)
    oracle_lib.indexer_cache_write(kb, seq, pos, pt, 64, c2, s2)
    c3 = np.zeros_like(cache)
    s3 = np.zeros_like(scale)
    oracle_lib.indexer_cache_write(_dec_bf16(kb).to(torch.float32).numpy(), seq, pos, pt, 64, c3, s3)
    np.testing.assert_array_equal(c2, c3)
    np.testing.assert_array_equal(s2, s3)


def test_latent_cache_write_places_rows(oracle_lib):
    rng = np.random.default_rng(35)
    pt = np.array([[2, 0], [1, 3]], np.int32)
    rows = rng.integers(0, 65535, (7, 576)).astype(np.uint16)
    seq = np.array([0, 0, 1, 1, 0, 1, 2], np.int32)
    pos = np.array([0, 70, 5, 127, 63, 200, 1], np.int32)   # the last two: no page, no sequence
    cache = np.zeros((4, 64, 576), np.uint16)
    assert oracle_lib.latent_cache_write(rows, seq, pos, pt, 64, cache) == 2
    flat = cache.reshape(-1, 576)
    for t in range(5):
        r = pt[seq[t], pos[t] // 64] * 64 + pos[t] % 64
        np.testing.assert_array_equal(flat[r], rows[t])
    assert np.count_nonzero(flat.any(axis=1)) == 5


# ---------------------------------------------------------------- the indexer's projections


def _bf16_rand(rng, *shape, scale=1.0):
    return workloads.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)))


def _f64_linear(x_bits, w_bits):
    # a linear layer with [out, in] weights, in float64 (a library matmul), rounded once to float32
    return (_dec_bf16(x_bits) @ _dec_bf16(w_bits).T).to(torch.float32).numpy()


def test_key_projection_is_a_linear_layer_then_the_cache_write(oracle_lib):
    """[DSA-blog] "Lightning Indexer": k_j from h_j. The oracle's keys equal torch's float64 matmul
    rounded to float32 (within one ulp: the two sum in different orders), and what lands in the
    paged cache equals the oracle's cache write of those keys (pinned against torch's FP8 codes)."""
    rng = np.random.default_rng(31)
    n_tok, d = 37, 192
    h = _bf16_rand(rng, n_tok, d)
    w_k = _bf16_rand(rng, 128, d, scale=1 / math.sqrt(d))
    seq = np.zeros(n_tok, np.int32)
    pos = rng.permutation(n_tok).astype(np.int32)
    pt = np.array([[2, 0, 1]], np.int32)
    kc = np.full((3, 64, 128), 0xAA, np.uint8)
    ks = np.full((3, 64), -1.0, np.float32)
    k, skipped = oracle_lib.indexer_key_project(h, w_k, seq, pos, pt, 64, kc, ks)
    assert skipped == 0
    ref = _f64_linear(h, w_k)
    np.testing.assert_array_max_ulp(k, ref, maxulp=1)
    kc2 = np.full_like(kc, 0xAA)
    ks2 = np.full_like(ks, -1.0)
    oracle_lib.indexer_cache_write(k, seq, pos, pt, 64, kc2, ks2)
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(ks, ks2)
    # a transposed weight or a dropped term would move the keys far beyond one ulp
    assert not np.allclose(k, _f64_linear(h[:, ::-1].copy(), w_k), rtol=1e-3)


def test_query_projection_codes_and_head_weights(oracle_lib):
    """[DSA-blog] "Lightning Indexer": the query heads from the MLA query latent, the head weights
    from h_t. q before coding and w equal torch's float64 matmuls rounded to float32 (one ulp), and
    the codes equal torch's float8_e4m3fn conversion of q (every |q| here is below 448)."""
    rng = np.random.default_rng(32)
    rows, d_cq, d, Hi, Di = 9, 128, 192, 4, 32
    c_q = _bf16_rand(rng, rows, d_cq)
    w_q = _bf16_rand(rng, Hi * Di, d_cq, scale=1 / math.sqrt(d_cq))
    h = _bf16_rand(rng, rows, d)
    w_w = _bf16_rand(rng, Hi, d, scale=1 / math.sqrt(d))
    q8, w, q = oracle_lib.indexer_query_project(c_q, w_q, h, w_w, Hi, Di)
    np.testing.assert_array_max_ulp(q.reshape(rows, -1), _f64_linear(c_q, w_q), maxulp=1)
    np.testing.assert_array_max_ulp(w, _f64_linear(h, w_w), maxulp=1)
    assert np.abs(q).max() < 448
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q8, codes)
