"""The indexer's projections on the GPU (dsa_indexer_key_project, dsa_indexer_query_project)
against the oracle.

Tolerances, from the arithmetic (the pages fix no precision for these projections): the GPU sums
K products of bf16 values, each exact in fp32, in fp32; any order of K fp32 additions stays within
gamma_K = K * 2^-24 of the sum of |products| (the recursive-summation bound), so
  w (fp32 out)   |w_gpu - w_ref| <= gamma_K * sum_c |h_c w_c|
  q8, key codes  each GPU code is the E4M3 coding of some value within that bound of the oracle's
                 value (x = q, or k / s for keys, whose scale s carries the bound of the row's
                 largest |k|); where the oracle's value is farther than that from a rounding
                 boundary the codes are equal
  key scale      |s_gpu - s_ref| <= bound of the row's largest |k| / 448 (+ one fp32 rounding)
Shapes: the pages' hidden size d = 7168 ([Handbook]'s per-token hidden width), a query latent of
1536 (a width the pages do not give; the kernels take any multiple of 64), 64 heads x 128 dims;
ragged row counts, a permuted page table, and tokens with no page (skipped, their rows untouched).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_06_amd import dsa

pytestmark = pytest.mark.gpu

THREADS = 8
E4M3_VALUES = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _sum_abs(x_bits, w_bits):
    """sum_c |x[i, c] w[o, c]| in float64 (a library matmul of absolute values)."""
    dec = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64)  # noqa: E731
    return (dec(x_bits).abs() @ dec(w_bits).abs().T).numpy()


def _codes_within(gpu_codes, x, delta):
    """Every GPU code decodes between the codings of x - delta and x + delta (E4M3 rounding is
    monotone). Returns the share of codes equal to the coding of x itself."""
    x = np.asarray(x, np.float64)
    lo = oracle.e4m3_quantize((x - delta).astype(np.float32))
    hi = oracle.e4m3_quantize((x + delta).astype(np.float32))
    v, vlo, vhi = E4M3_VALUES[gpu_codes], E4M3_VALUES[lo], E4M3_VALUES[hi]
    bad = ~((v >= vlo) & (v <= vhi))
    assert not bad.any(), f"{int(bad.sum())} codes outside the band, e.g. x={x[bad][:4]} gpu={v[bad][:4]}"
    return float((gpu_codes == oracle.e4m3_quantize(x.astype(np.float32))).mean())


def _case(seed, rows, d, d_cq, Hi=64, Di=128):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    h = torch.randn(rows, d, generator=g, device="cuda").to(torch.bfloat16)
    c_q = torch.randn(rows, d_cq, generator=g, device="cuda").to(torch.bfloat16)
    w_k = (torch.randn(Di, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    w_q = (torch.randn(Hi * Di, d_cq, generator=g, device="cuda") / d_cq ** 0.5).to(torch.bfloat16)
    w_w = (torch.randn(Hi, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    return h, c_q, w_k, w_q, w_w


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("rows,d,d_cq", [(131, 7168, 1536), (64, 128, 64), (1, 7168, 1536), (600, 7168, 1536),
                                         (3900, 7168, 512)])
def test_query_projection(oracle_lib, rows, d, d_cq, split):
    """Small batches take 32-row tiles and, with a workspace, a split-K head-weight projection;
    600 and 3900 rows take 128-row tiles (the last one ragged); 3900 rows with a workspace split
    the head-weight projection's K eight ways."""
    print(f"case: query projection rows={rows} d={d} d_cq={d_cq} split={split}", flush=True)
    h, c_q, w_k, w_q, w_w = _case(300 + rows, rows, d, d_cq)
    q8, w = dsa.indexer_query_project(c_q, w_q, h, w_w, 64, 128, ws=None if split else False)
    assert dsa.last_path() == "project"
    torch.cuda.synchronize()
    ref_q8, ref_w, ref_q = oracle.indexer_query_project(_bits(c_q), _bits(w_q), _bits(h), _bits(w_w), 64, 128,
                                                        threads=THREADS)
    bound_w = d * 2.0 ** -24 * _sum_abs(_bits(h), _bits(w_w))
    err_w = np.abs(w.cpu().numpy().astype(np.float64) - ref_w)
    assert (err_w <= bound_w).all(), f"w: max err / bound {np.max(err_w / bound_w):.3f}"
    bound_q = d_cq * 2.0 ** -24 * _sum_abs(_bits(c_q), _bits(w_q)).reshape(rows, 64, 128)
    same = _codes_within(q8.cpu().numpy(), ref_q, bound_q)
    print(f"query codes equal to the oracle's: {same:.6f}; w max err / bound {np.max(err_w / bound_w):.3e}", flush=True)


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("n_tok,d", [(300, 7168), (37, 128), (130, 7168)])
def test_key_projection_into_paged_cache(oracle_lib, n_tok, d, split):
    """With a workspace, these small token counts split K over workgroups (partial sums, then the
    quantising reduction); without one a single launch quantises in its epilogue."""
    print(f"case: key projection n_tok={n_tok} d={d} split={split}", flush=True)
    h, _, w_k, _, _ = _case(400 + n_tok, n_tok, d, 64)
    rng = np.random.default_rng(n_tok)
    n_seq, pps = 3, 3
    P = n_seq * pps + 2
    pt = rng.permutation(P)[: n_seq * pps].astype(np.int32).reshape(n_seq, pps)
    seq = rng.integers(0, n_seq, n_tok).astype(np.int32)
    pos = rng.integers(0, 64 * pps, n_tok).astype(np.int32)
    # one token per (sequence, position): duplicates would write one row twice
    _, first = np.unique(seq.astype(np.int64) * 100000 + pos, return_index=True)
    keep = np.zeros(n_tok, bool)
    keep[first] = True
    seq[~keep] = -1                      # no such sequence: skipped
    pos[n_tok // 2] = 64 * pps + 7       # past the page table: skipped
    kc = torch.full((P, 64, 128), 0xAA, dtype=torch.uint8, device="cuda")
    ks = torch.full((P, 64), -1.0, dtype=torch.float32, device="cuda")
    dsa.indexer_key_project(h, w_k, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                            torch.from_numpy(pt).cuda(), kc, ks, ws=None if split else False)
    assert dsa.last_path() == "project"
    torch.cuda.synchronize()
    ref_kc = np.full((P, 64, 128), 0xAA, np.uint8)
    ref_ks = np.full((P, 64), -1.0, np.float32)
    ref_k, skipped = oracle.indexer_key_project(_bits(h), _bits(w_k), seq, pos, pt, 64, ref_kc, ref_ks)
    assert skipped == int((seq < 0).sum()) + (1 if seq[n_tok // 2] >= 0 else 0)
    kc_h, ks_h = kc.cpu().numpy(), ks.cpu().numpy()
    written = ref_ks != -1.0
    np.testing.assert_array_equal(kc_h[~written], ref_kc[~written])   # untouched rows stay untouched
    np.testing.assert_array_equal(ks_h[~written], ref_ks[~written])
    bound = d * 2.0 ** -24 * _sum_abs(_bits(h), _bits(w_k))            # per (token, column)
    # written tokens, in the oracle's order of their rows
    toks = [t for t in range(n_tok) if seq[t] >= 0 and pos[t] < 64 * pps]
    rows = [int(pt[seq[t], pos[t] // 64]) * 64 + pos[t] % 64 for t in toks]
    # the row's largest |k| moves by at most the largest bound of its columns
    kmax_bound = bound[toks].max(axis=1)
    kmax = np.maximum(np.abs(ref_k[toks]).max(axis=1), 1e-30)
    s_ref = ref_ks.reshape(-1)[rows].astype(np.float64)
    s_gpu = ks_h.reshape(-1)[rows].astype(np.float64)
    assert (np.abs(s_gpu - s_ref) <= kmax_bound / 448 + 2.0 ** -23 * s_ref).all()
    # GPU value k_gpu / s_gpu against x = k_ref / s_ref: the key's own bound over s, the scale's
    # relative error times |x|, and the two divisions' roundings
    x = ref_k[toks] / s_ref[:, None]
    delta = 1.001 * (bound[toks] / s_ref[:, None] + np.abs(x) * (kmax_bound / kmax)[:, None]) + np.abs(x) * 2.0 ** -22
    same = _codes_within(kc_h.reshape(-1, 128)[rows], x, delta)
    print(f"key codes equal to the oracle's: {same:.6f}", flush=True)


def _check_key_rows(kc_h, ks_h, rows, h_bits, w_bits, ref_k, ref_ks_rows):
    """The scale and codes the GPU wrote at `rows` (one per sampled token, in order) against the
    oracle's values for those tokens, within the fp32 summation bound (see the module notes)."""
    d = h_bits.shape[1]
    bound = d * 2.0 ** -24 * _sum_abs(h_bits, w_bits)
    kmax_bound = bound.max(axis=1)
    kmax = np.maximum(np.abs(ref_k).max(axis=1), 1e-30)
    s_ref = ref_ks_rows.astype(np.float64)
    s_gpu = ks_h.reshape(-1)[rows].astype(np.float64)
    assert (np.abs(s_gpu - s_ref) <= kmax_bound / 448 + 2.0 ** -23 * s_ref).all()
    x = ref_k / s_ref[:, None]
    delta = 1.001 * (bound / s_ref[:, None] + np.abs(x) * (kmax_bound / kmax)[:, None]) + np.abs(x) * 2.0 ** -22
    return _codes_within(kc_h.reshape(-1, 128)[rows], x, delta)


def test_projections_at_the_benchmark_sizes(oracle_lib):
    """The launch configurations the projection benchmark times, at its sizes, on sampled rows:
    the key projection of a 131072-token prefix (128-row tiles, no workspace) and of a
    4096-token chunk (K split eight ways), through a permuted 64-token page table, and the query
    projection of a 4096-row chunk (query codes on 128-row tiles, head weights split eight ways).
    Sampled: the first and last tokens / rows and seeded ones between."""
    print("case: projections at the benchmark sizes", flush=True)
    d, d_cq, Hi, Di, page, n = 7168, 1536, 64, 128, 64, 131072
    g = torch.Generator(device="cuda")
    g.manual_seed(0xD5A1)
    w_k = (torch.randn(Di, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    w_q = (torch.randn(Hi * Di, d_cq, generator=g, device="cuda") / d_cq ** 0.5).to(torch.bfloat16)
    w_w = (torch.randn(Hi, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    h = torch.randn(n, d, generator=g, device="cuda").to(torch.bfloat16)
    pt = torch.randperm(n // page, generator=g, device="cuda").to(torch.int32).view(1, -1)
    seq = torch.zeros(n, dtype=torch.int32, device="cuda")
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(7)
    pt_h = pt.cpu().numpy()
    wk_bits = _bits(w_k)
    for nk, ws in ((n, False), (4096, None)):
        kc = torch.full((n // page, page, Di), 0xAA, dtype=torch.uint8, device="cuda")
        ks = torch.full((n // page, page), -1.0, dtype=torch.float32, device="cuda")
        dsa.indexer_key_project(h[:nk], w_k, seq[:nk], pos[:nk], pt, kc, ks, ws=ws)
        torch.cuda.synchronize()
        toks = np.unique(np.concatenate([np.arange(4), np.arange(nk - 4, nk), rng.integers(0, nk, 40)]))
        h_bits = _bits(h[torch.from_numpy(toks).cuda()])
        ref_kc = np.zeros((n // page, page, Di), np.uint8)
        ref_ks = np.full((n // page, page), -1.0, np.float32)
        ref_k, skipped = oracle.indexer_key_project(h_bits, wk_bits, np.zeros(toks.size, np.int32),
                                                    toks.astype(np.int32), pt_h, page, ref_kc, ref_ks)
        assert skipped == 0
        rows = [int(pt_h[0, t // page]) * page + t % page for t in toks]
        kc_h, ks_h = kc.cpu().numpy(), ks.cpu().numpy()
        same = _check_key_rows(kc_h, ks_h, rows, h_bits, wk_bits, ref_k, ref_ks.reshape(-1)[rows])
        assert int((ks_h != -1.0).sum()) == nk  # every token has a page: one scale written per token
        print(f"key projection of {nk} tokens: codes equal to the oracle's {same:.6f}", flush=True)
    rows_q = 4096
    c_q = torch.randn(rows_q, d_cq, generator=g, device="cuda").to(torch.bfloat16)
    q8, w = dsa.indexer_query_project(c_q, w_q, h[:rows_q], w_w, Hi, Di)
    assert dsa.last_path() == "project"
    torch.cuda.synchronize()
    r = np.unique(np.concatenate([np.arange(4), np.arange(rows_q - 4, rows_q), rng.integers(0, rows_q, 24)]))
    ri = torch.from_numpy(r).cuda()
    cq_bits, h_bits = _bits(c_q[ri]), _bits(h[:rows_q][ri])
    ref_q8, ref_w, ref_q = oracle.indexer_query_project(cq_bits, _bits(w_q), h_bits, _bits(w_w), Hi, Di, threads=THREADS)
    bound_w = d * 2.0 ** -24 * _sum_abs(h_bits, _bits(w_w))
    err_w = np.abs(w[ri].cpu().numpy().astype(np.float64) - ref_w)
    assert (err_w <= bound_w).all(), f"w: max err / bound {np.max(err_w / bound_w):.3f}"
    bound_q = d_cq * 2.0 ** -24 * _sum_abs(cq_bits, _bits(w_q)).reshape(r.size, Hi, Di)
    same = _codes_within(q8[ri].cpu().numpy(), ref_q, bound_q)
    print(f"query projection of {rows_q} rows: codes equal to the oracle's {same:.6f}", flush=True)


@pytest.mark.parametrize("rows,Hi,Di", [(5, 3, 16), (700, 3, 16), (300, 5, 32)])
def test_query_projection_narrow_heads(oracle_lib, rows, Hi, Di):
    """Query widths that end inside a 128-column tile (48 and 160 columns): the tile's missing
    columns re-read the last weight row and are never stored; head-weight widths of 3 and 5."""
    print(f"case: narrow query projection rows={rows} Hi={Hi} Di={Di}", flush=True)
    d, d_cq = 192, 128
    h, c_q, _, w_q, w_w = _case(700 + rows + Hi, rows, d, d_cq, Hi=Hi, Di=Di)
    q8 = torch.full((rows, Hi, Di), 0x5A, dtype=torch.uint8, device="cuda")
    q8, w = dsa.indexer_query_project(c_q, w_q, h, w_w, Hi, Di, q8=q8)
    torch.cuda.synchronize()
    ref_q8, ref_w, ref_q = oracle.indexer_query_project(_bits(c_q), _bits(w_q), _bits(h), _bits(w_w), Hi, Di,
                                                        threads=THREADS)
    bound_w = d * 2.0 ** -24 * _sum_abs(_bits(h), _bits(w_w))
    assert (np.abs(w.cpu().numpy().astype(np.float64) - ref_w) <= bound_w).all()
    bound_q = d_cq * 2.0 ** -24 * _sum_abs(_bits(c_q), _bits(w_q)).reshape(rows, Hi, Di)
    _codes_within(q8.cpu().numpy(), ref_q, bound_q)


def test_key_projection_with_every_token_skipped(oracle_lib):
    """Tokens with no sequence row or past the page table write nothing: the caches keep their
    contents, with and without the split-K workspace; zero tokens is a no-op."""
    print("case: key projection, all tokens skipped", flush=True)
    h, _, w_k, _, _ = _case(991, 200, 256, 64)
    pt = torch.arange(4, dtype=torch.int32, device="cuda").view(1, 4)
    seq = torch.full((200,), -1, dtype=torch.int32, device="cuda")
    seq[100:] = 0
    pos = torch.arange(200, dtype=torch.int32, device="cuda") + 256   # rows 100.. are past the 4 pages
    for ws in (None, False):
        kc = torch.full((4, 64, 128), 0x77, dtype=torch.uint8, device="cuda")
        ks = torch.full((4, 64), 3.0, dtype=torch.float32, device="cuda")
        dsa.indexer_key_project(h, w_k, seq, pos, pt, kc, ks, ws=ws)
        dsa.indexer_key_project(h[:0], w_k, seq[:0], pos[:0], pt, kc, ks, ws=ws)
        torch.cuda.synchronize()
        assert bool((kc == 0x77).all()) and bool((ks == 3.0).all())
