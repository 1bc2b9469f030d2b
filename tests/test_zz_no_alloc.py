"""The no-allocation decode attention entry point (dsa_sparse_mla_decode_noalloc) on the GPU.

It runs the same kernels as dsa_sparse_mla_decode, with the split-merge workspace taken from the
library's own device array instead of the caller's buffer, so its outputs must equal that entry
point's bit for bit. Two calls in a row on the shared array, the second with a smaller input: a
128-row batch (two splits per row, 256 units: most of the array) and then a 5-row one (16 splits
per row), so the second call runs over what the first left there. Also: a shape that needs no
workspace (one split per row) and the rejection of a missing output tensor.
"""
import numpy as np
import pytest
import torch

from sparse_attention_06_amd import dsa

pytestmark = pytest.mark.gpu


def _case(n_rows, ctx, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    pages = (ctx + 63) // 64
    num_pages = n_rows * pages + 3
    q = torch.randn(n_rows, 128, 576, generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn(num_pages, 64, 576, generator=g, device="cuda").to(torch.bfloat16)
    pt = torch.randperm(num_pages, generator=g, device="cuda")[: n_rows * pages].to(torch.int32).view(n_rows, pages)
    rng = np.random.default_rng(seed)
    q_pos = rng.integers(ctx // 2, ctx, n_rows).astype(np.int32)
    k = 2048
    idx = np.full((n_rows, k), -1, np.int32)
    for r, t in enumerate(q_pos):
        m = min(k, int(t) + 1)
        idx[r, :m] = np.sort(rng.choice(int(t) + 1, m, replace=False))
    return q, kv, pt.contiguous(), torch.from_numpy(q_pos).cuda(), torch.from_numpy(idx).cuda()


def _both(q, kv, pt, q_pos, idx):
    rows = q.shape[0]
    scale = 1.0 / 192 ** 0.5
    out_ws = torch.empty(rows, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse_ws = torch.empty(rows, 128, dtype=torch.float32, device="cuda")
    dsa.sparse_mla_decode(q, kv, pt, q_pos, rows, 1, idx, 576, 512, 0, scale, out=out_ws, lse=lse_ws)
    path_ws = dsa.last_path()
    out_na = torch.full_like(out_ws, float("nan"))
    lse_na = torch.full_like(lse_ws, float("nan"))
    dsa.sparse_mla_decode_noalloc(q, kv, pt, q_pos, rows, 1, idx, 576, 512, 0, scale, out_na, lse=lse_na)
    assert dsa.last_path() == path_ws
    torch.cuda.synchronize()
    return (out_ws, lse_ws), (out_na, lse_na), path_ws


@pytest.mark.parametrize("n_rows,ctx", [(128, 3000), (5, 2500)])
def test_noalloc_equals_workspace_entry_point(n_rows, ctx):
    print(f"case: noalloc decode rows={n_rows} ctx={ctx}", flush=True)
    need = dsa.sparse_mla_workspace_size(n_rows, 128, 512, 2048)
    assert need > 0
    (o1, l1), (o2, l2), path = _both(*_case(n_rows, ctx, seed=n_rows))
    assert path == "mla_mfma_split"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_noalloc_two_calls_in_a_row_second_smaller():
    print("case: noalloc decode, two calls in a row", flush=True)
    big, small = _case(128, 3000, seed=7), _case(5, 2500, seed=8)
    ref_big = _both(*big)[0]
    ref_small = _both(*small)[0]
    scale = 1.0 / 192 ** 0.5
    outs = []
    for case in (big, small):
        q, kv, pt, q_pos, idx = case
        out = torch.empty(q.shape[0], 128, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(q.shape[0], 128, dtype=torch.float32, device="cuda")
        dsa.sparse_mla_decode_noalloc(q, kv, pt, q_pos, q.shape[0], 1, idx, 576, 512, 0, scale, out, lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for (o, l), (ro, rl) in zip(outs, (ref_big, ref_small)):
        assert torch.equal(o.view(torch.int16), ro.view(torch.int16))
        assert torch.equal(l, rl)


def test_noalloc_without_split_and_argument_errors():
    print("case: noalloc decode, no split; argument errors", flush=True)
    q, kv, pt, q_pos, idx = _case(300, 1200, seed=9)            # 300 rows: one workgroup per row
    assert dsa.sparse_mla_workspace_size(300, 128, 512, 2048) == 0
    (o1, l1), (o2, l2), path = _both(q, kv, pt, q_pos, idx)
    assert path == "mla_mfma"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    with pytest.raises(ValueError):
        dsa.sparse_mla_decode_noalloc(q, kv, pt, q_pos, 300, 1, idx, 576, 512, 0, 0.1, None)
    bad = torch.empty(300, 128, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DSAError, match="INVALID_ARG"):
        dsa.sparse_mla_decode_noalloc(q, kv, pt, q_pos, 300, 1, idx, 576, 512, 65, 0.1, bad)
