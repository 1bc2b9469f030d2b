"""Shared test helpers: workload -> GPU tensors, tolerance checks written out explicitly.

Tolerances (for the DSA hot path):
  scores     per row r: max_j |I_gpu - I_ref| <= 1e-5 * max_j |I_ref|      (j <= q_pos[r])
  top-k      index sets equal, except positions whose reference score lies within
             1e-5 * max_j |I_ref| of the row's k-th largest reference score
  attention  max |o_gpu - o_ref| <= 2e-2 and ||o_gpu - o_ref||_2 / ||o_ref||_2 <= 5e-3
"""
import numpy as np
import torch

SCORE_REL = 1e-5
ATTN_MAX_ABS = 2e-2
ATTN_REL_RMS = 5e-3


def dev(a, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16).view(torch.uint16) if hasattr(torch, "uint16") else t
    return t.to(device)


def bf16_dev(bits, device="cuda"):
    """uint16 bf16 bits (numpy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_host_to_f32(t):
    return t.float().cpu().numpy()


def gpu_inputs(w, device="cuda"):
    d = {
        "q_pos": torch.from_numpy(w.q_pos).to(device),
        "page_table": torch.from_numpy(np.ascontiguousarray(w.page_table)).to(device),
        "iq": torch.from_numpy(np.ascontiguousarray(w.iq)).to(device),
        "iw": torch.from_numpy(np.ascontiguousarray(w.iw)).to(device),
        "ik": torch.from_numpy(np.ascontiguousarray(w.ik)).to(device),
        "iks": None if w.iks is None else torch.from_numpy(np.ascontiguousarray(w.iks)).to(device),
        "q": bf16_dev(w.q, device),
        "kv": bf16_dev(w.kv, device),
    }
    return d


def check_scores(gpu, ref, q_pos, rows=None):
    rows = range(ref.shape[0]) if rows is None else rows
    worst = 0.0
    for r in rows:
        n = int(q_pos[r]) + 1
        a, b = gpu[r, :n].astype(np.float64), ref[r, :n].astype(np.float64)
        scale = np.abs(b).max() if n else 0.0
        err = np.abs(a - b).max() if n else 0.0
        rel = err / scale if scale > 0 else err
        worst = max(worst, rel)
        assert rel <= SCORE_REL, f"row {r}: max|dI| = {err:.3e} > {SCORE_REL} * {scale:.3e}"
    return worst


def check_topk_sets(idx_gpu, idx_ref, ref_scores, q_pos, k, rows=None):
    """Sets must match except for positions within the tie band of the k-th reference score."""
    rows = range(idx_ref.shape[0]) if rows is None else rows
    n_diff = 0
    for r in rows:
        n = int(q_pos[r]) + 1
        g = idx_gpu[r]
        ref = idx_ref[r]
        m = min(n, k)
        assert (g[m:] == -1).all(), f"row {r}: padding"
        gs, rs = g[:m], ref[:m]
        assert (np.diff(gs) > 0).all(), f"row {r}: output not strictly ascending"
        assert gs.min() >= 0 and gs.max() < n, f"row {r}: position out of range"
        if np.array_equal(gs, rs):
            continue
        s = ref_scores[r, :n].astype(np.float64)
        kth = np.sort(s)[::-1][m - 1]
        band = SCORE_REL * np.abs(s).max()
        diff = np.setxor1d(gs, rs)
        n_diff += len(diff)
        assert np.all(np.abs(s[diff] - kth) <= band), f"row {r}: positions {diff[:8]} differ outside the tie band"
    return n_diff


def check_attn(out_gpu, out_ref):
    a = out_gpu.astype(np.float64)
    b = out_ref.astype(np.float64)
    assert np.isfinite(a).all(), "non-finite output"
    max_abs = np.abs(a - b).max() if a.size else 0.0
    rel_rms = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
    assert max_abs <= ATTN_MAX_ABS, f"max abs error {max_abs:.3e} > {ATTN_MAX_ABS}"
    assert rel_rms <= ATTN_REL_RMS, f"relative RMS error {rel_rms:.3e} > {ATTN_REL_RMS}"
    return max_abs, rel_rms
