"""Seeded synthetic inputs for the DeepSeek Sparse Attention hot path.

This module only draws random inputs and lays them out in the paged-cache format; it holds
none of the method's arithmetic (no scoring, selection or attention). Both the GPU library's
tests/benchmark and the CPU oracle consume the arrays it returns.

Workloads (sizes follow the decode/prefill regimes of the pages' cost tables: 4K, 16K, 128K):
  tiny            1 sequence, T=256 prefill, fp32 indexer (4 heads x 32), one attention head
                  (qk 64, v 64), k=32; q/k/v built from hidden states h ~ N(0,1), d=64
  decode_b16_4k   16 requests, lengths U{3584..4096}, 1 query each, identity paging
  decode_mtp_b64_16k 64 requests x 16384 tokens, 2 query rows each (positions L-2, L-1),
                  64-token pages through a randomly permuted page table
  prefill_8k      1 sequence, T queries at positions 0..T-1 over a T-token prefix (T=8192 default)
  prefill_chunk_128k 4096 queries at positions 126976..131071 over a 131072-token prefix
  decode_b4_128k  4 requests x 131072 tokens, 1 query each
Indexer operands (all but tiny): q8 = E4M3(N(0,1)) [rows, 64, 128]; keys k ~ N(0,1)^128 stored as
k8 = E4M3(k / s) with the per-token scale s = max|k| / 448; w ~ N(0,1)/8. The 128K workloads scale
round(1% of n) seeded key rows by 4 (their scale only). MLA: q ~ N(0,1) bf16 [rows, 128, 576],
latent rows ~ N(0,1) bf16 [.., 576], v = the first 512 columns, softmax scale 1/sqrt(192).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 0xD5A0
PAGE = 64
E4M3 = 0
F32 = 1

CONFIG_SEEDS = {
    "tiny": 0,
    "decode_b16_4k": 1,
    "decode_mtp_b64_16k": 2,
    "prefill_8k": 3,
    "prefill_chunk_128k": 4,
    "decode_b4_128k": 5,
}


@dataclass
class Workload:
    name: str
    n_seq: int
    q_per_seq: int
    q_pos: np.ndarray          # int32 [rows]
    page_table: np.ndarray     # int32 [n_seq, ld_pt]
    page_size: int
    max_ctx: int               # host-side bound: every q_pos < max_ctx
    topk: int
    # indexer
    fmt: int                   # E4M3 or F32
    iq: np.ndarray             # uint8 or float32 [rows, Hi, Di]
    iw: np.ndarray             # float32 [rows, Hi]
    ik: np.ndarray             # uint8 or float32 [num_pages, page, Di]
    iks: np.ndarray | None     # float32 [num_pages, page] or None
    # attention
    q: np.ndarray              # uint16 (bf16 bits) [rows, H, Dqk]
    kv: np.ndarray             # uint16 (bf16 bits) [num_pages, page, kv_dim]
    Dqk: int
    Dv: int
    v_col0: int
    sm_scale: float
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.n_seq * self.q_per_seq

    @property
    def Hi(self) -> int:
        return self.iq.shape[1]

    @property
    def Di(self) -> int:
        return self.iq.shape[2]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def kv_dim(self) -> int:
        return self.kv.shape[2]

    @property
    def num_pages(self) -> int:
        return self.kv.shape[0]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _randn(g, *shape) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Round a float32 tensor to bfloat16 (round to nearest even) and return the raw bits."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_bits(x: torch.Tensor) -> np.ndarray:
    """Round a float32 tensor (|x| <= 448) to OCP FP8 E4M3FN and return the raw bytes."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_keys(k: torch.Tensor):
    """Per-token FP8 keys: s = max|k|/448, k8 = E4M3(k / s). Returns (bytes, scales)."""
    s = k.abs().amax(dim=-1).clamp_min(1e-30) / 448.0
    k8 = e4m3_bits((k / s.unsqueeze(-1)).clamp(-448.0, 448.0))
    return k8, s.numpy().astype(np.float32)


def _identity_pages(n_seq: int, pages_per_seq: int) -> np.ndarray:
    return np.arange(n_seq * pages_per_seq, dtype=np.int32).reshape(n_seq, pages_per_seq)


def _fill_indexer_and_mla(g, rows, num_pages, Hi=64, Di=128, H=128, Dqk=576, boost_rows=None):
    n_tok = num_pages * PAGE
    iq = e4m3_bits(_randn(g, rows, Hi, Di))
    iw = (_randn(g, rows, Hi) / 8.0).numpy()
    k8, ks = quantize_keys(_randn(g, n_tok, Di))
    if boost_rows is not None and len(boost_rows):
        ks[boost_rows] *= 4.0
    q = bf16_bits(_randn(g, rows, H, Dqk))
    kv = bf16_bits(_randn(g, n_tok, Dqk))
    return (iq, iw, k8.reshape(num_pages, PAGE, Di), ks.reshape(num_pages, PAGE),
            q, kv.reshape(num_pages, PAGE, Dqk))


def make_tiny(seed: int | None = None) -> Workload:
    """Prefill of one 256-token sequence built from hidden states h ~ N(0,1), d = 64."""
    g = _gen(SEED_BASE + CONFIG_SEEDS["tiny"] if seed is None else seed)
    T, d, Hi, Di = 256, 64, 4, 32
    h = _randn(g, T, d)
    wq = _randn(g, d, Hi * Di) / math.sqrt(d)
    wk = _randn(g, d, Di) / math.sqrt(d)
    iw = _randn(g, T, Hi).numpy()
    WQ = _randn(g, d, 64) / math.sqrt(d)
    WK = _randn(g, d, 64) / math.sqrt(d)
    WV = _randn(g, d, 64) / math.sqrt(d)
    iq = (h @ wq).reshape(T, Hi, Di).numpy().astype(np.float32)
    ik = (h @ wk).numpy().astype(np.float32).reshape(T // PAGE, PAGE, Di)
    q = bf16_bits((h @ WQ).reshape(T, 1, 64))
    kv = bf16_bits(torch.cat([h @ WK, h @ WV], dim=1)).reshape(T // PAGE, PAGE, 128)
    return Workload("tiny", 1, T, np.arange(T, dtype=np.int32), _identity_pages(1, T // PAGE), PAGE, T, 32,
                    F32, iq, iw.astype(np.float32), ik, None, q, kv, 64, 64, 64, 1.0 / 8.0)


def make_decode_b16_4k(seed: int | None = None) -> Workload:
    g = _gen(SEED_BASE + CONFIG_SEEDS["decode_b16_4k"] if seed is None else seed)
    B, Lmax = 16, 4096
    lens = torch.randint(3584, 4097, (B,), generator=g).numpy().astype(np.int32)
    pps = Lmax // PAGE
    iq, iw, ik, iks, q, kv = _fill_indexer_and_mla(g, B, B * pps)
    return Workload("decode_b16_4k", B, 1, lens - 1, _identity_pages(B, pps), PAGE, Lmax, 2048,
                    E4M3, iq, iw, ik, iks, q, kv, 576, 512, 0, 1.0 / math.sqrt(192.0),
                    extra={"lens": lens})


def make_decode_mtp_b64_16k(seed: int | None = None, B: int = 64, L: int = 16384) -> Workload:
    g = _gen(SEED_BASE + CONFIG_SEEDS["decode_mtp_b64_16k"] if seed is None else seed)
    pps = L // PAGE
    perm = torch.randperm(B * pps, generator=g).numpy().astype(np.int32)
    iq, iw, ik, iks, q, kv = _fill_indexer_and_mla(g, 2 * B, B * pps)
    q_pos = np.tile(np.array([L - 2, L - 1], dtype=np.int32), B)
    return Workload("decode_mtp_b64_16k", B, 2, q_pos, perm.reshape(B, pps), PAGE, L, 2048,
                    E4M3, iq, iw, ik, iks, q, kv, 576, 512, 0, 1.0 / math.sqrt(192.0))


def make_prefill(T: int = 8192, seed: int | None = None) -> Workload:
    g = _gen(SEED_BASE + CONFIG_SEEDS["prefill_8k"] + 16 * (T != 8192) * T if seed is None else seed)
    pps = (T + PAGE - 1) // PAGE
    iq, iw, ik, iks, q, kv = _fill_indexer_and_mla(g, T, pps)
    return Workload(f"prefill_{T}", 1, T, np.arange(T, dtype=np.int32), _identity_pages(1, pps), PAGE, T, 2048,
                    E4M3, iq, iw, ik, iks, q, kv, 576, 512, 0, 1.0 / math.sqrt(192.0))


def _boost(g, n_tok):
    n = int(round(0.01 * n_tok))
    return torch.randperm(n_tok, generator=g)[:n].numpy()


def make_prefill_chunk_128k(seed: int | None = None, S: int = 131072, Tq: int = 4096) -> Workload:
    g = _gen(SEED_BASE + CONFIG_SEEDS["prefill_chunk_128k"] if seed is None else seed)
    pps = S // PAGE
    boost = _boost(g, S)
    iq, iw, ik, iks, q, kv = _fill_indexer_and_mla(g, Tq, pps, boost_rows=boost)
    q_pos = np.arange(S - Tq, S, dtype=np.int32)
    return Workload("prefill_chunk_128k", 1, Tq, q_pos, _identity_pages(1, pps), PAGE, S, 2048,
                    E4M3, iq, iw, ik, iks, q, kv, 576, 512, 0, 1.0 / math.sqrt(192.0),
                    extra={"boost_rows": boost})


def make_decode_b4_128k(seed: int | None = None, B: int = 4, L: int = 131072) -> Workload:
    g = _gen(SEED_BASE + CONFIG_SEEDS["decode_b4_128k"] if seed is None else seed)
    pps = L // PAGE
    boost = _boost(g, B * L)
    iq, iw, ik, iks, q, kv = _fill_indexer_and_mla(g, B, B * pps, boost_rows=boost)
    q_pos = np.full(B, L - 1, dtype=np.int32)
    return Workload("decode_b4_128k", B, 1, q_pos, _identity_pages(B, pps), PAGE, L, 2048,
                    E4M3, iq, iw, ik, iks, q, kv, 576, 512, 0, 1.0 / math.sqrt(192.0),
                    extra={"boost_rows": boost})


def make_random(n_seq, q_per_seq, q_pos, max_ctx, *, Hi=64, Di=128, H=128, Dqk=576, Dv=512, v_col0=0,
                kv_dim=None, topk=2048, fmt=E4M3, seed=12345, permute_pages=False, extra_pages=0):
    """Generic generator for parity tests: arbitrary shapes, optional permuted page table."""
    g = _gen(seed)
    kv_dim = kv_dim or max(Dqk, v_col0 + Dv)
    pps = (max_ctx + PAGE - 1) // PAGE
    num_pages = n_seq * pps + extra_pages
    rows = n_seq * q_per_seq
    n_tok = num_pages * PAGE
    if permute_pages:
        ids = torch.randperm(num_pages, generator=g)[: n_seq * pps].numpy().astype(np.int32)
    else:
        ids = np.arange(n_seq * pps, dtype=np.int32)
    if fmt == E4M3:
        iq = e4m3_bits(_randn(g, rows, Hi, Di))
        ik8, iks = quantize_keys(_randn(g, n_tok, Di))
        ik = ik8.reshape(num_pages, PAGE, Di)
        iks = iks.reshape(num_pages, PAGE)
    else:
        iq = _randn(g, rows, Hi, Di).numpy()
        ik = _randn(g, n_tok, Di).numpy().reshape(num_pages, PAGE, Di)
        iks = None
    iw = (_randn(g, rows, Hi) / 8.0).numpy()
    q = bf16_bits(_randn(g, rows, H, Dqk))
    kv = bf16_bits(_randn(g, n_tok, kv_dim)).reshape(num_pages, PAGE, kv_dim)
    return Workload(f"random_{n_seq}x{q_per_seq}", n_seq, q_per_seq, np.asarray(q_pos, dtype=np.int32),
                    ids.reshape(n_seq, pps), PAGE, max_ctx, topk, fmt, iq, iw, ik, iks, q, kv,
                    Dqk, Dv, v_col0, 1.0 / math.sqrt(Dqk if Dqk != 576 else 192.0))


MAKERS = {
    "tiny": make_tiny,
    "decode_b16_4k": make_decode_b16_4k,
    "decode_mtp_b64_16k": make_decode_mtp_b64_16k,
    "prefill_8k": make_prefill,
    "prefill_chunk_128k": make_prefill_chunk_128k,
    "decode_b4_128k": make_decode_b4_128k,
}
