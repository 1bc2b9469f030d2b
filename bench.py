"""Benchmark of the DSA decode hot path on one MI355X.

A step = one pass of the whole hot path over one batch: Lightning Indexer scores for every
visible position (dsa_indexer_scores), exact top-2048 (dsa_topk), and sparse MLA attention over
the selected latent rows (dsa_sparse_mla_decode). Default workload: MTP-verification decode,
64 requests x 16384-token context, 2 query rows per request (128 queries per step), 64-token
pages through a randomly permuted page table, synthetic inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --crossover     # dense fallback vs sparse prefill at T = 1K/2K/4K/8K

Prints ONE JSON line (the contract) on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode queries/s + achieved HBM GB/s (indexer+top-2048+sparse MLA), 16K ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16/f16 MFMA
KV_ROW_BYTES = 576 * 2         # latent row, bf16
IDX_KEY_BYTES = 128 + 4        # FP8 indexer key + fp32 scale


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ analytic model
# Unit costs of the method's shapes: the [Handbook] "稀疏注意力：NSA 与 DSA" dims (absorbed MLA: 128
# heads over one 512 + 64 latent row per position, value = its first 512 columns; the indexer: 64
# heads of 128 dims, FP8 keys with a float scale; the expanded form: per head 128 + 64 qk dims and
# 128 value dims).
def attention_pair_flops(H=128, Dqk=576, Dv=512):
    """FLOPs of one (query, position) pair: a Dqk-long logit and a Dv-wide value update per head."""
    return 2 * H * Dqk + 2 * H * Dv


def indexer_pair_flops(Hi=64, Di=128):
    """FLOPs of one (query, key) index score: one Di-long dot per indexer head (the ReLU and the
    head-weighted sum are not counted)."""
    return 2 * Hi * Di


def per_layer_cost(L, k=2048):
    """One layer, one sequence of context L, dense MLA against DSA (index set of min(L, k)):
      decode_flops   one query: every position attended, against every key scored plus the
                     selected positions attended
      decode_bytes   the cache rows that query reads: every latent row, against every indexer key
                     plus the selected latent rows
      prefill_flops  L causal queries: dense runs the expanded form over L^2 / 2 pairs (the count the
                     page's table uses), DSA scores the same pairs and attends L * min(L, k) pairs
                     in the absorbed form
    Each entry is a (dense, dsa) pair."""
    sel = min(L, k)
    pairs = L * L / 2
    mla, idx = attention_pair_flops(), indexer_pair_flops()
    return {
        "decode_flops": (L * mla, L * idx + sel * mla),
        "decode_bytes": (L * KV_ROW_BYTES, L * IDX_KEY_BYTES + sel * KV_ROW_BYTES),
        "prefill_flops": (pairs * attention_pair_flops(128, 128 + 64, 128), pairs * idx + L * sel * mla),
    }


def decode_step_bytes(n_seq, q_per_seq, ctx_per_seq, k, H=128, Dqk=576, Dv=512, Hi=64, Di=128):
    """Algorithmic bytes of one decode step, per kernel (what the method must move; the fp32 score
    and index round trips between kernels are intermediates)."""
    rows = n_seq * q_per_seq
    keys = int(np.sum(ctx_per_seq)) * IDX_KEY_BYTES                 # once per request
    qw = rows * (Hi * Di + Hi * 4)
    kv = rows * k * KV_ROW_BYTES
    q_out = rows * (H * Dqk * 2 + H * Dv * 2)
    scores = int(np.sum(np.repeat(ctx_per_seq, q_per_seq))) * 4
    return {"indexer": keys + qw, "topk": scores + rows * k * 4, "mla": kv + q_out,
            "step": keys + qw + kv + q_out}


def decode_step_flops(n_seq, q_per_seq, ctx_per_seq, k, H=128, Dqk=576, Dv=512, Hi=64, Di=128):
    rows_ctx = int(np.sum(np.repeat(ctx_per_seq, q_per_seq)))
    return {"indexer": rows_ctx * indexer_pair_flops(Hi, Di),
            "mla": n_seq * q_per_seq * k * attention_pair_flops(H, Dqk, Dv)}


# ------------------------------------------------------------------ GPU step
class DecodeStep:
    """Device buffers for `copies` independent copies of a decode workload and its calls: the
    indexer, the top-k and the sparse attention, or (fused) the indexer and top-k as one call
    sharing the first radix pass, then the attention."""

    def __init__(self, w, copies=2, fused=False):
        import torch
        from sparse_attention_06_amd import dsa

        self.w, self.dsa, self.torch = w, dsa, torch
        self.copies = []
        for c in range(copies):
            d = {
                "iq": torch.from_numpy(np.ascontiguousarray(w.iq)).cuda(),
                "iw": torch.from_numpy(np.ascontiguousarray(w.iw)).cuda(),
                "ik": torch.from_numpy(np.ascontiguousarray(w.ik)).cuda(),
                "iks": torch.from_numpy(np.ascontiguousarray(w.iks)).cuda(),
                "q": torch.from_numpy(np.ascontiguousarray(w.q).view(np.int16)).view(torch.bfloat16).cuda(),
                "kv": torch.from_numpy(np.ascontiguousarray(w.kv).view(np.int16)).view(torch.bfloat16).cuda(),
                "page_table": torch.from_numpy(np.ascontiguousarray(w.page_table)).cuda(),
                "q_pos": torch.from_numpy(w.q_pos).cuda(),
            }
            d["scores"] = torch.empty(w.rows, w.max_ctx, dtype=torch.float32, device="cuda")
            d["idx"] = torch.empty(w.rows, w.topk, dtype=torch.int32, device="cuda")
            d["out"] = torch.empty(w.rows, w.H, w.Dv, dtype=torch.bfloat16, device="cuda")
            need = dsa.sparse_mla_workspace_size(w.rows, w.H, w.Dv, w.topk)
            d["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need else None
            tneed = dsa.topk_workspace_size(w.rows, w.max_ctx, w.topk)
            d["tws"] = torch.empty(tneed, dtype=torch.uint8, device="cuda") if tneed else None
            # the fused call's workspace starts zeroed and every call leaves it so
            fneed = dsa.indexer_topk_workspace_size(w.rows, w.max_ctx, w.topk)
            d["fws"] = torch.zeros(fneed, dtype=torch.uint8, device="cuda")
            self.copies.append(d)
        self.stream = torch.cuda.current_stream()
        self.fused = fused
        self.calls = ((self.call_indexer_topk, self.call_mla) if fused else
                      (self.call_indexer, self.call_topk, self.call_mla))

    def call_indexer_topk(self, c, st):
        w, d = self.w, self.copies[c % len(self.copies)]
        self.dsa.indexer_topk(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], w.n_seq,
                              w.q_per_seq, w.max_ctx, w.topk, scores=d["scores"], idx=d["idx"], ws=d["fws"],
                              stream=st)

    def call_indexer(self, c, st):
        w, d = self.w, self.copies[c % len(self.copies)]
        self.dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["page_table"], d["q_pos"], w.n_seq,
                                w.q_per_seq, w.max_ctx, scores=d["scores"], stream=st)

    def call_topk(self, c, st):
        w, d = self.w, self.copies[c % len(self.copies)]
        self.dsa.topk(d["scores"], d["q_pos"], w.max_ctx, w.topk, idx=d["idx"], ws=d["tws"], stream=st)

    def call_mla(self, c, st):
        w, d = self.w, self.copies[c % len(self.copies)]
        # decode / MTP rows (at most 2 per request) and prefill blocks have their own entry points
        fn = self.dsa.sparse_mla_decode if w.q_per_seq <= 2 else self.dsa.sparse_mla_prefill
        fn(d["q"], d["kv"], d["page_table"], d["q_pos"], w.n_seq, w.q_per_seq, d["idx"], w.Dqk, w.Dv, w.v_col0,
           w.sm_scale, out=d["out"], ws=d["ws"], stream=st)

    def run(self, c, events=None, stream=None):
        """One step; with `events` (4), events[0..3] bracket indexer | top-k | attention (fused:
        events[1] and [2] both sit between the fused call and the attention)."""
        st = stream if stream is not None else self.stream
        if events and self.fused:
            events[0].record(st)
            self.call_indexer_topk(c, st)
            events[1].record(st)
            events[2].record(st)
            self.call_mla(c, st)
            events[3].record(st)
            return
        for i, fn in enumerate(self.calls):
            if events:
                events[i].record(st)
            fn(c, st)
        if events:
            events[3].record(st)

    def capture(self, fns=None):
        """One HIP graph per input copy holding `fns` (default: the whole step, i.e. the four
        kernel launches), so replays carry no host-side launch gaps."""
        torch = self.torch
        fns = fns or self.calls
        graphs = []
        for c in range(len(self.copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st = torch.cuda.current_stream()
                for fn in fns:
                    fn(c, st)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs


def time_call(step, fn, steps, reps=8):
    """Average duration of one call of `fn` (ms): a HIP graph holding `reps` calls back to back,
    alternating the input copies, replayed `steps` times; dividing by reps spreads the graph's own
    launch cost over the calls, so the figure is the calls' duration (what the kernel trace
    reports), not one launch overhead per call."""
    torch = step.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for i in range(reps):
            fn(i % len(step.copies), st)
    torch.cuda.synchronize()
    return time_replays(torch, [g], steps)[0] / reps


def time_replays(torch, graphs, steps):
    """ms per replay over `steps` replays (alternating graphs) between device-wide syncs."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def time_graph_steps(step, steps, warmup):
    """Time `steps` whole-step graph replays (alternating input copies) between device-wide
    synchronisations; returns (ms per step, wall seconds). The first replay of every graph is
    checked against an eager step on the same inputs."""
    torch = step.torch
    for i in range(warmup):
        step.run(i)
    torch.cuda.synchronize()
    eager = [(d["idx"].clone(), d["out"].clone()) for d in step.copies]
    graphs = step.capture()
    for c, g in enumerate(graphs):
        g.replay()
        torch.cuda.synchronize()
        d = step.copies[c]
        if not (torch.equal(d["idx"], eager[c][0]) and torch.equal(d["out"], eager[c][1])):
            bad_idx = int((d["idx"] != eager[c][0]).sum())
            bad_out = int((d["out"].view(torch.int16) != eager[c][1].view(torch.int16)).sum())
            raise SystemExit(f"graph replay differs from the eager step (copy {c}: {bad_idx} index entries, "
                             f"{bad_out} output elements)")
    return time_replays(torch, graphs, steps)


def time_eager_steps(step, steps):
    """ms per step over `steps` eager steps (the calls launched one after another on one stream,
    no events between them), bracketed by device synchronisations; and the wall seconds."""
    torch = step.torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step.run(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def time_eager_same_copy(step, steps):
    """ms per eager step when every step reads the same input copy (caches warm: what the last
    step left in L2 and the 256 MB MALL is there for the next)."""
    torch = step.torch
    for _ in range(20):
        step.run(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step.run(0)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def input_copies(w):
    """Input copies to rotate so that a step's inputs were last touched more than the MALL's
    256 MB of other traffic ago (at least 2)."""
    per_copy = (w.ik.nbytes + (w.iks.nbytes if w.iks is not None else 0) + w.kv.nbytes + w.q.nbytes +
                w.iq.nbytes + w.iw.nbytes)
    return max(2, -(-384 * 2**20 // max(per_copy, 1)))


def time_steps(step, steps, warmup):
    torch = step.torch
    for i in range(warmup):
        step.run(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                     e[0].elapsed_time(e[3])] for e in evs])  # ms
    return wall, per


# ------------------------------------------------------------------ CPU baseline (the oracle)
def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, max_threads=16):
    """The oracle as it stands, on the host cores, over a bounded sample of the same workload:
    whole requests (all their query rows), indexer + top-k + attention, one request per thread.
    Threads: the cores this process may run on, at most max_threads (the per-GPU CPU share of the
    boxes this runs on); also timed on one thread with one request."""
    import oracle

    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    threads = max(1, min(visible, max_threads))
    qps = w.q_per_seq

    def one_request(s):
        rows = list(range(s * qps, (s + 1) * qps))
        sc = oracle.indexer_scores(w.iq, w.iw, w.ik, w.iks, w.page_table, w.page_size, w.q_pos, w.n_seq, qps, w.fmt,
                                   w.max_ctx, rows=rows)
        idx = oracle.topk(sc, w.q_pos, w.topk, rows=rows)
        oracle.sparse_mla(w.q, w.kv, w.page_table, w.page_size, w.q_pos, w.n_seq, qps, idx, w.Dqk, w.Dv, w.v_col0,
                          w.sm_scale, rows=rows)

    def timed(reqs):
        t0 = time.perf_counter()
        ths = [threading.Thread(target=one_request, args=(s,)) for s in reqs]
        for t in ths:
            t.start()
        for t in ths:
            t.join()
        return time.perf_counter() - t0

    reqs = list(range(min(threads, w.n_seq)))
    dt = timed(reqs)
    dt1 = timed([w.n_seq - 1])
    return {"value": len(reqs) * qps / dt, "unit": "queries/s", "cores": len(reqs), "kind": "oracle",
            "sample": f"{len(reqs)} requests x {qps} query rows of the benchmark workload (indexer over "
                      f"{int(w.q_pos[0]) + 1}+ positions, top-{w.topk}, 128-head attention), one request per "
                      f"thread, {dt:.1f} s wall; then 1 request on 1 thread, {dt1:.1f} s",
            "cpu_model": cpu_model(), "cores_visible": visible, "value_1core": qps / dt1}


# ------------------------------------------------------------------ roofline / traffic
def _src_hash():
    h = hashlib.sha256()
    for f in ("mla.hip", "dsa_internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on this
    workload and the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    ent = t.get(kernel_key)
    if not ent or ent.get("source_hash") != _src_hash() or ent.get("workload") != workload:
        return None
    return ent.get("bytes_per_launch")


def run_decode_bench(args):
    import torch

    import workloads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    t0 = time.time()
    w = workloads.MAKERS[args.workload]()
    log(f"[bench] workload {w.name}: {w.n_seq} requests x {w.q_per_seq} rows, ctx {w.max_ctx}, "
        f"generated in {time.time() - t0:.1f} s")
    copies = input_copies(w)
    step = DecodeStep(w, copies=copies, fused=not args.separate_indexer_topk)
    if args.no_graph:
        # eager steps only (for profiler runs that do not follow graph launches)
        wall, per = time_steps(step, args.steps, args.settle + args.warmup)
        ms = [float(x) for x in per.mean(axis=0)]
        ms_step = ms[3]
    else:
        # the step as launched: eager steps, the four launches back to back on one stream (on this
        # GPU-bound step they run a few percent faster than graph replays of the same launches,
        # which are timed too, after a bit-for-bit check against the eager result); per-call times
        # from graphs of repeated calls; an eager pass with events between the calls
        for i in range(args.settle + args.warmup):
            step.run(i)
        ms_step, wall = time_eager_steps(step, args.steps)
        ms_step = float(ms_step)
        ms_graph, _ = time_graph_steps(step, args.steps, 0)
        ms_warm = time_eager_same_copy(step, args.steps)
        ms = [time_call(step, fn, args.steps) for fn in (step.call_indexer, step.call_topk, step.call_mla)]
        ms_fused = time_call(step, step.call_indexer_topk, args.steps)
        _, per = time_steps(step, args.steps, 1)
        ms.append(float(per.mean(axis=0)[3]))
    ctx = w.q_pos.reshape(w.n_seq, w.q_per_seq).max(axis=1) + 1
    by = decode_step_bytes(w.n_seq, w.q_per_seq, ctx, w.topk)
    fl = decode_step_flops(w.n_seq, w.q_per_seq, ctx, w.topk)
    rows = w.rows
    qps = rows / (ms_step * 1e-3)
    detail = {
        "ms": {"indexer": float(ms[0]), "topk": float(ms[1]), "sparse_mla": float(ms[2]), "step": ms_step,
               "step_graph_replay": None if args.no_graph else float(ms_graph),
               "step_eager_with_events": float(ms[3]),
               "indexer_topk_fused": None if args.no_graph else float(ms_fused),
               "step_warm_same_inputs": None if args.no_graph else float(ms_warm)},
        "input_copies": copies,
        "step_calls": "indexer_topk (fused) + sparse_mla" if step.fused else "indexer + topk + sparse_mla",
        "wall_ms_per_step": wall / args.steps * 1e3,
        "algorithmic_GBps": {"indexer": by["indexer"] / ms[0] / 1e6, "topk": by["topk"] / ms[1] / 1e6,
                             "sparse_mla": by["mla"] / ms[2] / 1e6, "step": by["step"] / ms_step / 1e6},
        "algorithmic_MB": {k: v / 1e6 for k, v in by.items()},
        "tokens_per_s": {"indexer_keys_scored": float(np.sum(np.repeat(ctx, w.q_per_seq))) / (ms[0] * 1e-3),
                         "topk_rows": rows / (ms[1] * 1e-3), "mla_queries": rows / (ms[2] * 1e-3)},
        "mfma_TFLOPs": {"indexer_f16": fl["indexer"] / ms[0] / 1e9, "sparse_mla_bf16": fl["mla"] / ms[2] / 1e9},
        "requests_per_s": w.n_seq / (ms_step * 1e-3),
    }
    if w.q_per_seq == 2:
        # KV rows the two MTP rows of a request read: each row's own set, and their union (what a
        # gather shared by the two rows would read)
        idx = step.copies[0]["idx"].cpu().numpy().reshape(w.n_seq, 2, w.topk)
        own = sum(int((idx[s_] >= 0).sum()) for s_ in range(w.n_seq))
        union = sum(np.union1d(idx[s_, 0][idx[s_, 0] >= 0], idx[s_, 1][idx[s_, 1] >= 0]).size
                    for s_ in range(w.n_seq))
        row_bytes = 2 * 576
        detail["mtp_kv_rows"] = {"per_row_sets": own, "union_of_request_sets": union,
                                 "per_row_MB": own * row_bytes / 1e6, "union_MB": union * row_bytes / 1e6}
    log("[bench] " + json.dumps(detail))
    mla_bytes = by["mla"]
    achieved = mla_bytes / (ms[2] * 1e-3) / 1e9
    # the call's two launches: the attention kernel and the merge of its key splits
    tr = [measured_traffic(key, args.workload) for key in ("sparse_mla_decode", "sparse_mla_combine")]
    traffic = None if None in tr else sum(tr)
    roof = {"bound": "hbm", "kernel": "dsa_sparse_mla_decode (mla_mfma_kernel + mla_combine_kernel)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "algorithmic_bytes_per_launch": mla_bytes}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(w)
    line = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": args.settle, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "requests": w.n_seq, "query_rows_per_request": w.q_per_seq,
                   "context": int(w.max_ctx), "topk": w.topk, "indexer": "64 heads x 128 dims, FP8 E4M3",
                   "mla": "128 heads, 576-wide bf16 latent rows, v 512", "page_size": w.page_size,
                   "step_GBps": round(by["step"] / ms_step / 1e6, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


def run_prefill_bench(args):
    """One prefill block (indexer prefill contraction + top-k + sparse MLA prefill) timed like the
    decode step: graph replays of the whole block, and of each call on its own."""
    import torch

    import workloads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    t0 = time.time()
    w = workloads.MAKERS[args.workload]()
    log(f"[bench] workload {w.name}: {w.rows} query rows over {w.max_ctx} positions, generated in "
        f"{time.time() - t0:.1f} s")
    # rows over one 16384-position top-k chunk take the fused indexer + top-k call (its chunk stage
    # starts from the scan's counts: faster at the 128K chunk); shorter ones the separate calls
    # (faster at the 8K block, where the scan's counting costs more than the top-k saves)
    step = DecodeStep(w, copies=1, fused=w.max_ctx > 16384)
    # a prefill block takes milliseconds: a few warm-up and timed blocks suffice
    steps, warmup = min(args.steps, 20), min(args.warmup, 5)
    if args.no_graph:
        # eager blocks with events between the calls (for profiler runs that do not follow graphs)
        wall, per = time_steps(step, steps, warmup)
        ms = [float(x) for x in per.mean(axis=0)[:3]]
        ms_step = float(per.mean(axis=0)[3])
    else:
        ms_step, wall = time_graph_steps(step, steps, warmup)
        ms = [time_call(step, fn, steps, reps=2) for fn in (step.call_indexer, step.call_topk, step.call_mla)]
    ms_fused = time_call(step, step.call_indexer_topk, steps, reps=2) if step.fused and not args.no_graph else None
    ctx = w.q_pos.astype(np.int64) + 1
    sel = np.minimum(ctx, w.topk)
    flops = {"indexer": float(np.sum(ctx)) * 2 * w.Hi * w.Di,
             "mla": float(np.sum(sel)) * 2 * w.H * (w.Dqk + w.Dv)}
    tflops = {"indexer_f16": flops["indexer"] / ms[0] / 1e9, "sparse_mla_bf16": flops["mla"] / ms[2] / 1e9}
    dominant = "indexer" if ms[0] >= ms[2] else "mla"
    achieved = tflops["indexer_f16"] if dominant == "indexer" else tflops["sparse_mla_bf16"]
    roof = {"bound": "mfma",
            "kernel": ("indexer_scan_kernel<2> (dsa_indexer_scores)" if w.page_size == 64 else
                       "indexer_prefill_kernel (dsa_indexer_scores)") if dominant == "indexer"
            else "mla_mfma_kernel (dsa_sparse_mla_prefill)",
            "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": flops[dominant]}
    if dominant == "indexer" and step.fused:
        roof["note"] = ("timed as the dsa_indexer_scores call; the step's fused call runs the same scan "
                        "with the top-k's first-digit counts added")
    line = {
        "metric": "DSA prefill queries/s (indexer + top-2048 + sparse MLA)", "value": round(w.rows / (ms_step * 1e-3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(float(ms_step), 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "query_rows": w.rows, "context": int(w.max_ctx), "topk": w.topk,
                   "indexer": "64 heads x 128 dims, FP8 E4M3", "mla": "128 heads, 576-wide bf16 latent rows, v 512",
                   "page_size": w.page_size},
        "roofline": roof,
        "cpu_baseline": None,
        "detail": {"ms": {"indexer": ms[0], "topk": ms[1], "sparse_mla": ms[2], "step": float(ms_step),
                          "indexer_topk_fused": ms_fused},
                   "step_calls": "indexer_topk (fused) + sparse_mla" if step.fused else "indexer + topk + sparse_mla",
                   "wall_ms_per_step": wall / steps * 1e3, "mfma_TFLOPs": tflops,
                   "TFLOP": {k: v / 1e12 for k, v in flops.items()},
                   "topk_rows_per_s": w.rows / (ms[1] * 1e-3)},
    }
    print(json.dumps(line), flush=True)


class CrossoverCase:
    """The crossover sweep's inputs and calls for one sequence of T queries over a T-token prefix:
    the sparse path (indexer + top-k + sparse attention), the absorbed dense fallback, the expanded
    multi-head fallback (dense causal, and masked to the sparse path's index sets) and the two
    up-projection GEMMs the expanded form needs. With keep_host, the workload's host arrays stay in
    `w` (for checks against the oracle); otherwise the large ones are dropped after the upload."""

    def __init__(self, T, keep_host=False):
        import torch

        import workloads
        from sparse_attention_06_amd import dsa

        self.T, self.dsa, self.torch = T, dsa, torch
        w = workloads.make_prefill(T)
        self.d = d = {
            "iq": torch.from_numpy(w.iq).cuda(), "iw": torch.from_numpy(w.iw).cuda(),
            "ik": torch.from_numpy(w.ik).cuda(), "iks": torch.from_numpy(w.iks).cuda(),
            "q": torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).cuda(),
            "kv": torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).cuda(),
            "pt": torch.from_numpy(w.page_table).cuda(), "qp": torch.from_numpy(w.q_pos).cuda(),
        }
        if not keep_host:
            del w.q, w.kv
        self.w = w
        self.scores = torch.empty(T, T, dtype=torch.float32, device="cuda")
        self.idx = torch.empty(T, 2048, dtype=torch.int32, device="cuda")
        self.out = torch.empty(T, 128, 512, dtype=torch.bfloat16, device="cuda")
        # expanded operands (seeded, N(0,1) rounded to bf16) and the up-projection GEMM operands
        g = torch.Generator(device="cuda")
        g.manual_seed(0xD5A0 + T)
        self.xq = torch.randn(T, 128, 192, generator=g, device="cuda").to(torch.bfloat16)
        self.xkn = torch.randn(1, 128, T, 128, generator=g, device="cuda").to(torch.bfloat16)
        self.xkr = torch.randn(1, T, 64, generator=g, device="cuda").to(torch.bfloat16)
        self.xv = torch.randn(1, 128, T, 128, generator=g, device="cuda").to(torch.bfloat16)
        self.xout = torch.empty(T, 128, 128, dtype=torch.bfloat16, device="cuda")
        self.mws = torch.empty(dsa.expanded_mha_workspace_size(T, T, 2048), dtype=torch.uint8, device="cuda")
        self.lat = d["kv"].view(-1, 576)[:T, :512]
        self.wuk = (torch.randn(512, 128 * 128, generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
        self.kexp = torch.empty(T, 128 * 128, dtype=torch.bfloat16, device="cuda")
        self.scale = 1 / 192 ** 0.5

    def sparse(self):
        d, T, dsa = self.d, self.T, self.dsa
        dsa.indexer_scores(d["iq"], d["iw"], d["ik"], d["iks"], d["pt"], d["qp"], 1, T, T, scores=self.scores)
        dsa.topk(self.scores, d["qp"], T, 2048, idx=self.idx)
        dsa.sparse_mla_prefill(d["q"], d["kv"], d["pt"], d["qp"], 1, T, self.idx, 576, 512, 0, self.scale, out=self.out)

    def dense(self):
        d, T = self.d, self.T
        self.dsa.dense_mla_prefill(d["q"], d["kv"], d["pt"], d["qp"], 1, T, T, 576, 512, 0, self.scale, out=self.out)

    def expanded(self):
        self.dsa.expanded_mha_prefill(self.xq, self.xkn, self.xkr, self.xv, self.d["qp"], 1, self.T, self.scale,
                                      out=self.xout)

    def masked(self):
        self.dsa.expanded_mha_prefill(self.xq, self.xkn, self.xkr, self.xv, self.d["qp"], 1, self.T, self.scale,
                                      idx=self.idx, out=self.xout, ws=self.mws)

    def gemm(self):  # k_nope and v of all heads from the latent rows: two [T,512] x [512,16384]
        self.torch.matmul(self.lat, self.wuk, out=self.kexp)
        self.torch.matmul(self.lat, self.wuk, out=self.kexp)


def run_crossover(args):
    """Dense fallbacks vs sparse prefill (indexer + top-k + sparse attention) for one sequence of
    T queries over a T-token prefix. Two dense fallbacks: the absorbed form (the same attention
    kernel over every visible position) and the expanded multi-head form (per head 192-dim
    query/key and 128-dim value), dense causal and in the masked mode over the same index sets.
    The expanded form also needs its per-head keys and values up-projected from the latent rows
    (two plain GEMMs, timed here with torch.matmul as `expand_gemm_ms`)."""
    import torch

    sizes = [int(x) for x in args.crossover_T.split(",")]
    res = []
    for T in sizes:
        c = CrossoverCase(T)
        row = {"T": T}
        reps = min(args.steps, 10)
        for name, fn in (("sparse_ms", c.sparse), ("dense_absorbed_ms", c.dense), ("dense_expanded_ms", c.expanded),
                         ("masked_expanded_ms", c.masked), ("expand_gemm_ms", c.gemm)):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            row[name] = e0.elapsed_time(e1) / reps
        pairs = T * (T + 1) / 2
        row["expanded_TFLOPs"] = pairs * 128 * (2 * 192 + 2 * 128) / (row["dense_expanded_ms"] * 1e-3) / 1e12
        row["absorbed_wins"] = row["dense_absorbed_ms"] < row["sparse_ms"]
        row["expanded_wins"] = row["dense_expanded_ms"] + row["expand_gemm_ms"] < row["sparse_ms"]
        log(f"[crossover] {row}")
        res.append(row)
        del c
        torch.cuda.empty_cache()
    first = lambda key: next((r["T"] for r in res if not r[key]), None)  # noqa: E731
    print(json.dumps({"crossover": res, "sparse_beats_absorbed_dense_from_T": first("absorbed_wins"),
                      "sparse_beats_expanded_dense_from_T": first("expanded_wins")}), flush=True)


def run_cache_bench(args):
    """The step before the indexer at prefill scale: 131072 tokens of one sequence written into
    both paged caches (indexer keys quantised from f32, latent rows copied) and the indexer
    queries of a 4096-row block quantised; HBM GB/s of each against the peak."""
    import torch

    from sparse_attention_06_amd import dsa

    n, page = 131072, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(0xD5A0 + 7)
    pages = n // page
    pt = torch.randperm(pages, generator=g, device="cuda").to(torch.int32).view(1, pages)
    seq = torch.zeros(n, dtype=torch.int32, device="cuda")
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    k = torch.randn(n, 128, generator=g, device="cuda")
    rows = torch.randn(n, 576, generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.empty(pages, page, 128, dtype=torch.uint8, device="cuda")
    ks = torch.empty(pages, page, dtype=torch.float32, device="cuda")
    kv = torch.empty(pages, page, 576, dtype=torch.bfloat16, device="cuda")
    q = torch.randn(4096, 64, 128, generator=g, device="cuda")
    q8 = torch.empty(4096, 64, 128, dtype=torch.uint8, device="cuda")
    calls = {
        "indexer_cache_write": (lambda: dsa.indexer_cache_write(k, seq, pos, pt, kc, ks), n * (128 * 4 + 8 + 128 + 4)),
        "latent_cache_write": (lambda: dsa.latent_cache_write(rows, seq, pos, pt, kv), n * (2 * 1152 + 8)),
        "e4m3_quantize": (lambda: dsa.e4m3_quantize(q, out=q8), q.numel() * 5),
    }
    res = {}
    for name, (fn, nbytes) in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"us": ms * 1e3, "MB": nbytes / 1e6, "GBps": nbytes / (ms * 1e-3) / 1e9,
                     "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[cache] {name}: {res[name]}")
    print(json.dumps({"cache_write": res, "tokens": n, "query_rows": 4096}), flush=True)


def run_projection_bench(args):
    """The indexer's projections at the pages' hidden size d = 7168 (query latent 1536, 64 heads x
    128 dims): the key projection of a 131072-token prefix into the paged cache, of a 4096-token
    prefill chunk and of the decode step's 128 new keys, and the query projection (codes and head
    weights) of a 4096-row prefill chunk and of the decode step's 128 rows. TFLOP/s against the
    bf16 peak; also GB/s of weights and activations read (the decode-sized query projection
    streams 25 MB of w_q for 128 rows)."""
    import torch

    from sparse_attention_06_amd import dsa

    d, d_cq, Hi, Di, page = 7168, 1536, 64, 128, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(0xD5A0 + 9)
    w_k = (torch.randn(Di, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    w_q = (torch.randn(Hi * Di, d_cq, generator=g, device="cuda") / d_cq ** 0.5).to(torch.bfloat16)
    w_w = (torch.randn(Hi, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    n = 131072
    h = torch.randn(n, d, generator=g, device="cuda").to(torch.bfloat16)
    pt = torch.randperm(n // page, generator=g, device="cuda").to(torch.int32).view(1, -1)
    seq = torch.zeros(n, dtype=torch.int32, device="cuda")
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    kc = torch.empty(n // page, page, Di, dtype=torch.uint8, device="cuda")
    ks = torch.empty(n // page, page, dtype=torch.float32, device="cuda")
    res = {}

    def timed(name, fn, flops, nbytes, reps=8):
        # a graph of `reps` calls replayed `steps` times: the calls' GPU time without host gaps
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        ms = time_replays(torch, [gr], args.steps)[0] / reps
        res[name] = {"us": ms * 1e3, "TFLOPs": flops / (ms * 1e-3) / 1e12,
                     "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "GBps": nbytes / (ms * 1e-3) / 1e9}
        log(f"[proj] {name}: {res[name]}")

    timed("key_project_131072", lambda: dsa.indexer_key_project(h, w_k, seq, pos, pt, kc, ks, ws=False),
          2.0 * n * Di * d, n * d * 2 + Di * d * 2 + n * (Di + 4), reps=2)
    # a 4096-token prefill chunk's keys, and the decode step's new keys (one per query row, 128)
    for nk in (4096, 128):
        ws = torch.empty(max(16, dsa.indexer_projection_workspace_size(nk, d)), dtype=torch.uint8, device="cuda")
        timed(f"key_project_{nk}",
              lambda: dsa.indexer_key_project(h[:nk], w_k, seq[:nk], pos[:nk], pt, kc, ks, ws=ws),
              2.0 * nk * Di * d, nk * d * 2 + Di * d * 2 + nk * (Di + 4))
    for rows in (4096, 128):
        c_q = torch.randn(rows, d_cq, generator=g, device="cuda").to(torch.bfloat16)
        hr = h[:rows]
        q8 = torch.empty(rows, Hi, Di, dtype=torch.uint8, device="cuda")
        wo = torch.empty(rows, Hi, dtype=torch.float32, device="cuda")
        wsq = torch.empty(max(16, dsa.indexer_projection_workspace_size(rows, d)), dtype=torch.uint8, device="cuda")
        timed(f"query_project_{rows}",
              lambda: dsa.indexer_query_project(c_q, w_q, hr, w_w, Hi, Di, q8=q8, w=wo, ws=wsq),
              2.0 * rows * (Hi * Di * d_cq + Hi * d),
              rows * (d_cq + d) * 2 + (Hi * Di * d_cq + Hi * d) * 2 + rows * (Hi * Di + 4 * Hi))
    print(json.dumps({"projections": res, "d": d, "d_cq": d_cq, "heads": Hi, "head_dim": Di}), flush=True)


def run_copy_calibration(args):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch): the reference
    for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    n = 1 << 28  # float32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(args.steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                                           "launches": max(args.steps, 1)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10, help="untimed warmup steps before the timed ones")
    ap.add_argument("--settle", type=int, default=300,
                    help="further untimed steps run before the warmup, whatever --warmup is: the decode step "
                         "takes ~150 steps (~30 ms) to reach its steady speed (reported as settle_steps)")
    ap.add_argument("--workload", default="decode_mtp_b64_16k",
                    choices=["decode_mtp_b64_16k", "decode_b16_4k", "decode_b4_128k", "prefill_8k",
                             "prefill_chunk_128k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-indexer-topk", action="store_true",
                    help="decode step as three calls (indexer, top-k, attention) instead of the fused indexer+top-k")
    ap.add_argument("--no-graph", action="store_true", help="time eager steps (for counter-collection runs)")
    ap.add_argument("--crossover", action="store_true")
    ap.add_argument("--crossover-T", default="1024,2048,4096,8192,16384",
                    help="prefix lengths of the crossover sweep")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cache-write", action="store_true", help="time the cache writes and query quantisation")
    ap.add_argument("--projections", action="store_true", help="time the indexer's q / w / k projections")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the DSA "
              "hot path here is a single-GPU library with no collectives.", file=sys.stderr)
        raise SystemExit(2)
    if args.copy_calibration:
        run_copy_calibration(args)
    elif args.cache_write:
        run_cache_bench(args)
    elif args.projections:
        run_projection_bench(args)
    elif args.crossover:
        run_crossover(args)
    elif args.workload.startswith("prefill"):
        run_prefill_bench(args)
    else:
        run_decode_bench(args)


if __name__ == "__main__":
    main()
