"""The benchmark's analytic cost model against the figures the handbook page prints (CPU only).

bench.per_layer_cost is built from the same unit costs as the benchmark's algorithmic bytes and
FLOPs (attention_pair_flops, indexer_pair_flops, the 1152-byte latent row and the 132-byte FP8
indexer key); tests/golden/handbook_cost_table.json holds the page's printed table. Each printed
number must be reproduced at the precision it is printed with, so a wrong unit cost (a missing
rope term, bf16 vs FP8 bytes, the scale's 4 bytes, the wrong k clamp) fails here.
"""
import json
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "handbook_cost_table.json")) as f:
        return json.load(f)


def _printed(x, ndigits):
    return round(x, ndigits)


def test_unit_costs_match_the_page():
    g = _golden()["pair"]
    assert round(bench.attention_pair_flops() / 1e3) == g["mla_kflops"]
    assert round(bench.indexer_pair_flops() / 1e3) == g["indexer_kflops"]
    assert round(100 * bench.IDX_KEY_BYTES / bench.KV_ROW_BYTES) == g["index_cache_extra_percent"]


def test_per_layer_costs_reproduce_the_printed_table():
    for row in _golden()["rows"]:
        c = bench.per_layer_cost(row["L"])
        dec = [x / 1e9 for x in c["decode_flops"]]
        rd = [x / 2 ** 20 for x in c["decode_bytes"]]
        pre = [x / 1e12 for x in c["prefill_flops"]]
        assert [_printed(x, 2) for x in dec] == row["decode_gflops"], (row["L"], dec)
        assert _printed(dec[0] / dec[1], 1) == row["decode_gflops_ratio"]
        assert [_printed(x, 1) for x in rd] == row["decode_mib"], (row["L"], rd)
        assert _printed(rd[0] / rd[1], 1) == row["decode_mib_ratio"]
        assert [_printed(x, 1) for x in pre] == row["prefill_tflops"], (row["L"], pre)
        assert _printed(pre[0] / pre[1], 1) == row["prefill_ratio"]


def test_decode_step_model_uses_the_same_unit_costs():
    """One request, one query row: the step model's indexer FLOPs and cache bytes are the per-layer
    model's DSA decode figures (plus the query/output and indexer-query bytes the step also moves)."""
    L, k = 16384, 2048
    c = bench.per_layer_cost(L, k)
    fl = bench.decode_step_flops(1, 1, [L], k)
    by = bench.decode_step_bytes(1, 1, [L], k)
    assert fl["indexer"] + fl["mla"] == c["decode_flops"][1]
    q_out = 128 * 576 * 2 + 128 * 512 * 2
    q8_w = 64 * 128 + 64 * 4
    assert by["step"] == c["decode_bytes"][1] + q_out + q8_w


def test_measured_traffic_only_for_the_measured_workload_and_source():
    """The bench's roofline takes HBM bytes from the committed counter summary only for the
    workload and kernel source the counters were taken on."""
    with open(os.path.join(HERE, "..", "profiles", "traffic.json")) as f:
        t = json.load(f)
    ent = t["sparse_mla_decode"]
    got = bench.measured_traffic("sparse_mla_decode", ent["workload"])
    assert got == (ent["bytes_per_launch"] if ent["source_hash"] == bench._src_hash() else None)
    assert bench.measured_traffic("sparse_mla_decode", "decode_b16_4k") is None
    assert bench.measured_traffic("no_such_kernel", ent["workload"]) is None
