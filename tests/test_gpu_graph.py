"""The decode step (indexer -> top-k -> sparse attention, four kernel launches) captured into HIP
graphs, as the benchmark runs it: every replay must reproduce the eager result exactly, with eager
work and synchronisations between replays and the outputs clobbered before each one."""
import numpy as np
import pytest
import torch

import bench
import workloads

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    print("case: decode step graph replays", flush=True)
    q_pos = np.array([4999, 5000, 3000, 3001, 700, 701, 2047, 2048], np.int32)  # 4 requests x 2 rows
    w = workloads.make_random(4, 2, q_pos, 5001, seed=77, permute_pages=True, extra_pages=3)
    step = bench.DecodeStep(w, copies=2)
    for c in range(2):
        step.run(c)
    torch.cuda.synchronize()
    eager = [(d["scores"].clone(), d["idx"].clone(), d["out"].clone()) for d in step.copies]
    graphs = step.capture()
    for rep in range(3):
        for c, g in enumerate(graphs):
            d = step.copies[c]
            d["idx"].fill_(-7)
            d["out"].zero_()
            d["scores"].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(d["idx"], eager[c][1]), (rep, c)
            assert torch.equal(d["out"].view(torch.int16), eager[c][2].view(torch.int16)), (rep, c)
            for r, t in enumerate(q_pos):  # scores past q_pos are unspecified
                assert torch.equal(d["scores"][r, : t + 1], eager[c][0][r, : t + 1]), (rep, c, r)
