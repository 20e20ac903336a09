"""Top-k and gather captured in a HIP graph give the eager result on every replay.

The benchmark times graph replays, so this pins that a captured call (split
rows included: their workspace must come back zeroed for the next replay)
reproduces the eager output, with eager work and synchronisations between
replays.
"""
import pytest
import torch

import workloads as W
from parity import say, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as dsel
    dev = torch.device("cuda")
    s = torch.cuda.Stream()
    x = to_device(W.random_rows(91, 4, 204800, W.BF16, "normal"))      # split rows
    xs = to_device(W.random_rows(92, 300, 3000, W.F32, "ties"))         # one workgroup per row
    re = W.random_row_end(93, 300, 0, 3000).to(dev)
    key = W.random_keys(94, 3, 3000, 128).to(dev)
    say("[graph] eager reference")
    with torch.cuda.stream(s):
        ev, ei, ef = dsel.topk(x, 1024, sorted_index=True, stream=s)
        _, ei2, ef2 = dsel.topk(xs, 100, end=re, return_value=False, stream=s)
        eg = dsel.gather_rows(key, ei2.view(3, 100, 100), stream=s)
        evv, eiv, _ = dsel.topk(xs, 700, end=re, by_value=True, stream=s)   # value order
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gv, gi, gf = dsel.topk(x, 1024, sorted_index=True, stream=s)
        _, gi2, gf2 = dsel.topk(xs, 100, end=re, return_value=False, stream=s)
        gg = dsel.gather_rows(key, gi2.view(3, 100, 100), stream=s)
        gvv, giv, _ = dsel.topk(xs, 700, end=re, by_value=True, stream=s)
    for rep in range(4):
        say(f"[graph] replay {rep}")
        for t in (gv, gi, gf, gi2, gf2, gg, gvv, giv):
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gi, ei) and torch.equal(gv.view(torch.int16), ev.view(torch.int16))
        assert torch.equal(gf, ef) and torch.equal(gi2, ei2) and torch.equal(gf2, ef2)
        assert torch.equal(gg.view(torch.int16), eg.view(torch.int16))
        assert torch.equal(giv, eiv) and torch.equal(gvv.view(torch.int32), evv.view(torch.int32))
        # eager work between replays on the same workspace
        dsel.topk(x, 512, stream=s)
        s.synchronize()
