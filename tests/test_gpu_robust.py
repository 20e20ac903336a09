"""Failure reporting and stream / workspace handling of the binding, on the GPU.

* A split-row rendezvous that gives up (forced from the host with a tiny
  spin limit, so every kernel still exits normally) is reported by the call
  (``check=True``) and the workspace is reset: the next call is exact.
* ``stream=s`` with ``s`` not the current stream: outputs and workspace are
  allocated and zeroed on ``s``.
* A HIP graph captured with one workspace still replays correctly after a
  later call on the same stream needed a bigger one.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_topk, gpu_bits, oracle_topk, say, to_device, valid_lengths
from test_gpu_topk import assert_workspaces_clean, blocks_per_row, check_case, one_exchange

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    return d


class spin_limit:
    """Set DSEL_SPIN_LIMIT (polls of a split-row rendezvous) inside a block."""

    def __init__(self, n):
        self.n = n

    def __enter__(self):
        self.old = os.environ.get("DSEL_SPIN_LIMIT")
        os.environ["DSEL_SPIN_LIMIT"] = str(self.n)

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("DSEL_SPIN_LIMIT", None)
        else:
            os.environ["DSEL_SPIN_LIMIT"] = self.old


@pytest.mark.parametrize("one", [None, False])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_rendezvous_give_up_is_reported(dsel, orc, dt, one):
    """With one poll allowed, the first workgroup of a row to arrive cannot
    see its 64 peers: it gives up, the kernels finish, check=True raises
    DSEL_ERR_SPLIT, and the reset workspace serves the next call exactly."""
    x = W.random_rows(171, 4, 204800, dt, "normal")
    xd = to_device(x)
    torch.cuda.synchronize()
    say(f"[robust] give-up dt={dt} one={one}")
    with spin_limit(1), blocks_per_row(64), one_exchange(one):
        with pytest.raises(dsel.DselError) as e:
            dsel.topk(xd, 1024, sorted_index=True, check=True)
    assert e.value.code == dsel.DSEL_ERR_SPLIT
    assert_workspaces_clean(dsel)
    check_case(dsel, orc, f"after-give-up/{dt}", x, 1024, None, True, torch.int32, True, 64, one)
    dsel.check_workspaces()  # nothing to report now
    assert_workspaces_clean(dsel)


def test_explicit_stream_not_current(dsel, orc):
    """stream=s while the default stream is current: every output and the
    workspace come from s, and the result is exact (split bf16 and fp32
    rows, and one-wave rows)."""
    s = torch.cuda.Stream()
    cases = [(W.random_rows(181, 6, 100000, W.BF16, "normal"), 777, True),
             (W.random_rows(182, 3, 70000, W.F32, "ties"), 2000, False),
             (W.random_rows(183, 50, 1500, W.BF16, "normal"), 300, True)]
    for x, k, sorted_index in cases:
        say(f"[robust] stream shape={tuple(x.shape)} k={k}")
        xd = to_device(x)
        torch.cuda.synchronize()
        assert torch.cuda.current_stream() != s
        v, i, f = dsel.topk(xd, k, sorted_index=sorted_index, stream=s)
        s.synchronize()
        got = (gpu_bits(v), i.cpu().numpy(), f.cpu().numpy())
        want = oracle_topk(orc, x, k, None, sorted_index, torch.int32, True)
        compare_topk(got, want, valid_lengths(x.shape[0], x.shape[1], None), k, sorted_index,
                     "explicit stream")
    torch.cuda.synchronize()
    assert_workspaces_clean(dsel)


def test_graph_survives_workspace_growth(dsel):
    """A graph captured with a small workspace, then an eager fp32 split call
    on the same stream that needs a bigger one: replays of the graph still
    match the eager result (the old workspace is kept alive)."""
    dsel._WORKSPACES.clear()
    s = torch.cuda.Stream()
    x = to_device(W.random_rows(191, 4, 204800, W.BF16, "normal"))
    xf = to_device(W.random_rows(192, 16, 129280, W.F32, "normal"))
    with torch.cuda.stream(s):
        ev, ei, ef = dsel.topk(x, 1024, sorted_index=True, stream=s)
    s.synchronize()
    small = dsel._WORKSPACES[(x.device.index, int(s.cuda_stream))].numel()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gv, gi, gf = dsel.topk(x, 1024, sorted_index=True, stream=s)
    with torch.cuda.stream(s):
        fv, fi, _ = dsel.topk(xf, 4096, indices_type=torch.int64, stream=s)
    s.synchronize()
    big = dsel._WORKSPACES[(x.device.index, int(s.cuda_stream))].numel()
    assert big > small, "the fp32 call should have needed a bigger workspace"
    for rep in range(3):
        say(f"[robust] replay {rep} after workspace growth")
        for t in (gv, gi, gf):
            t.fill_(-7)
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert torch.equal(gi, ei) and torch.equal(gv.view(torch.int16), ev.view(torch.int16))
        assert torch.equal(gf, ef)
        with torch.cuda.stream(s):
            fv2, fi2, _ = dsel.topk(xf, 4096, indices_type=torch.int64, stream=s)
        s.synchronize()
        assert torch.equal(fi2, fi)
    del g
    torch.cuda.synchronize()
    assert_workspaces_clean(dsel)
