"""GPU gather against the CPU oracle and torch indexing, bit for bit.

Cases follow the unit-test list of MindSpore hyper-parallel PR #1094: equal
to two-tensor advanced indexing for one batch and several, batches do not
mix, shape and dtype, a non-contiguous key, repeated positions, and the
selection chain (top-k then gather) at batch 1 and batch 3.
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import workloads as W
from parity import gpu_bits, oracle_topk, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    return d


def host_key(k: torch.Tensor) -> np.ndarray:
    return P.bf16_bits(k) if k.dtype == torch.bfloat16 else k.numpy()


def check_gather(dsel, orc, name, key, pos):
    say(f"[gather] {name} key={tuple(key.shape)} stride={key.stride()} pos={tuple(pos.shape)} {pos.dtype}")
    out = dsel.gather_rows(to_device(key), pos.cuda())
    torch.cuda.synchronize()
    got = gpu_bits(out)
    want = orc.gather(host_key(key), pos.numpy())
    assert got.shape == want.shape
    assert np.array_equal(got, want.view(got.dtype)), f"{name}: gathered rows differ"
    return out


@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
@pytest.mark.parametrize("ptype", [torch.int32, torch.int64])
def test_equals_advanced_indexing(dsel, orc, B, dt, ptype):
    key = W.random_keys(100 + B, B, 777, 128, dt)
    pos = W.random_positions(200 + B, B, 33, 65, 777, ptype, oob=True)
    out = check_gather(dsel, orc, f"adv/B{B}/{dt}/{ptype}", key, pos)
    safe = pos.long().clamp(0, 776)
    bidx = torch.arange(B).view(B, 1, 1).expand_as(safe)
    assert torch.equal(out.cpu(), key[bidx, safe])
    assert out.shape == (B, 33, 65, 128) and out.dtype == key.dtype


def test_batches_do_not_mix(dsel, orc):
    B, L, D = 5, 64, 64
    key = torch.arange(B, dtype=torch.float32).view(B, 1, 1).expand(B, L, D).contiguous()
    pos = W.random_positions(7, B, 9, 31, L, torch.int32)
    out = check_gather(dsel, orc, "no-mix", key, pos).cpu()
    for b in range(B):
        assert (out[b] == b).all()


def test_noncontiguous_key_and_repeats(dsel, orc):
    key = W.random_keys(8, 2, 5000, 128, W.BF16, layout="transposed")
    assert not key.is_contiguous()
    pos = W.random_positions(9, 2, 17, 300, 5000, torch.int32)
    pos[:, :, ::3] = pos[:, :, :1]
    check_gather(dsel, orc, "transposed+repeats", key, pos)
    key = W.random_keys(10, 3, 400, 64, W.F32, layout="padded")
    pos = W.random_positions(11, 3, 5, 129, 400, torch.int64)
    check_gather(dsel, orc, "padded-rows", key, pos)


@pytest.mark.parametrize("D", [8, 24, 96, 512])
def test_other_row_widths(dsel, orc, D):
    key = W.random_keys(12 + D, 2, 300, D, W.BF16)
    pos = W.random_positions(13, 2, 7, 50, 300, torch.int32)
    check_gather(dsel, orc, f"D{D}", key, pos)


def test_strided_position_rows(dsel, orc):
    """A top-k index buffer with a padded row stride feeds the gather directly."""
    key = W.random_keys(14, 2, 1000, 128, W.BF16)
    buf = W.random_positions(15, 1, 2 * 6, 40, 1000, torch.int32)[0]
    view = buf[:, :37].reshape(2, 6, 37) if False else buf.view(2, 6, 40)[:, :, :37]
    out = dsel.gather_rows(key.cuda(), buf.cuda().view(2, 6, 40)[:, :, :37])
    torch.cuda.synchronize()
    want = orc.gather(host_key(key), np.ascontiguousarray(view.numpy()))
    assert np.array_equal(gpu_bits(out), want)


def test_empty(dsel):
    key = torch.zeros(2, 10, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, 0, 5, dtype=torch.int32, device="cuda")
    assert dsel.gather_rows(key, pos).shape == (2, 0, 5, 128)


@pytest.mark.parametrize("B", [1, 3])
def test_selection_chain(dsel, orc, B):
    """top-k then gather, against oracle top-k then oracle gather."""
    R, L, k = 40, 3000, 256
    x = W.random_rows(300 + B, B * R, L, W.BF16, "normal")
    re = W.random_row_end(301 + B, B * R, 100, L)
    key = W.random_keys(302 + B, B, L, 128, W.BF16)
    say(f"[chain] B={B}")
    _, idx, _ = dsel.topk(to_device(x), k, end=re.cuda(), return_value=False)
    out = dsel.gather_rows(to_device(key), idx.view(B, R, k))
    torch.cuda.synchronize()
    _, widx, _ = oracle_topk(orc, x, k, re, True, torch.int32, False)
    want = orc.gather(host_key(key), widx.reshape(B, R, k))
    assert np.array_equal(gpu_bits(out), want)


@pytest.mark.parametrize("cfg", [3, 5])
def test_workload_chain_full_size(dsel, orc, cfg):
    """The full prefill (4096 x 2048) and long-context (2 x 1024 x 16384) chains."""
    case = W.make_config(cfg)
    say(f"[chain] {case.name} full size")
    _, idx, _ = dsel.topk(case.x.cuda(), case.k, end=case.row_end.cuda(), return_value=False,
                          indices_type=case.indices_type)
    _, widx, _ = oracle_topk(orc, case.x, case.k, case.row_end, True, case.indices_type, False)
    B = case.gather_batch
    R = case.x.shape[0] // B
    pos_gpu = idx.view(B, R, case.k) if idx.is_contiguous() else idx.contiguous().view(B, R, case.k)
    pos_host = widx.reshape(B, R, case.k).copy()
    if case.repeat_every:
        pos_gpu = pos_gpu.clone()
        pos_gpu[:, :, ::case.repeat_every] = pos_gpu[:, :, :1]
        pos_host[:, :, ::case.repeat_every] = pos_host[:, :, :1]
    for ki, key in enumerate(case.keys):
        out = dsel.gather_rows(to_device(key), pos_gpu)
        torch.cuda.synchronize()
        want = orc.gather(host_key(key), pos_host)
        assert np.array_equal(gpu_bits(out), want), f"{case.name} key {ki}"
        del out
