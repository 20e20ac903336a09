"""Top-k fused with the key gather (dsel_topk_gather) against the oracle.

The reference is the chain on the CPU: the oracle's top-k (ascending
indices, or the value order for sorted_index 2), then the oracle's gather of
every key at those positions, clamped or zero-filled (MindSpore
hyper-parallel PR #1094: top-k, the masked fill, then
key[batch_ids, safe_positions]).  Indices, NaN flags and every gathered row
must match bit for bit.  Cases cover both fused kernels (one-wave bf16 rows,
whole rows) and the rows that run select-then-gather (fp32 one-wave rows,
split rows, value order), one to four keys, strided keys, both index types,
and the prefill and long-context workloads at full size.
"""
import numpy as np
import pytest
import torch

import oracle_pins as P
import workloads as W
from parity import gpu_bits, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    return d


def host_key(k: torch.Tensor) -> np.ndarray:
    return P.bf16_bits(k) if k.dtype == torch.bfloat16 else k.numpy()


def check_fused(dsel, orc, name, x, k, keys, rpb, row_end=None, by_value=False,
                indices_type=torch.int32, pad="clamp"):
    rows = x.shape[0]
    B = rows // rpb
    say(f"[fused] {name} x={tuple(x.shape)} {x.dtype} k={k} keys={[tuple(t.shape) for t in keys]} "
        f"rpb={rpb} by_value={by_value} idx={indices_type} pad={pad}")
    re = row_end.cuda() if row_end is not None else None
    idx, flag, outs = dsel.topk_gather(to_device(x), k, [to_device(t) for t in keys],
                                       rows_per_batch=rpb, end=re, by_value=by_value,
                                       indices_type=indices_type, pad=pad)
    torch.cuda.synchronize()
    it = np.int32 if indices_type == torch.int32 else np.int64
    _, widx, wflag = orc.topk(P.to_host(x), k, row_end=row_end.numpy() if row_end is not None else None,
                              sorted_index=2 if by_value else True, indices_type=it,
                              return_value=False)
    gidx = idx.cpu().numpy()
    assert np.array_equal(gidx, widx), f"{name}: indices differ"
    assert np.array_equal(flag.cpu().numpy(), wflag), f"{name}: NaN flags differ"
    for g, (kt, out) in enumerate(zip(keys, outs)):
        want = orc.gather(host_key(kt), widx.reshape(B, rpb, k), pad=pad)
        got = gpu_bits(out).reshape(want.shape)
        assert np.array_equal(got, want.view(got.dtype)), f"{name}: key {g} gathered rows differ"
    return idx, outs


def causal_end(rows, cols):
    return ((torch.arange(rows, dtype=torch.int64) + 1) * cols // rows).to(torch.int32)


@pytest.mark.parametrize("pad", ["clamp", "zero"])
@pytest.mark.parametrize("itype", [torch.int32, torch.int64])
def test_one_wave_rows(dsel, orc, itype, pad):
    """bf16 rows of at most 2048 columns (the one-wave kernel gathers), with
    causal row ends so short rows pad with -1; one and two keys, a strided
    key; k whose index slots fit the wave's stage and k that do not."""
    x = W.random_rows(0xF0, 96, 2000, W.BF16, "normal")
    W.plant_nans(x, 0xF1, 4)
    re = causal_end(96, 2000)
    ka = W.random_keys(0xF2, 4, 1500, 128, W.BF16)
    kb = W.random_keys(0xF3, 4, 2000, 64, W.BF16, "transposed")
    for k in (1, 300, 1024, 1500):
        check_fused(dsel, orc, f"wave/k{k}", x, k, [ka, kb], 24, re, indices_type=itype, pad=pad)
    k1 = W.random_keys(0xF8, 1, 2000, 64, W.BF16, "transposed")
    check_fused(dsel, orc, "wave/full-rows", x, 700, [k1], 96, None, indices_type=itype, pad=pad)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_whole_rows(dsel, orc, dt):
    """Rows of 2049 to 16384 columns (one workgroup per row gathers); fp32
    keys, four keys, ragged row ends, k up to 4096."""
    x = W.random_rows(0xF4, 40, 9000, dt, "ties")
    re = W.random_row_end(0xF5, 40, -5, 9100)
    keys = [W.random_keys(0xF6 + i, 5, 3000, 32 * (i + 1), W.F32 if i % 2 else W.BF16)
            for i in range(4)]
    for k in (512, 4096):
        check_fused(dsel, orc, f"whole/{dt}/k{k}", x, k, keys, 8, re)
    check_fused(dsel, orc, f"whole/{dt}/zero", x, 2000, keys[:1], 8, re, pad="zero")


def test_select_then_gather_rows(dsel, orc):
    """Rows whose kernel does not fuse the gather: fp32 one-wave rows, split
    rows (bf16 and fp32), and value order; the result is the same chain."""
    kk = W.random_keys(0xF7, 2, 70000, 128, W.BF16)
    xf = W.random_rows(0xF8, 8, 1500, W.F32, "normal")
    check_fused(dsel, orc, "chain/f32-wave", xf, 400, [kk], 4, causal_end(8, 1500))
    xs = W.random_rows(0xF9, 4, 70000, W.BF16, "normal")
    check_fused(dsel, orc, "chain/split-bf16", xs, 1024, [kk], 2, None, pad="zero")
    xs32 = W.random_rows(0xFA, 4, 70000, W.F32, "normal")
    check_fused(dsel, orc, "chain/split-f32", xs32, 2000, [kk], 2, causal_end(4, 70000),
                indices_type=torch.int64)
    xv = W.random_rows(0xFB, 16, 3000, W.BF16, "ties")
    check_fused(dsel, orc, "chain/by-value", xv, 500, [kk], 8, causal_end(16, 3000), by_value=True)


@pytest.mark.parametrize("pad", ["clamp", "zero"])
@pytest.mark.parametrize("cfg", [3, 5])
def test_workloads_full_size(dsel, orc, cfg, pad):
    """The prefill rows (4096 x 2048 causal, one key [1, 2048, 128]) and the
    long-context rows (2 x 1024 rows x 16384, two keys, one of them a
    strided view) at full size, the way the bench times them."""
    case = W.make_config(cfg)
    rpb = case.x.shape[0] // case.gather_batch
    check_fused(dsel, orc, f"cfg{cfg}", case.x, case.k, case.keys, rpb, case.row_end,
                indices_type=case.indices_type, pad=pad)


def test_matches_the_two_call_chain(dsel):
    """On the GPU: dsel_topk_gather equals topk then gather_rows (clamp)."""
    case = W.make_config(5)
    B = case.gather_batch
    x = case.x.cuda()
    re = case.row_end.cuda()
    keys = [k.cuda() for k in case.keys]
    idx, flag, outs = dsel.topk_gather(x, case.k, keys, rows_per_batch=x.shape[0] // B, end=re)
    _, idx2, flag2 = dsel.topk(x, case.k, end=re, return_value=False)
    assert torch.equal(idx, idx2) and torch.equal(flag, flag2)
    pos = idx2.contiguous().view(B, -1, case.k)
    for kt, out in zip(keys, outs):
        ref = dsel.gather_rows(kt, pos)
        assert torch.equal(out.view(torch.int16), ref.reshape(out.shape).view(torch.int16))


def test_argument_errors(dsel):
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    key = torch.zeros(2, 10, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        dsel.topk_gather(x, 4, [key], rows_per_batch=3)
    with pytest.raises(ValueError):
        dsel.topk_gather(x, 4, [], rows_per_batch=4)
    with pytest.raises(ValueError):
        dsel.topk_gather(x, 4, [key], rows_per_batch=4, pad="nan")
    with pytest.raises(dsel.DselError):
        dsel.topk_gather(x, 4, [key[:, :, :60]], rows_per_batch=4)  # 120-byte rows
