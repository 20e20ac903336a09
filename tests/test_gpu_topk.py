"""GPU top-k against the CPU oracle, bit for bit, through the C ABI binding."""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle_pins as P
import workloads as W
from parity import compare_topk, gpu_bits, oracle_topk, say, to_device, valid_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    return d


class blocks_per_row:
    """Force the number of workgroups per row (DSEL_BLOCKS_PER_ROW) inside a block."""

    def __init__(self, g):
        self.g = g

    def __enter__(self):
        self.old = os.environ.get("DSEL_BLOCKS_PER_ROW")
        if self.g is None:
            os.environ.pop("DSEL_BLOCKS_PER_ROW", None)
        else:
            os.environ["DSEL_BLOCKS_PER_ROW"] = str(self.g)

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("DSEL_BLOCKS_PER_ROW", None)
        else:
            os.environ["DSEL_BLOCKS_PER_ROW"] = self.old


class one_exchange:
    """Turn the one-exchange select of split bf16 rows on or off
    (DSEL_SPLIT_ONE_EXCHANGE) inside a block; None keeps the default (on)."""

    def __init__(self, on):
        self.on = on

    def __enter__(self):
        self.old = os.environ.get("DSEL_SPLIT_ONE_EXCHANGE")
        if self.on is None:
            os.environ.pop("DSEL_SPLIT_ONE_EXCHANGE", None)
        else:
            os.environ["DSEL_SPLIT_ONE_EXCHANGE"] = "1" if self.on else "0"

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("DSEL_SPLIT_ONE_EXCHANGE", None)
        else:
            os.environ["DSEL_SPLIT_ONE_EXCHANGE"] = self.old


def assert_workspaces_clean(dsel):
    """Every workspace is back in the state the next call needs: word 0 (error
    bits) clear and every word past the exchange region (the 64-word header,
    then 8 * CUs * 544 words of per-workgroup scratch) zero."""
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    region = (64 + 8 * cus * 544) * 4
    for ws in dsel._WORKSPACES.values():
        assert int(ws[:4].count_nonzero()) == 0, "an error bit is set (a rendezvous timed out)"
        assert int(ws[region:].count_nonzero()) == 0, "row slots must be zero after a call"


def run_gpu(dsel, x, k, row_end, sorted_index, indices_type, return_value, output_idx=None,
            row_order=None):
    xd = to_device(x)
    re = row_end.cuda() if row_end is not None else None
    v, i, f = dsel.topk(xd, k, end=re, sorted_index=sorted_index, indices_type=indices_type,
                        return_value=return_value, output_idx=output_idx, row_order=row_order)
    torch.cuda.synchronize()
    return (gpu_bits(v) if v is not None else None, i.cpu().numpy(), f.cpu().numpy())


def check_case(dsel, orc, name, x, k, row_end=None, sorted_index=False,
               indices_type=torch.int32, return_value=True, G=None, one=None, row_order=None):
    say(f"[topk] {name} shape={tuple(x.shape)} stride={x.stride()} k={k} G={G} one={one} "
        f"sorted={sorted_index} idx={indices_type} val={return_value} order={row_order}")
    with blocks_per_row(G), one_exchange(one):
        got = run_gpu(dsel, x, k, row_end, sorted_index, indices_type, return_value,
                      row_order=row_order)
    want = oracle_topk(orc, x, k, row_end, sorted_index, indices_type, return_value)
    n = valid_lengths(x.shape[0], x.shape[1], row_end)
    compare_topk(got, want, n, k, sorted_index, name)
    # the GPU always returns ascending indices
    gi = got[1].astype(np.int64)
    for r in range(min(gi.shape[0], 64)):
        c = int(min(k, n[r]))
        assert (np.diff(gi[r, :c]) > 0).all()
    return got


SMALL = [
    # name, rows, cols, dtype, dist, k
    ("normal_bf16", 9, 3000, W.BF16, "normal", 100),
    ("normal_f32", 9, 3000, W.F32, "normal", 100),
    ("ties_bf16", 7, 5000, W.BF16, "ties", 777),
    ("ties_f32", 7, 5000, W.F32, "ties", 4096),
    ("equal_bf16", 3, 4100, W.BF16, "equal", 1000),
    ("equal_f32", 3, 4100, W.F32, "equal", 4096),
    ("ascending_f32", 4, 6000, W.F32, "ascending", 300),
    ("descending_bf16", 4, 6000, W.BF16, "descending", 300),
    ("special_bf16", 11, 2500, W.BF16, "special", 64),
    ("special_f32", 11, 2500, W.F32, "special", 64),
    ("special_bf16_bigk", 5, 2500, W.BF16, "special", 2000),
    ("special_f32_bigk", 5, 2500, W.F32, "special", 2000),
    ("narrow_bf16", 5, 16384, W.BF16, "narrow", 2000),
    ("ragged_bf16", 6, 2043, W.BF16, "normal", 17),
    ("ragged_f32", 6, 1037, W.F32, "normal", 1),
    ("k_ge_cols", 5, 300, W.F32, "normal", 512),
    ("one_col", 5, 1, W.BF16, "normal", 3),
]


@pytest.mark.parametrize("G,one", [(None, None), (3, None), (7, None), (3, False), (7, False)])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_small_cases(dsel, orc, case, G, one):
    name, rows, cols, dt, dist, k = case
    x = W.random_rows(zlib.crc32(name.encode()) & 0xFFFF, rows, cols, dt, dist)
    for ret in (True, False):
        check_case(dsel, orc, f"{name}/G{G}/val{int(ret)}", x, k, None, False, torch.int32, ret,
                   G, one)


@pytest.mark.parametrize("one", [True, False])
@pytest.mark.parametrize("G", [7, 25, 64])
def test_split_one_exchange(dsel, orc, G, one):
    """bf16 rows split over G workgroups, through the one-exchange select
    (on) and the multi-pass select (off): full chunks, a short last chunk,
    chunks wholly past the row end, rows too short for any chunk to hold k
    keys, a NaN row and a row with a few huge values (both must leave the
    one exchange for the multi-pass select), k from 1 to 4096."""
    rows, cols = 9, 100000
    x = W.random_rows(131 + G, rows, cols, W.BF16, "normal")
    x[6, 4321] = float("nan")
    x[7, [5, 50000, 99990]] = torch.tensor([300.0, -250.0, 1e30]).to(x.dtype)
    ends = [100000, 99999, 61234, 40001, 20000, 8193, 100000, 77777, 4097]
    re = torch.tensor(ends, dtype=torch.int32)
    for k, sorted_index, itype, ret in ((1, False, torch.int32, True),
                                        (100, True, torch.int64, True),
                                        (1024, True, torch.int32, True),
                                        (1024, False, torch.int32, False),
                                        (4096, False, torch.int32, True)):
        check_case(dsel, orc, f"one/G{G}/on{int(one)}/k{k}", x, k, re, sorted_index, itype, ret,
                   G, one)
    assert_workspaces_clean(dsel)


@pytest.mark.parametrize("G", [None, 4])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_row_end_and_nan(dsel, orc, dt, G):
    x = W.random_rows(21, 64, 3000, dt, "normal")
    W.plant_nans(x, 22, 40)
    re = W.random_row_end(23, 64, -50, 3100)
    re[:4] = torch.tensor([0, 200, 201, 3000], dtype=torch.int32)
    check_case(dsel, orc, f"row_end_nan/{dt}", x, 200, re, True, torch.int64, True, G)
    check_case(dsel, orc, f"row_end_nan/{dt}/idx-only", x, 200, re, False, torch.int32, False, G)


@pytest.mark.parametrize("G", [None, 4, 7])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_nan_just_past_row_end(dsel, orc, dt, G):
    """A NaN at column n (just past a row's end) is out of range: no flag, and
    it must not reach the selection; odd n puts it in the same 32-bit word as
    the last valid bf16 element."""
    rows, cols = 24, 3001
    x = W.random_rows(25, rows, cols, dt, "normal")
    ends = [1001, 1003, 1500, 1501, 2047, 2049, 2999, 3000, 3001, 257, 511, 777,
            1025, 1999, 2001, 2221, 2500, 2501, 2887, 2901, 1203, 1333, 1777, 2993]
    re = torch.tensor(ends, dtype=torch.int32)
    for r, n in enumerate(ends):
        if n < cols:
            x[r, n] = float("nan")
    got = check_case(dsel, orc, f"nan_past_end/{dt}", x, 200, re, False, torch.int32, True, G)
    assert not got[2].any(), "no row holds a NaN in range"


@pytest.mark.parametrize("G", [4, 8])
def test_split_f32_nan_in_each_load(dsel, orc, G):
    """fp32 split rows whose NaNs sit in the loads a chunk histograms (every
    fourth 1024-column load of a chunk, load 0 first) and in the loads it
    does not, positive and negative NaN payloads, one or several per row,
    up to the chunk's partial last load."""
    rows, cols = 8, 40000
    x = W.random_rows(131, rows, cols, W.F32, "normal")
    xi = x.view(torch.int32)
    chunk = cols // G
    neg_nan = -4194304  # 0xFFC00000
    # row 0: no NaN; 1: load 1 of chunk 1 (not sampled); 2: load 0 of chunk 2
    # (sampled); 3: the last column; 4: three loads not sampled, over two
    # chunks; 5: a negative NaN in load 5; 6: sampled and not sampled; 7:
    # load 2 and a negative NaN in load 3 of chunk 0
    x[1, chunk + 1500] = float("nan")
    x[2, 2 * chunk + 100] = float("nan")
    x[3, cols - 1] = float("nan")
    x[4, 1100] = float("nan")
    x[4, 3 * 1024 + 7] = float("nan")
    x[4, chunk + 2 * 1024 + 500] = float("nan")
    xi[5, 5 * 1024 + 33] = neg_nan
    x[6, 4 * 1024 + 1] = float("nan")
    x[6, 6 * 1024 + 2] = float("nan")
    x[7, 2 * 1024 + 9] = float("nan")
    xi[7, 3 * 1024 + 10] = neg_nan
    re = torch.tensor([cols] * 7 + [cols - 777], dtype=torch.int32)
    for k, sorted_index, itype, ret in ((2000, True, torch.int64, True), (37, False, torch.int32, True),
                                        (4096, False, torch.int32, False)):
        got = check_case(dsel, orc, f"f32_nan_loads/G{G}/k{k}", x, k, re, sorted_index, itype, ret, G)
        assert got[2].tolist() == [0, 1, 1, 1, 1, 1, 1, 1]
    assert_workspaces_clean(dsel)


@pytest.mark.parametrize("G", [4, 8])
def test_split_f32_window_bin_capacity(dsel, orc, G):
    """fp32 split rows whose boundary bin holds exactly as many keys as one
    window bin of a workgroup's exchange area takes (341), and one more, in
    one chunk: the first row goes through the window exchange, the second
    overflows the bin and takes the multi-pass select; both exact."""
    rows, cols = 4, 40000
    g = torch.Generator().manual_seed(151)
    x = -20.0 - torch.rand(rows, cols, generator=g)  # far below the boundary bin
    chunk = cols // G
    k0 = 200
    for r, m in enumerate((341, 342, 340, 700)):
        # values in [1.5, 1.625), one 12-bit key bin: m of them in chunk 1,
        # three times each chunk's share of k in every other chunk (so that
        # every chunk's window holds the bin)
        for c in range(G):
            cnt = m if c == 1 else 3 * (k0 // G)
            x[r, c * chunk + torch.randperm(chunk, generator=g)[:cnt]] = \
                1.5 + 0.12 * torch.rand(cnt, generator=g)
    for k in (k0, 150):
        check_case(dsel, orc, f"f32_bin_cap/G{G}/k{k}", x, k, None, True, torch.int64, True, G)
    assert_workspaces_clean(dsel)


@pytest.mark.parametrize("G", [4, 8])
def test_split_f32_boundary_among_special_values(dsel, orc, G):
    """fp32 split rows without NaN whose k-th largest value falls among
    denormals, signed zeros or infinities (the exchange compares raw floats
    before it makes keys): -0 and +0 tie, denormals of both signs order by
    value, -inf and +inf sit at the ends."""
    rows, cols = 6, 40000
    g = torch.Generator().manual_seed(141)
    x = -1.0 - torch.rand(rows, cols, generator=g)  # every value below -1 ...
    tiny = torch.tensor(1e-45, dtype=torch.float32)  # the smallest denormal
    mags = torch.randint(1, 1 << 20, (rows, cols), generator=g).float() * tiny
    sign = torch.where(torch.rand(rows, cols, generator=g) < 0.5, -1.0, 1.0)
    pick = torch.rand(rows, cols, generator=g)
    # ... but these: row 0 denormals of both signs; row 1 signed zeros; row 2
    # zeros and denormals; row 3 +inf and denormals; row 4 mostly -inf; row 5
    # the largest negative denormal and -0
    x[0] = torch.where(pick[0] < 0.15, mags[0] * sign[0], x[0])
    x[1] = torch.where(pick[1] < 0.10, torch.where(sign[1] > 0, 0.0, -0.0), x[1])
    x[2] = torch.where(pick[2] < 0.05, torch.where(sign[2] > 0, 0.0, -0.0),
                       torch.where(pick[2] < 0.12, mags[2] * sign[2], x[2]))
    x[3] = torch.where(pick[3] < 0.02, float("inf"), torch.where(pick[3] < 0.2, mags[3], x[3]))
    x[4] = torch.where(pick[4] < 0.95, float("-inf"), x[4])
    x[4, :5] = float("-inf")
    x[5] = torch.where(pick[5] < 0.04, -tiny, torch.where(pick[5] < 0.08, -0.0, x[5]))
    assert not torch.isnan(x).any()
    re = torch.tensor([cols, cols - 3, cols, 31111, cols, cols - 1], dtype=torch.int32)
    for k, sorted_index, itype, ret in ((4096, True, torch.int64, True), (1000, False, torch.int32, True),
                                        (3000, True, torch.int32, True)):
        got = check_case(dsel, orc, f"f32_special_bound/G{G}/k{k}", x, k, re, sorted_index, itype, ret, G)
        assert not got[2].any()
    assert_workspaces_clean(dsel)


@pytest.mark.parametrize("dist", ["ascending", "descending", "ties", "narrow"])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_split_crowded_chunks(dsel, orc, dt, dist):
    """Split rows whose candidates crowd into one chunk (ascending: the last,
    descending: the first), so one workgroup's list overflows and it re-reads
    its range while the others use their lists; ties and narrow ranges put
    many keys at the boundary."""
    x = W.random_rows(81 + len(dist), 5, 40000, dt, dist)
    for k, G in ((2000, 8), (4096, 5), (37, 16)):
        for one in (None, False):
            check_case(dsel, orc, f"crowded/{dist}/{dt}/k{k}/G{G}", x, k, None, True,
                       torch.int64, True, G, one)


@pytest.mark.parametrize("G", [40, 80])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_split_many_workgroups(dsel, orc, dt, G):
    """Rows split over many workgroups (short chunks, most of them without a
    candidate), with ragged row ends."""
    x = W.random_rows(91 + G, 3, 100000, dt, "normal")
    re = torch.tensor([100000, 77777, 3001], dtype=torch.int32)
    for k, sorted_index in ((1000, True), (64, False)):
        for one in (None, False):
            check_case(dsel, orc, f"many/{dt}/G{G}/k{k}", x, k, re, sorted_index, torch.int32,
                       True, G, one)


@pytest.mark.parametrize("dist", ["normal", "ties", "equal", "ascending", "descending",
                                  "narrow", "special"])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_long_whole_rows(dsel, orc, dt, dist):
    """Whole rows of up to 16384 columns (the widest one workgroup takes)
    with ragged ends from 2048 to 16384, every value distribution, NaN rows,
    k from 1 to 2000."""
    rows, cols = 24, 16384
    x = W.random_rows(101 + len(dist), rows, cols, dt, dist)
    W.plant_nans(x, 102, 3)
    ends = [16384, 16383, 9000, 8191, 4096, 4095, 5001, 12345, 16000, 7777, 3000, 2048,
            16384, 10000, 4500, 6001, 15999, 8192, 4097, 11111, 13000, 2500, 14000, 9999]
    re = torch.tensor(ends, dtype=torch.int32)
    for k, sorted_index, itype, ret in ((1, False, torch.int32, True), (64, True, torch.int64, True),
                                        (500, False, torch.int32, False), (2000, True, torch.int32, True)):
        check_case(dsel, orc, f"long/{dist}/{dt}/k{k}", x, k, re, sorted_index, itype, ret)


@pytest.mark.parametrize("cols", [1, 37, 512, 513, 1024, 1500, 2048])
@pytest.mark.parametrize("dist", ["normal", "ties", "equal", "special", "ascending"])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_short_rows_one_wave(dsel, orc, dt, dist, cols):
    """Rows of at most 2048 columns, one wave each: ragged ends, NaN rows,
    every output form, k below, at and above the row length."""
    rows = 70
    x = W.random_rows(111 + cols + len(dist), rows, cols, dt, dist)
    W.plant_nans(x, 112 + cols, 5)
    re = W.random_row_end(113 + cols, rows, -3, cols + 3)
    re[:3] = torch.tensor([cols, 0, max(cols - 1, 0)], dtype=torch.int32)
    for k, sorted_index, itype, ret in ((1, False, torch.int32, True), (17, True, torch.int64, True),
                                        (max(cols // 2, 1), False, torch.int32, False),
                                        (cols, True, torch.int32, True), (cols + 5, False, torch.int64, True)):
        if k > 4096:
            continue
        check_case(dsel, orc, f"wave/{dist}/{dt}/c{cols}/k{k}", x, k, re, sorted_index, itype, ret)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_padded_stride(dsel, orc, dt):
    x = W.random_rows(31, 12, 2000, dt, "normal", stride=2048)
    assert not x.is_contiguous()
    check_case(dsel, orc, f"padded/{dt}", x, 333, None, True, torch.int32, True)
    check_case(dsel, orc, f"padded/{dt}/split", x, 333, None, True, torch.int32, True, G=5)


def test_k_max_and_long_rows(dsel, orc):
    x = W.random_rows(41, 3, 70000, W.F32, "normal")
    check_case(dsel, orc, "k4096_long_f32", x, 4096, None, False, torch.int64, True)
    x = W.random_rows(42, 2, 100000, W.BF16, "ties")
    check_case(dsel, orc, "k4096_long_bf16_ties", x, 4096, None, True, torch.int32, True)


def test_empty_rows(dsel):
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    v, i, f = dsel.topk(x, 8)
    assert i.shape == (0, 8) and f.shape == (0,)


def test_caller_owned_index_buffer(dsel, orc):
    x = W.random_rows(51, 10, 4000, W.BF16, "normal")
    buf = torch.full((10, 520), 7, dtype=torch.int32, device="cuda")
    v, i, f = dsel.topk(x.cuda(), 500, output_idx=buf, return_value=False)
    torch.cuda.synchronize()
    assert i.data_ptr() == buf.data_ptr()
    assert (buf[:, 500:] == 7).all(), "slots beyond k must be untouched"
    want = oracle_topk(orc, x, 500, None, True, torch.int32, False)
    assert np.array_equal(buf[:, :500].cpu().numpy(), want[1])


def test_run_to_run_identical(dsel):
    x = W.random_rows(61, 16, 40000, W.BF16, "ties").cuda()
    a = dsel.topk(x, 1024)
    b = dsel.topk(x, 1024)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))


def test_errors(dsel):
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsel.DselError) as e:
        dsel.topk(x, 0)
    assert e.value.code == -2
    with pytest.raises(dsel.DselError) as e:
        dsel.topk(x, 4097)
    assert e.value.code == -2
    xs = torch.zeros(4, 70, dtype=torch.bfloat16, device="cuda")[:, :65]  # stride 140 B
    with pytest.raises(dsel.DselError) as e:
        dsel.topk(xs, 4)
    assert e.value.code == -3


def test_workspace_reuse(dsel, orc):
    """One workspace serves calls of different shapes (so different per-row
    slot layouts) back to back: each call returns its slots to zero, and no
    rendezvous times out (error word 0 stays clear)."""
    dsel._WORKSPACES.clear()
    cases = [(W.random_rows(71, 8, 50000, W.F32, "normal"), 100, 6),
             (W.random_rows(72, 8, 50000, W.F32, "normal"), 2000, 6),
             (W.random_rows(73, 5, 30000, W.BF16, "ties"), 1500, 9),
             (W.random_rows(74, 8, 50000, W.F32, "equal"), 300, 4),
             (W.random_rows(71, 8, 50000, W.F32, "normal"), 100, 6)]
    cases += [(W.random_rows(75, 4, 60000, W.BF16, "normal"), 1024, 8),
              (W.random_rows(76, 4, 60000, W.BF16, "normal"), 64, 20),
              (W.random_rows(73, 5, 30000, W.BF16, "ties"), 1500, 9)]
    for i, (x, k, G) in enumerate(cases):
        check_case(dsel, orc, f"reuse{i}", x, k, None, False, torch.int32, True, G)
    assert_workspaces_clean(dsel)


# ---------------------------------------------------------------------------
# the five named workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_topk_full_size(dsel, orc, cfg):
    case = W.make_config(cfg)
    check_case(dsel, orc, case.name, case.x, case.k, case.row_end, case.sorted_index,
               case.indices_type, case.return_value)


def test_workload_split_path_cfg1(dsel, orc):
    case = W.make_config(1)
    for G in (1, 4):
        check_case(dsel, orc, f"cfg1/G{G}", case.x, case.k, None, False, torch.int32, True, G)


def check_value_order(dsel, orc, name, x, k, row_end=None, indices_type=torch.int32,
                      return_value=True, G=None):
    """by_value=True against the oracle's value order, position by position."""
    say(f"[topk by value] {name} shape={tuple(x.shape)} k={k} G={G} idx={indices_type} "
        f"val={return_value}")
    xd = to_device(x)
    re = row_end.cuda() if row_end is not None else None
    with blocks_per_row(G):
        v, i, f = dsel.topk(xd, k, end=re, indices_type=indices_type, return_value=return_value,
                            by_value=True)
    torch.cuda.synchronize()
    got = (gpu_bits(v) if v is not None else None, i.cpu().numpy(), f.cpu().numpy())
    want = oracle_topk(orc, x, k, row_end, 2, indices_type, return_value)
    n = valid_lengths(x.shape[0], x.shape[1], row_end)
    compare_topk(got, want, n, k, True, name)  # positional


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_value_order_small(dsel, orc, case):
    """Value order (sorted_index 2) over every small distribution: ties,
    all-equal rows, +-0, +-inf, denormals and NaN payloads, k >= cols."""
    name, rows, cols, dt, dist, k = case
    x = W.random_rows(zlib.crc32(name.encode()) & 0xFFFF, rows, cols, dt, dist)
    for ret, itype in ((True, torch.int32), (False, torch.int64)):
        check_value_order(dsel, orc, f"{name}/val{int(ret)}", x, k, None, itype, ret)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_value_order_paths(dsel, orc, dt):
    """Value order after every select path: one wave per row, one workgroup
    per row, split rows (one exchange and multi-pass), with ragged row
    ends, NaN rows and k up to 4096."""
    x = W.random_rows(151, 6, 50000, dt, "normal")
    W.plant_nans(x, 152, 2)
    re = torch.tensor([50000, 49999, 30000, 4097, 1500, 0], dtype=torch.int32)
    for k in (1, 100, 1024, 4096):
        check_value_order(dsel, orc, f"split/{dt}/k{k}", x, k, re)
    xw = W.random_rows(153, 9, 16000, dt, "special")
    rw = torch.tensor([16000, 9000, 2048, 2000, 700, 300, 1, 0, 12345], dtype=torch.int32)
    for k in (5, 512, 2000):
        check_value_order(dsel, orc, f"whole/{dt}/k{k}", xw, k, rw, torch.int64)
    xs = W.random_rows(154, 13, 1900, dt, "ties")
    check_value_order(dsel, orc, f"wave/{dt}", xs, 333, None, torch.int32, False)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_value_order_key_spans(dsel, orc, dt):
    """Value order where the selected keys span nothing (all equal), one
    8-bit digit, just over one, several digits, the whole finite range and,
    with a NaN among them, the whole key range: the sort runs as many digit
    passes as the span needs, and equal keys stay in column order."""
    rng = np.random.default_rng(0x5A17)
    cols, k = 3072, 1000
    if dt == W.BF16:
        base, low, nan = 0x3F80, 0xBF80, 0x7FC0
        spans = [0, 1, 255, 256, 257, 511, 512, 0x3FFF]
    else:
        base, low, nan = 0x3F800000, 0xBF800000, 0x7FC00000
        spans = [0, 1, 255, 256, 65535, 65536, (1 << 24) - 1, 1 << 24, 0x3FFFFFFF]
    rows = []
    for span in spans:
        r = np.full(cols, low, dtype=np.int64)
        top = base + rng.integers(0, span + 1, size=k)
        top[0], top[-1] = base, base + span
        r[rng.permutation(cols)[:k]] = top
        rows.append(r)
    r = rows[-1].copy()
    r[int(np.flatnonzero(r != low)[7])] = nan
    rows.append(r)
    arr = np.stack(rows)
    if dt == W.BF16:
        x = torch.from_numpy(arr.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(arr.astype(np.uint32).view(np.int32)).view(torch.float32)
    for ret, itype in ((True, torch.int32), (False, torch.int64)):
        check_value_order(dsel, orc, f"spans/{dt}/val{int(ret)}", x, k, None, itype, ret)
        check_value_order(dsel, orc, f"spans/{dt}/val{int(ret)}/short", x, k,
                          torch.tensor([3072, 999, 1000, 2, 1, 0, 1500, 3000, 2048, 17][:len(rows)],
                                       dtype=torch.int32), itype, ret)


@pytest.mark.parametrize("cfg", [2, 4])
def test_value_order_workloads(dsel, orc, cfg):
    """The 4 x 204800 bf16 and 128 x 129280 fp32 (sampling) workloads ordered by value."""
    case = W.make_config(cfg)
    check_value_order(dsel, orc, f"{case.name}/by_value", case.x, case.k, case.row_end,
                      case.indices_type, case.return_value)


@pytest.mark.parametrize("cols", [2048, 1536])
def test_wave_rows_with_values_staged(dsel, orc, cols):
    """One-wave bf16 rows with values, every way the output is staged in
    LDS: k int32 indices (up to k = 1024) or int64 indices (up to 512) fit
    the wave's histogram space, then the k values take their place there
    (k = 300, 512, 726, 1001, 1024); larger k take an LDS region of their own
    (1500, 2000; int64 at 1001).  k not a multiple of 4 or 8, rows longer
    and shorter than k, NaN rows, +-0 and infinities; ascending and value
    order."""
    x = W.random_rows(0x57A6 + cols, 24, cols, W.BF16, "special")
    W.plant_nans(x, 0x57A7 + cols, 3)
    ends = [cols, cols - 1, cols - 7, 2000, 1800, 1500, 1200, 1100, 1025, 1024, 1023, 1001,
            1000, 900, 727, 726, 725, 600, 100, 3, 1, 0, cols, cols - 33]
    re = torch.tensor([min(e, cols) for e in ends], dtype=torch.int32)
    for k in (300, 512, 726, 1001, 1024, 1500, 2000):
        if k >= cols:
            continue
        check_case(dsel, orc, f"staged/{cols}/k{k}", x, k, re, False, torch.int32, True)
        check_case(dsel, orc, f"staged/{cols}/k{k}/sorted", x, k, re, True, torch.int32, True)
        check_value_order(dsel, orc, f"staged/{cols}/k{k}/by_value", x, k, re, torch.int32, True)
    for k in (300, 512, 1001):
        check_case(dsel, orc, f"staged/{cols}/k{k}/i64", x, k, re, False, torch.int64, True)


@pytest.mark.parametrize("order", ["natural", "dual_chunk", None])
@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_row_orders(dsel, orc, dt, order):
    """Every row order gives the oracle's output: one-wave rows (2048 and
    700 columns) and whole rows (9000 columns) under causal row ends, odd
    and even row counts, a single row, and rows without row ends."""
    shapes = ((257, 2048, 700), (256, 2048, 1024), (64, 700, 100), (33, 9000, 512), (1, 1000, 10))
    for i, (rows, cols, k) in enumerate(shapes):
        x = W.random_rows(0x0D0 + i, rows, cols, dt, "normal")
        re = ((torch.arange(rows, dtype=torch.int64) + 1) * cols // rows).to(torch.int32)
        check_case(dsel, orc, f"order/{order}/{rows}x{cols}", x, k, re, False, torch.int32, True,
                   row_order=order)
        check_case(dsel, orc, f"order/{order}/{rows}x{cols}/full", x, k, None, False, torch.int64,
                   False, row_order=order)


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_custom_fills(dsel, orc, dt):
    """idx_oob_fill_value / value_oob_fill_value on short rows of every select
    path (one wave, one workgroup, split rows), both index types, values on
    and off, in ascending and value order."""
    fill_val = 2.5
    bits = 0x4020 if dt == W.BF16 else 0x40200000
    for cols, G in ((1500, None), (9000, None), (40000, 5)):
        x = W.random_rows(161 + cols, 5, cols, dt, "normal")
        re = torch.tensor([cols, 0, 3, 700, cols - 1], dtype=torch.int32)
        for k, itype, fill, ret, order in ((1000, torch.int32, -5, True, 1),
                                           (2048, torch.int64, 2 ** 40, False, 0),
                                           (777, torch.int32, 123456, True, 2)):
            xd = to_device(x)
            with blocks_per_row(G):
                v, i, f = dsel.topk(xd, k, end=re.cuda(), sorted_index=order == 1,
                                    by_value=order == 2, indices_type=itype, return_value=ret,
                                    idx_oob_fill_value=fill, value_oob_fill_value=fill_val)
            torch.cuda.synchronize()
            got = (gpu_bits(v) if v is not None else None, i.cpu().numpy(), f.cpu().numpy())
            xh = x.view(torch.int16).numpy().view(np.uint16) if dt == W.BF16 else x.numpy()
            want = orc.topk(xh, k, row_end=re.numpy(), sorted_index=order, indices_type=np.dtype(
                np.int32 if itype == torch.int32 else np.int64), return_value=ret,
                idx_fill=fill, val_fill_bits=bits)
            n = valid_lengths(5, cols, re)
            compare_topk(got, want, n, k, order != 0, f"fills/{dt}/{cols}/k{k}")
            assert (got[1][1] == fill).all(), "an empty row is all fill"


def test_abort_when_nan_found(dsel):
    """abort_when_nan_found=True raises for a NaN in a row longer than k, and
    not for a NaN in a row of length <= k (which is never checked)."""
    x = torch.randn(3, 5000).to(torch.bfloat16)
    x[2, 10] = float("nan")
    re = torch.tensor([5000, 5000, 100], dtype=torch.int32)
    dsel.topk(x.cuda(), 200, end=re.cuda(), abort_when_nan_found=True)  # row 2: n <= k
    x[1, 4000] = float("nan")
    with pytest.raises(FloatingPointError):
        dsel.topk(x.cuda(), 200, end=re.cuda(), abort_when_nan_found=True)
    _, _, f = dsel.topk(x.cuda(), 200, end=re.cuda())
    assert f.cpu().tolist() == [0, 1, 0]


@pytest.mark.parametrize("seed", range(6))
def test_random_sweep(dsel, orc, seed):
    """Seeded random configurations against the oracle: rows 1..9, columns
    1..70000, k 1..4096, both dtypes, every distribution, forced workgroups
    per row (split paths), the one exchange on or off, all three orders,
    both index types, values on or off, ragged and empty row ends, fills."""
    rng = np.random.default_rng(1000 + seed)
    dists = ["normal", "ties", "equal", "ascending", "descending", "narrow", "special"]
    for case in range(10):
        rows = int(rng.integers(1, 10))
        cols = int(rng.choice([int(rng.integers(1, 2100)), int(rng.integers(2100, 16400)),
                               int(rng.integers(16400, 70000))]))
        k = int(min(4096, max(1, rng.integers(1, 2 * cols + 2))))
        dt = W.BF16 if rng.random() < 0.6 else W.F32
        dist = dists[int(rng.integers(0, len(dists)))]
        x = W.random_rows(int(rng.integers(0, 1 << 16)), rows, cols, dt, dist)
        if rng.random() < 0.3:
            W.plant_nans(x, int(rng.integers(0, 1 << 16)), 1)
        re = None
        if rng.random() < 0.6:
            re = torch.from_numpy(rng.integers(-3, cols + 4, size=rows).astype(np.int32))
        G = None
        if cols > 2048 and rng.random() < 0.6:
            G = int(rng.integers(2, 65))
        one = [None, False][int(rng.integers(0, 2))]
        order = int(rng.integers(0, 3))
        itype = torch.int32 if rng.random() < 0.6 else torch.int64
        ret = bool(rng.random() < 0.7)
        fill = int(rng.integers(-9, 9))
        name = (f"sweep{seed}.{case}: {rows}x{cols} {dt} {dist} k={k} G={G} one={one} "
                f"order={order} {itype} val={ret} re={re is not None} fill={fill}")
        say("[topk] " + name)
        xd = to_device(x)
        with blocks_per_row(G), one_exchange(one):
            v, i, f = dsel.topk(xd, k, end=re.cuda() if re is not None else None,
                                sorted_index=order == 1, by_value=order == 2,
                                indices_type=itype, return_value=ret, idx_oob_fill_value=fill)
        torch.cuda.synchronize()
        got = (gpu_bits(v) if v is not None else None, i.cpu().numpy(), f.cpu().numpy())
        xh = x.view(torch.int16).numpy().view(np.uint16) if dt == W.BF16 else x.numpy()
        want = orc.topk(xh, k, row_end=re.numpy() if re is not None else None,
                        sorted_index=order,
                        indices_type=np.int32 if itype == torch.int32 else np.int64,
                        return_value=ret, idx_fill=fill)
        n = valid_lengths(rows, cols, re)
        compare_topk(got, want, n, k, order != 0, name)
    assert_workspaces_clean(dsel)


def test_exchange_region_garbage(dsel, orc):
    """The exchange region may hold anything between calls: with random bits
    written over it (headers and counts included), the one-exchange select
    of the 4 x 204800 workload and of ragged split rows still matches the
    oracle, and the row slots come back zero."""
    case = W.make_config(2)
    x2 = W.random_rows(141, 5, 70000, W.BF16, "normal")
    re2 = torch.tensor([70000, 65000, 30001, 9000, 0], dtype=torch.int32)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    region = (64 + 8 * cus * 544) * 4
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        check_case(dsel, orc, f"garbage{rep}/cfg2", case.x, case.k, case.row_end,
                   case.sorted_index, case.indices_type, case.return_value)
        check_case(dsel, orc, f"garbage{rep}/ragged", x2, 700, re2, True, torch.int32, True, 9)
        torch.cuda.synchronize()
        for ws in dsel._WORKSPACES.values():
            if ws.numel() > region:
                ws[256:region] = torch.randint(0, 256, (region - 256,), generator=gen,
                                               dtype=torch.uint8, device=ws.device)
    assert_workspaces_clean(dsel)


def test_workload_cfg2_multipass(dsel, orc):
    """The 4 x 204800 workload through the multi-pass split select too."""
    case = W.make_config(2)
    check_case(dsel, orc, "cfg2/multipass", case.x, case.k, case.row_end, case.sorted_index,
               case.indices_type, case.return_value, None, False)
