"""dsel_topk_noalloc (split-row scratch taken from the library, nothing
allocated) against dsel_topk_ex with a caller's workspace, through the C ABI.

Both entry points run on the same inputs into separate outputs; indices,
values and NaN flags must be equal byte for byte.  Each shape family is
called twice in a row, the second call with a smaller input, so the second
call runs on the scratch the first one left behind.  Split rows cover the
one-exchange select (bf16), the multi-pass select (bf16 with it turned off,
and fp32); a one-wave shape uses no scratch at all.
"""
import ctypes
import os

import pytest
import torch

import workloads as W
from parity import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsel():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsel_amd as d
    f = d._lib.dsel_topk_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int]
    return d


def _outputs(rows, k, itype, vdtype):
    isz = 4 if itype == torch.int32 else 8
    vsz = 2 if vdtype == torch.bfloat16 else 4
    istride = -(-k * isz // 16) * 16 // isz
    vstride = -(-k * vsz // 16) * 16 // vsz
    idx = torch.full((rows, istride), -77, dtype=itype, device="cuda")
    val = torch.full((rows, vstride), 7.0, dtype=vdtype, device="cuda")
    flag = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    return idx, val, flag, istride, vstride


def _run_both(dsel, x, k, row_end, order, itype, ret, fill=-1):
    rows, cols = x.shape
    dt = 0 if x.dtype == torch.bfloat16 else 1
    it = 0 if itype == torch.int32 else 1
    fill_bits = 0xFF80 if dt == 0 else 0xFF800000
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    re = row_end.data_ptr() if row_end is not None else None
    a = _outputs(rows, k, itype, x.dtype)
    b = _outputs(rows, k, itype, x.dtype)
    # dsel_topk_ex with a zeroed workspace of the queried size
    nb = ctypes.c_size_t(0)
    args = (x.data_ptr(), dt, rows, cols, x.stride(0), k, re, order, it, int(ret),
            a[0].data_ptr(), a[3], a[1].data_ptr(), a[4], a[2].data_ptr())
    assert dsel._lib.dsel_topk_ex(*args, None, ctypes.byref(nb), sp, fill, fill_bits, 0) == 0
    ws = torch.zeros(max(nb.value, 256), dtype=torch.uint8, device="cuda")
    nb = ctypes.c_size_t(ws.numel())
    assert dsel._lib.dsel_topk_ex(*args, ws.data_ptr(), ctypes.byref(nb), sp, fill, fill_bits, 0) == 0
    # the entry point that allocates nothing
    st = dsel._lib.dsel_topk_noalloc(x.data_ptr(), dt, rows, cols, x.stride(0), k, re, order, it,
                                     int(ret), b[0].data_ptr(), b[3], b[1].data_ptr(), b[4],
                                     b[2].data_ptr(), sp, fill, fill_bits, 0)
    assert st == 0, st
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]), "indices differ"
    va, vb = (a[1], b[1]) if x.dtype == torch.float32 else (a[1].view(torch.int16), b[1].view(torch.int16))
    if x.dtype == torch.float32:
        va, vb = va.view(torch.int32), vb.view(torch.int32)
    if ret:
        assert torch.equal(va, vb), "values differ"
    assert torch.equal(a[2], b[2]), "NaN flags differ"
    bits = ctypes.c_uint32(0)
    assert dsel._lib.dsel_topk_check(None, 0, ctypes.c_void_p(sp), ctypes.byref(bits)) == 0
    assert bits.value == 0


FAMILIES = [
    # name, (rows, cols, dtype, dist, k, order, itype, values, ends?), second smaller call
    ("bf16 one exchange", (6, 204800, W.BF16, "normal", 1024, 1, torch.int32, True, True),
     (3, 70000, W.BF16, "normal", 300, 0, torch.int32, True, False)),
    ("fp32 multi-pass", (9, 129280, W.F32, "normal", 4096, 0, torch.int64, True, False),
     (2, 40000, W.F32, "ties", 100, 2, torch.int32, False, True)),
    ("one wave, no scratch", (50, 1500, W.BF16, "special", 300, 0, torch.int32, True, True),
     (7, 900, W.BF16, "normal", 100, 1, torch.int64, True, False)),
]


@pytest.mark.parametrize("fam", FAMILIES, ids=lambda f: f[0])
def test_noalloc_matches_workspace_entry(dsel, fam):
    name, first, second = fam
    for i, (rows, cols, dt, dist, k, order, itype, ret, ends) in enumerate((first, second)):
        say(f"[noalloc] {name} call {i}: {rows}x{cols} {dt} {dist} k={k} order={order}")
        x = W.random_rows(0xA110C + 17 * i + cols, rows, cols, dt, dist)
        if i == 0:
            W.plant_nans(x, 0xA110D + cols, 1)
        re = None
        if ends:
            re = W.random_row_end(0xA110E + cols, rows, -2, cols + 2).cuda()
        _run_both(dsel, to_device(x), k, re, order, itype, ret)


def test_noalloc_multipass_bf16(dsel):
    """bf16 split rows with the one exchange turned off, two calls in a row."""
    old = os.environ.get("DSEL_SPLIT_ONE_EXCHANGE")
    os.environ["DSEL_SPLIT_ONE_EXCHANGE"] = "0"
    try:
        for i, (rows, cols, k) in enumerate(((5, 150000, 2048), (2, 60000, 64))):
            say(f"[noalloc] bf16 multi-pass call {i}: {rows}x{cols} k={k}")
            x = W.random_rows(0xB0B + i, rows, cols, W.BF16, "ties")
            _run_both(dsel, to_device(x), k, None, 1, torch.int32, True)
    finally:
        if old is None:
            os.environ.pop("DSEL_SPLIT_ONE_EXCHANGE", None)
        else:
            os.environ["DSEL_SPLIT_ONE_EXCHANGE"] = old
