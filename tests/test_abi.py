"""The C ABI library loads and exports every entry point include/dsel.h declares.

Only calls that fail host-side argument checks are made here (they return
before touching a device), so this runs without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsel.h")
LIB = os.path.join(ROOT, "sparse_attention_indexer_dsel_amd", "libdsel.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # by path: the package's __init__ needs the library this builds
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_dsel_build_lib", os.path.join(ROOT, "sparse_attention_indexer_dsel_amd", "build_lib.py"))
        build_lib = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build_lib)
        build_lib.build()
    return ctypes.CDLL(LIB)


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\bint\s+(dsel_\w+)\s*\(", text)))


def test_header_declares_the_calls():
    assert declared() == ["dsel_gather_rows", "dsel_read_floor", "dsel_stride_requirement",
                          "dsel_topk", "dsel_topk_check", "dsel_topk_ex", "dsel_topk_gather",
                          "dsel_topk_noalloc"]


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for name in declared():
        assert name in exported, name
        assert getattr(lib, name)


def test_stride_requirement_host_only(lib):
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    assert lib.dsel_stride_requirement(ctypes.byref(a), ctypes.byref(b)) == 0
    assert (a.value, b.value) == (16, 16)
    assert lib.dsel_stride_requirement(None, ctypes.byref(b)) == -1


def _topk(lib, **kw):
    args = dict(x=16, dtype=0, rows=4, cols=64, stride=64, k=8, row_end=None, sorted_index=0,
                itype=0, ret=0, oi=16, ois=16, ov=None, ovs=0, flag=None, ws=None)
    args.update(kw)
    nb = ctypes.c_size_t(0)
    f = lib.dsel_topk
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return f(args["x"], args["dtype"], args["rows"], args["cols"], args["stride"], args["k"],
             args["row_end"], args["sorted_index"], args["itype"], args["ret"], args["oi"],
             args["ois"], args["ov"], args["ovs"], args["flag"], args["ws"], ctypes.byref(nb), None)


def test_topk_host_checks(lib):
    assert _topk(lib, k=0) == -2
    assert _topk(lib, k=4097) == -2
    assert _topk(lib, dtype=7) == -1
    assert _topk(lib, itype=3) == -1
    assert _topk(lib, sorted_index=3) == -1   # 0/1: ascending columns, 2: by value
    assert _topk(lib, sorted_index=-1) == -1
    assert _topk(lib, cols=0) == -1
    assert _topk(lib, rows=-1) == -1
    assert _topk(lib, x=None) == -1
    assert _topk(lib, ret=1, ov=None) == -1
    assert _topk(lib, stride=63) == -1                     # stride < cols
    assert _topk(lib, ois=7) == -1                         # idx stride < k
    assert _topk(lib, stride=68) == -3                     # 136 B row stride
    assert _topk(lib, x=18) == -3                          # misaligned base
    assert _topk(lib, rows=0) == 0                         # empty: nothing launched


def test_gather_host_checks(lib):
    f = lib.dsel_gather_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    ok = dict(key=16, dt=0, B=2, L=10, D=128, kbs=1280, krs=128, pos=16, pt=0, R=3, P=5, prs=5,
              out=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["key"], a["dt"], a["B"], a["L"], a["D"], a["kbs"], a["krs"], a["pos"], a["pt"],
                 a["R"], a["P"], a["prs"], a["out"], None)
    assert call(dt=5) == -1
    assert call(pt=5) == -1
    assert call(L=0) == -1
    assert call(key=None) == -1
    assert call(prs=4) == -1
    assert call(D=100) == -3          # 200 B rows are not 16 B multiples
    assert call(krs=129) == -3
    assert call(out=24) == -3
    assert call(R=0) == 0             # empty: nothing launched


def _topk_ex(lib, idx_fill, val_bits, dtype=0, itype=0, row_order=0):
    nb = ctypes.c_size_t(0)
    f = lib.dsel_topk_ex
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_uint32, ctypes.c_int]
    return f(16, dtype, 4, 64, 64, 8, None, 0, itype, 0, 16, 16, None, 0, None, None,
             ctypes.byref(nb), None, idx_fill, val_bits, row_order)


def test_topk_ex_fill_checks(lib):
    """Fills that do not fit the output types are refused before any launch."""
    assert _topk_ex(lib, 2 ** 31, 0xFF80) == -1               # int32 index fill out of range
    assert _topk_ex(lib, -(2 ** 31) - 1, 0xFF80) == -1
    assert _topk_ex(lib, -1, 0x1FF80) == -1                    # bf16 fill wider than 16 bits
    assert _topk_ex(lib, -1, 0xFF80, row_order=3) == -1        # no such row order
    assert _topk_ex(lib, -1, 0xFF80, row_order=-1) == -1


def test_topk_check_host_checks(lib):
    """dsel_topk_check: a NULL error-bits pointer is refused; a NULL or
    too-small workspace had no split rows run on it (nothing to report);
    a misaligned one is refused.  None of these touch a device."""
    f = lib.dsel_topk_check
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    bits = ctypes.c_uint32(7)
    assert f(16, 1024, None, None) == -1
    assert f(None, 1024, None, ctypes.byref(bits)) == 0 and bits.value == 0
    bits.value = 7
    assert f(16, 2, None, ctypes.byref(bits)) == 0 and bits.value == 0
    assert f(20, 1024, None, ctypes.byref(bits)) == -3


def test_read_floor_host_checks(lib):
    """dsel_read_floor refuses NULL pointers, sizes that are not a positive
    multiple of 16 and a misaligned buffer before it launches anything."""
    f = lib.dsel_read_floor
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 64, 16, None) == -1
    assert f(16, 64, None, None) == -1
    assert f(16, 0, 16, None) == -1
    assert f(16, -16, 16, None) == -1
    assert f(16, 40, 16, None) == -1
    assert f(24, 64, 16, None) == -3


class GatherKey(ctypes.Structure):
    _fields_ = [("key", ctypes.c_void_p), ("dtype", ctypes.c_int), ("len", ctypes.c_int64),
                ("dim", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("out", ctypes.c_void_p)]


def _topk_gather(lib, keys, n_keys=None, pad=0, rows=4, rpb=2):
    f = lib.dsel_topk_gather
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(GatherKey),
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                  ctypes.c_void_p]
    arr = (GatherKey * max(1, len(keys)))(*keys)
    nb = ctypes.c_size_t(0)
    return f(16, 0, rows, 64, 64, 8, None, 0, 0, 16, 16, None, rpb, arr,
             len(keys) if n_keys is None else n_keys, pad, None, ctypes.byref(nb), None)


def test_topk_gather_host_checks(lib):
    """dsel_topk_gather refuses bad key descriptors, key counts, pad modes
    and batch shapes before anything reaches a device."""
    good = GatherKey(16, 0, 32, 128, 32 * 128, 128, 16)
    assert _topk_gather(lib, [good], n_keys=0) == -1         # no key
    assert _topk_gather(lib, [good] * 5) == -1               # more than four keys
    assert _topk_gather(lib, [good], pad=2) == -1            # no such pad mode
    assert _topk_gather(lib, [good], rows=5, rpb=2) == -1    # rows not a multiple
    assert _topk_gather(lib, [good], rpb=0) == -1
    assert _topk_gather(lib, [GatherKey(16, 2, 32, 128, 4096, 128, 16)]) == -1   # key dtype
    assert _topk_gather(lib, [GatherKey(16, 0, 0, 128, 4096, 128, 16)]) == -1    # len 0
    assert _topk_gather(lib, [GatherKey(16, 0, 32, 100, 3200, 100, 16)]) == -3   # 200-byte rows
    assert _topk_gather(lib, [GatherKey(24, 0, 32, 128, 4096, 128, 16)]) == -3   # key pointer
    assert _topk_gather(lib, [GatherKey(16, 0, 32, 128, 4096, 129, 16)]) == -3   # row stride
    assert _topk_gather(lib, [good, GatherKey(16, 0, 32, 128, 4096, 128, 8)]) == -3  # out pointer
