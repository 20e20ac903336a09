"""CPU oracle for the selection step (row-wise top-k, then key gather).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The product path never imports it.

The arithmetic lives in ``dsel_oracle.c`` (plain C, one row at a time,
``qsort`` under a total order, ``memcpy`` for every copied value); this file
only marshals numpy arrays into it.  bf16 data is passed as its raw uint16
bit patterns.

Pins: every function here is checked against brute force, invariants,
closed forms and library special cases in ``tests/test_oracle_pins.py``;
``tests/test_oracle_mutants.py`` shows those pins fail on planted mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dsel_oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

OR_BF16, OR_F32 = 0, 1
OR_I32, OR_I64 = 0, 1


def compile_oracle(out_path: str = DEFAULT_LIB, mutant: int = 0) -> str:
    """Build the oracle shared library with gcc (``mutant`` > 0 plants a mistake)."""
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-shared", "-fPIC", "-pthread",
           f"-DORACLE_MUTANT={int(mutant)}", SOURCE, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


class Oracle:
    """ctypes front end to ``liboracle.so``."""

    def __init__(self, lib_path: str = DEFAULT_LIB):
        if not os.path.exists(lib_path):
            compile_oracle(lib_path)
        self.path = lib_path
        self.lib = ctypes.CDLL(lib_path)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        self.lib.oracle_topk.restype = i32
        self.lib.oracle_topk.argtypes = [vp, i32, i64, i64, i64, i64, vp, i32, i32, i32,
                                         vp, i64, vp, i64, vp, i32, i64, ctypes.c_uint32]
        self.lib.oracle_gather.restype = i32
        self.lib.oracle_gather.argtypes = [vp, i32, i64, i64, i64, i64, i64, vp, i32, i64,
                                           i64, i64, vp, i32]

    # -- top-k -------------------------------------------------------------
    def topk(self, x: np.ndarray, k: int, row_end: Optional[np.ndarray] = None,
             sorted_index: bool = False, indices_type=np.int32, return_value: bool = True,
             threads: Optional[int] = None, idx_fill: int = -1,
             val_fill_bits: Optional[int] = None
             ) -> Tuple[Optional[np.ndarray], np.ndarray, np.ndarray]:
        """x: 2-D uint16 (bf16 bits) or float32, last dim contiguous.

        sorted_index: False/0 (any order; here the value order), True/1
        (ascending index) or 2 (by value: largest first, equal values by
        ascending index).
        idx_fill / val_fill_bits: index and raw value bits of the slots past
        a short row's length (default -1 and -inf).
        Returns (values or None, indices [rows, k], nan_flag uint8 [rows]).
        Values come back in the input's storage type (uint16 bits for bf16).
        """
        if x.ndim != 2 or (x.size and x.shape[1] > 1 and x.strides[1] != x.itemsize):
            raise ValueError("x must be 2-D with a contiguous last dim")
        if x.dtype == np.uint16:
            dt = OR_BF16
        elif x.dtype == np.float32:
            dt = OR_F32
        else:
            raise TypeError(x.dtype)
        rows, cols = x.shape
        stride = x.strides[0] // x.itemsize if rows > 0 else cols
        itype = np.dtype(indices_type)
        it = OR_I32 if itype == np.int32 else OR_I64
        idx = np.empty((rows, k), dtype=itype)
        vals = np.empty((rows, k), dtype=x.dtype) if return_value else None
        flag = np.zeros(rows, dtype=np.uint8)
        re = None
        if row_end is not None:
            re = np.ascontiguousarray(row_end, dtype=np.int32)
            if re.shape != (rows,):
                raise ValueError("row_end must be [rows]")
        nt = host_threads() if threads is None else int(threads)
        st = self.lib.oracle_topk(
            x.ctypes.data if rows else None, dt, rows, cols, max(stride, cols), k,
            re.ctypes.data if re is not None else None,
            int(sorted_index), it, int(bool(return_value)),
            idx.ctypes.data, k, vals.ctypes.data if vals is not None else None, k,
            flag.ctypes.data, nt, int(idx_fill),
            (0xFF80 if dt == OR_BF16 else 0xFF800000) if val_fill_bits is None else int(val_fill_bits))
        if st != 0:
            raise RuntimeError(f"oracle_topk failed: {st}")
        return vals, idx, flag

    # -- gather --------------------------------------------------------------
    def gather(self, key: np.ndarray, pos: np.ndarray, pad: str = "clamp") -> np.ndarray:
        """key: [B, L, D] (any strides, last dim contiguous); pos: [B, R, P] int32/int64.

        pad "clamp": positions clamped into [0, L-1] (the "safe" positions);
        "zero": a position outside [0, L) gives a row of zeros (the masked fill).
        """
        if pad not in ("clamp", "zero"):
            raise ValueError(pad)
        if key.ndim != 3 or key.strides[2] != key.itemsize:
            raise ValueError("key must be [B, L, D] with a contiguous last dim")
        if key.itemsize not in (2, 4):
            raise TypeError(key.dtype)
        B, L, D = key.shape
        pos = np.ascontiguousarray(pos)
        if pos.ndim != 3 or pos.shape[0] != B:
            raise ValueError("pos must be [B, R, P]")
        pt = OR_I32 if pos.dtype == np.int32 else OR_I64
        if pos.dtype not in (np.int32, np.int64):
            raise TypeError(pos.dtype)
        _, R, P = pos.shape
        out = np.empty((B, R, P, D), dtype=key.dtype)
        st = self.lib.oracle_gather(
            key.ctypes.data, key.itemsize, B, L, D, key.strides[0] // key.itemsize,
            key.strides[1] // key.itemsize, pos.ctypes.data, pt, R, P, P, out.ctypes.data,
            1 if pad == "zero" else 0)
        if st != 0:
            raise RuntimeError(f"oracle_gather failed: {st}")
        return out


_DEFAULT: Optional[Oracle] = None


def get_oracle() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
