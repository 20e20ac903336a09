"""Helpers shared by the GPU parity tests: run both sides, compare exactly.

Comparison rules: indices, values (bytewise) and NaN flags must be equal.
With ``sorted_index`` the comparison is positional; without it each row's
first c = min(k, n) (index, value) pairs are put in index order on both sides
first.  Slots c..k-1 must be padding on both sides.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle_pins as P


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: torch.Tensor) -> torch.Tensor:
    """Device copy of a host tensor that keeps its strides (row padding included)."""
    d = torch.empty_strided(tuple(x.shape), tuple(x.stride()), dtype=x.dtype, device="cuda")
    d.copy_(x)
    return d


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a GPU tensor as raw bits (uint16 for bf16, uint32 for fp32)."""
    h = t.detach().cpu()
    if h.dtype == torch.bfloat16:
        return h.view(torch.int16).numpy().view(np.uint16)
    if h.dtype == torch.float32:
        return h.numpy().view(np.uint32)
    return h.numpy()


def oracle_topk(orc, x: torch.Tensor, k, row_end, sorted_index, indices_type, return_value):
    xh = P.to_host(x)
    it = np.int32 if indices_type == torch.int32 else np.int64
    re = row_end.numpy() if row_end is not None else None
    return orc.topk(xh, k, row_end=re, sorted_index=sorted_index, indices_type=it,
                    return_value=return_value)


def canonical(idx: np.ndarray, vals, n_valid: np.ndarray, k: int):
    """Per row, put the first c pairs in index order (c = min(k, n))."""
    idx = idx.astype(np.int64).copy()
    vals = None if vals is None else vals.copy()
    for i in range(idx.shape[0]):
        c = int(min(k, n_valid[i]))
        order = np.argsort(idx[i, :c], kind="stable")
        idx[i, :c] = idx[i, :c][order]
        if vals is not None:
            vals[i, :c] = vals[i, :c][order]
    return idx, vals


def valid_lengths(rows: int, cols: int, row_end) -> np.ndarray:
    if row_end is None:
        return np.full(rows, cols, dtype=np.int64)
    return np.clip(row_end.numpy().astype(np.int64), 0, cols)


def compare_topk(got, want, n_valid, k, sorted_index, what=""):
    gv, gi, gf = got
    wv, wi, wf = want
    gi = gi.astype(np.int64)
    wi = wi.astype(np.int64)
    if not sorted_index:
        gi, gv = canonical(gi, gv, n_valid, k)
        wi, wv = canonical(wi, wv, n_valid, k)
    bad = np.nonzero((gi != wi).any(axis=1))[0]
    assert bad.size == 0, f"{what}: indices differ in {bad.size} rows, first row {bad[0]}: " \
                          f"got {gi[bad[0]][:16]} want {wi[bad[0]][:16]}"
    if wv is not None:
        wvb = P.raw_bits(wv)
        bad = np.nonzero((gv != wvb).any(axis=1))[0]
        assert bad.size == 0, f"{what}: values differ in {bad.size} rows, first {bad[0]}"
    assert np.array_equal(gf, wf), f"{what}: NaN flags differ in rows {np.nonzero(gf != wf)[0][:10]}"
