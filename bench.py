"""Benchmark of the selection step (row-wise top-k, then key gather) on one GPU.

Byte accounting (algorithmic bytes: what the method must move):
  top-k  = sum over rows of the valid-prefix read (a row of valid length
           n <= k read only when values are returned), + 4*rows for row_end,
           + rows*k*index bytes, + rows*k*value bytes when values are
           returned, + rows bytes of NaN flag.
  gather = written bytes + position bytes read + one compulsory read of each
           distinct key row touched.
The gather is also reported in the pages' convention (gathered output bytes
over time; MindSpore hyper-parallel PR #1094, mechanism check).
"""
from __future__ import annotations

import numpy as np

HBM_PEAK_GBPS = 8000.0


def output_convention_gbps(out_bytes: float, seconds: float) -> float:
    """Gathered (output) bytes per second, in GB/s."""
    return out_bytes / seconds / 1e9


def topk_algorithmic_bytes(n_valid: np.ndarray, k: int, elt: int, idx_elt: int,
                           return_value: bool, has_row_end: bool) -> int:
    n = np.asarray(n_valid, dtype=np.int64)
    read = n if return_value else np.where(n > k, n, 0)
    rows = int(n.shape[0])
    total = int(read.sum()) * elt
    total += 4 * rows if has_row_end else 0
    total += rows * k * idx_elt
    total += rows * k * elt if return_value else 0
    total += rows
    return total


def gather_algorithmic_bytes(n_positions: int, dim: int, elt: int, pos_elt: int,
                             distinct_rows: int) -> int:
    return n_positions * dim * elt + n_positions * pos_elt + distinct_rows * dim * elt


if __name__ == "__main__":
    raise SystemExit("GPU benchmark not built yet")
