"""Seeded synthetic inputs for the selection step (top-k then key gather).

This module only draws random numbers and lays them out.  It holds none of
the selection or gather arithmetic, so both the CPU oracle and the GPU path
can be fed from it without sharing any of the method.

Every tensor is produced on the host from ``torch.Generator().manual_seed``
and returned as CPU tensors; callers copy them to the device.  bf16 data is
drawn in fp32 and rounded with ``.to(torch.bfloat16)`` (round to nearest
even).

Workload shapes follow the pages:

* DeepSelect tutorial ("Sheshisa Imisebenzi ye-PyTorch TopK nge-DeepSelect"),
  section "Ukusebenzisa i-TopK Okuyisisekelo": a 4 x 204800 bf16 input with
  k = 1024; section "Ukusebenza Ngemigqa Enobude Obuhlukahlukene": fp32 rows
  of 129280 columns with a per-row exclusive end; section "Imithwalo Yomsebenzi
  Esekelwayo": bf16 for the lightning indexer, fp32 with a vocabulary near
  128K for sampling, k <= 4096.
* MindSpore hyper-parallel PR #1094 (gather compressed keys through one
  index_select), English description: sequence 4096 over compressed length
  2048, head_dim 128, gathers of 1024 x 1024 and 1024 x 512 positions, and a
  compressed length of 16384; Chinese body, release geometry: index_topk 512.

The five named workloads are ``CONFIGS``; ``make_config(i)`` builds one.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

BF16 = "bf16"
F32 = "f32"


@dataclass
class TopkCase:
    """One top-k call's inputs and flags (all CPU tensors)."""

    name: str
    x: torch.Tensor                      # [rows, cols] (possibly a strided view)
    k: int
    row_end: Optional[torch.Tensor]      # int32 [rows] or None
    sorted_index: bool
    indices_type: torch.dtype            # torch.int32 / torch.int64
    return_value: bool
    # gather stage (optional): keys [B, L, D] and how the [rows, k] indices
    # are viewed as positions [B, R, k]
    keys: list = field(default_factory=list)
    gather_batch: int = 0
    repeat_every: int = 0                # overwrite every n-th slot with slot 0 (parity only)

    @property
    def dtype(self) -> str:
        return BF16 if self.x.dtype == torch.bfloat16 else F32


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def config1() -> TopkCase:
    """4 rows x 8192 bf16 ~N(0,1), k=256, full rows, unsorted i32 + values."""
    g = _gen(1)
    x = torch.randn(4, 8192, generator=g).to(torch.bfloat16)
    return TopkCase("cfg1", x, 256, None, False, torch.int32, True)


def config2() -> TopkCase:
    """4 x 204800 bf16 ~N(0,1), k=1024, ascending indices, i32 + values."""
    g = _gen(2)
    x = torch.randn(4, 204800, generator=g).to(torch.bfloat16)
    return TopkCase("cfg2", x, 1024, None, True, torch.int32, True)


def config3() -> TopkCase:
    """Prefill selection: 4096 query rows over 2048 compressed positions.

    Causal end row_end[i] = (i+1)//2, k=1024, index-only i32, 41 rows (1%)
    carry one NaN at a uniform column; then a gather from a [1, 2048, 128]
    bf16 key with the indices viewed as [1, 4096, 1024].
    """
    g = _gen(3)
    rows, cols = 4096, 2048
    x = torch.randn(rows, cols, generator=g).to(torch.bfloat16)
    row_end = ((torch.arange(rows, dtype=torch.int64) + 1) // 2).to(torch.int32)
    n_nan = round(0.01 * rows)
    nan_rows = torch.randperm(rows, generator=g)[:n_nan]
    nan_cols = torch.randint(0, cols, (n_nan,), generator=g)
    x[nan_rows, nan_cols] = float("nan")
    key = torch.randn(1, cols, 128, generator=g).to(torch.bfloat16)
    return TopkCase("cfg3", x, 1024, row_end, False, torch.int32, False,
                    keys=[key], gather_batch=1)


def config4() -> TopkCase:
    """Sampling: 128 x 129280 fp32 logits 2*N(0,1) with 32 spikes ~N(12,1).

    The spikes overwrite 32 distinct uniformly drawn columns per row.
    k=4096, unsorted i64 + values.
    """
    g = _gen(4)
    rows, cols = 128, 129280
    x = 2.0 * torch.randn(rows, cols, generator=g)
    for r in range(rows):
        c = torch.randperm(cols, generator=g)[:32]
        x[r, c] = 12.0 + torch.randn(32, generator=g)
    return TopkCase("cfg4", x, 4096, None, False, torch.int64, True)


def config5() -> TopkCase:
    """Long-context indexer: 2 x 1024 rows over 16384 compressed positions.

    row_end uniform in [512, 16384], k=512, index-only i32; two gathers, one
    from a contiguous [2, 16384, 128] key and one from a transposed view
    (batch stride 128, row stride 256 elements).  ``repeat_every`` = 64 makes
    the parity run overwrite every 64th selected slot with slot 0's position.
    """
    g = _gen(5)
    x = torch.randn(2, 1024, 16384, generator=g).to(torch.bfloat16).view(2048, 16384)
    row_end = torch.randint(512, 16385, (2048,), generator=g).to(torch.int32)
    key_a = torch.randn(2, 16384, 128, generator=g).to(torch.bfloat16)
    key_b = torch.randn(16384, 2, 128, generator=g).to(torch.bfloat16).transpose(0, 1)
    return TopkCase("cfg5", x, 512, row_end, False, torch.int32, False,
                    keys=[key_a, key_b], gather_batch=2, repeat_every=64)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make_config(i: int) -> TopkCase:
    return CONFIGS[int(i)]()


# ----------------------------------------------------------------------------
# Parametric small cases for parity and edge-case tests.
# ----------------------------------------------------------------------------

def random_rows(seed: int, rows: int, cols: int, dtype: str = BF16,
                dist: str = "normal", stride: Optional[int] = None,
                scale: float = 1.0) -> torch.Tensor:
    """A [rows, cols] input whose row stride is ``stride`` elements.

    By default the stride is cols rounded up to a 16-byte multiple (the
    alignment a row of the input must have); a larger ``stride`` gives a
    padded view.

    ``dist``: "normal" (N(0, scale^2)), "ties" (integers in [-8, 8): heavy
    ties), "equal" (all entries 1.5), "ascending", "descending",
    "special" (normal mixed with +-0, +-inf, denormals and NaN payloads),
    "narrow" (N(0,1) quantised to a few bf16 steps around one value).
    """
    g = _gen(seed)
    per = 8 if dtype == BF16 else 4  # elements per 16 bytes
    st = -(-max(cols, 1) // per) * per if stride is None else int(stride)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    base = torch.empty(rows, max(st, 1), dtype=torch.float32)
    if dist == "normal":
        base.copy_(scale * torch.randn(rows, max(st, 1), generator=g))
    elif dist == "ties":
        base.copy_(torch.randint(-8, 8, (rows, max(st, 1)), generator=g).float())
    elif dist == "equal":
        base.fill_(1.5)
    elif dist == "ascending":
        base.copy_(torch.arange(max(st, 1), dtype=torch.float32).expand(rows, -1) * 0.25)
    elif dist == "descending":
        base.copy_(-torch.arange(max(st, 1), dtype=torch.float32).expand(rows, -1) * 0.25)
    elif dist == "narrow":
        base.copy_(2.0 + 0.02 * torch.randn(rows, max(st, 1), generator=g))
    elif dist == "special":
        base.copy_(torch.randn(rows, max(st, 1), generator=g))
        pick = torch.randint(0, 10, (rows, max(st, 1)), generator=g)
        base[pick == 0] = 0.0
        base[pick == 1] = -0.0
        base[pick == 2] = float("inf")
        base[pick == 3] = float("-inf")
        base[pick == 4] = 1e-40 if dtype == BF16 else 1e-42
        base[pick == 5] = -1e-40 if dtype == BF16 else -1e-42
    else:
        raise ValueError(dist)
    out = base.to(tdt)
    if dist == "special":
        # NaNs with assorted payloads and signs, set through the bit pattern
        pick = torch.randint(0, 40, (rows, max(st, 1)), generator=g)
        if dtype == BF16:
            bits = out.view(torch.int16)
            bits[pick == 0] = 0x7FC1
            bits[pick == 1] = -0x0001  # 0xFFFF: negative NaN
            bits[pick == 2] = 0x7F81
        else:
            bits = out.view(torch.int32)
            bits[pick == 0] = 0x7FC00001
            bits[pick == 1] = -0x00000001
            bits[pick == 2] = 0x7F800001
    return out[:, :cols]


def random_row_end(seed: int, rows: int, lo: int, hi: int) -> torch.Tensor:
    """int32 [rows] uniform in [lo, hi] (inclusive); may exceed cols or be negative."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (rows,), generator=g).to(torch.int32)


def plant_nans(x: torch.Tensor, seed: int, count: int) -> torch.Tensor:
    """Set ``count`` random (row, col) entries of x to NaN, in place."""
    g = _gen(seed)
    rows, cols = x.shape
    r = torch.randint(0, rows, (count,), generator=g)
    c = torch.randint(0, cols, (count,), generator=g)
    x[r, c] = float("nan")
    return x


def random_keys(seed: int, batch: int, length: int, dim: int, dtype: str = BF16,
                layout: str = "contiguous") -> torch.Tensor:
    """A [batch, length, dim] key; ``layout`` "transposed" gives a strided view."""
    g = _gen(seed)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    if layout == "contiguous":
        return torch.randn(batch, length, dim, generator=g).to(tdt)
    if layout == "transposed":
        return torch.randn(length, batch, dim, generator=g).to(tdt).transpose(0, 1)
    if layout == "padded":
        return torch.randn(batch, length, dim + 8, generator=g).to(tdt)[:, :, :dim]
    raise ValueError(layout)


def random_positions(seed: int, batch: int, rows: int, per_row: int, length: int,
                     dtype: torch.dtype = torch.int32, oob: bool = False) -> torch.Tensor:
    """Positions [batch, rows, per_row]; ``oob`` mixes in -1 and >= length."""
    g = _gen(seed)
    lo, hi = (-3, length + 3) if oob else (0, length)
    return torch.randint(lo, hi, (batch, rows, per_row), generator=g).to(dtype)
