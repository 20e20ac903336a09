"""Pins for the CPU oracle: checks that owe nothing to the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the pages or plain mathematics fix:

* brute force over every c-subset of tiny rows (the selected set is the one
  whose values, sorted in decreasing order, are lexicographically largest,
  then whose indices are lexicographically smallest);
* an O(n^2) pairwise dominance check on larger rows;
* special cases that reduce to library routines (``numpy.argsort`` stable on
  rows without NaN; ``torch.topk`` on rows with distinct values; torch
  advanced indexing and ``index_select`` for the gather);
* closed forms (all-equal, ascending and descending rows, k >= n, empty rows,
  the prefill workload's selected and padding totals);
* the NaN-flag rule of the DeepSelect tutorial's NaN section (rows whose
  valid length is <= k are not checked) and the OOB fill rule of its
  variable-length section.

The same functions run against planted-mistake builds of the oracle to show
that each plausible mistake fails at least one of them.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

BF16_NEG_INF = np.uint16(0xFF80)
F32_NEG_INF_BITS = np.uint32(0xFF800000)


# ---------------------------------------------------------------------------
# independent helpers (value decoding and the ranking relation)
# ---------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (strides kept)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16).numpy().view(np.uint16)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Oracle input form: uint16 bits for bf16, float32 otherwise."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.numpy()


def decode(arr: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bits or float32."""
    with np.errstate(invalid="ignore"):
        if arr.dtype == np.uint16:
            w = (arr.astype(np.uint32) << np.uint32(16))
            return w.view(np.float32).astype(np.float64)
        return arr.astype(np.float64)


def beats(a: float, b: float) -> bool:
    """a ranks strictly above b: NaN above everything, NaNs equal, -0 == +0."""
    an, bn = math.isnan(a), math.isnan(b)
    if an or bn:
        return an and not bn
    return a > b


def same_rank(a: float, b: float) -> bool:
    an, bn = math.isnan(a), math.isnan(b)
    if an or bn:
        return an and bn
    return a == b


def valid_len(row_end, i: int, cols: int) -> int:
    n = cols if row_end is None else int(row_end[i])
    return max(0, min(n, cols))


def raw_bits(arr: np.ndarray) -> np.ndarray:
    return arr.view(np.uint16) if arr.dtype == np.uint16 else arr.view(np.uint32)


def check_row_contract(xrow_vals, xrow_bits, n, k, idx_row, val_row_bits, sorted_index,
                       is_bf16: bool):
    """Invariants every output row satisfies (the spec list)."""
    c = min(k, n)
    sel = [int(v) for v in idx_row[:c]]
    assert all(0 <= s < n for s in sel), "index outside [0, n)"
    assert len(set(sel)) == c, "indices not distinct"
    assert all(int(v) == -1 for v in idx_row[c:]), "padding must be -1"
    if sorted_index:
        assert all(sel[j] < sel[j + 1] for j in range(c - 1)), "not ascending"
    if val_row_bits is not None:
        for j, s in enumerate(sel):
            assert val_row_bits[j] == xrow_bits[s], "value is not a bit copy"
        pad = BF16_NEG_INF if is_bf16 else F32_NEG_INF_BITS
        assert all(v == pad for v in val_row_bits[c:]), "value padding must be -inf"
    return sel


def expected_flag(xrow_vals, n, k) -> int:
    return int(n > k and bool(np.isnan(xrow_vals[:n]).any()))


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def brute_force_select(vals, n, k):
    """The best c-subset by (values desc, lexicographic) then (indices asc)."""
    c = min(k, n)
    best = None
    best_key = None
    for sub in itertools.combinations(range(n), c):
        # values sorted in decreasing rank; NaN first
        vs = sorted((vals[j] for j in sub),
                    key=lambda v: (0 if math.isnan(v) else 1, -v if not math.isnan(v) else 0.0))
        vkey = tuple((1, 0.0) if math.isnan(v) else (0, v) for v in vs)
        # larger value vector wins; compare element-wise using beats/same_rank
        if best is None:
            best, best_key = sub, (vkey, sub)
            continue
        bv, bsub = best_key
        better = None
        for a, b in zip(vkey, bv):
            av = float("nan") if a[0] else a[1]
            bvv = float("nan") if b[0] else b[1]
            if beats(av, bvv):
                better = True
                break
            if beats(bvv, av):
                better = False
                break
        if better is None:
            better = sub < bsub   # itertools yields sorted tuples
        if better:
            best, best_key = sub, (vkey, sub)
    return sorted(best) if best is not None else []


TINY_POOL = [0.0, -0.0, 1.0, -1.0, 2.5, float("inf"), float("-inf"), float("nan"), 1e-40]


def _tiny_rows(rng, rows, cols, dtype):
    pool = np.array(TINY_POOL, dtype=np.float32)
    x = pool[rng.integers(0, len(pool), size=(rows, cols))]
    if dtype == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        bits = bf16_bits(t).copy()
        # give some NaNs other payloads and the sign bit
        nanpos = np.isnan(decode(bits))
        alt = rng.integers(0, 3, size=bits.shape)
        bits[nanpos & (alt == 1)] = 0xFFC1
        bits[nanpos & (alt == 2)] = 0x7F81
        return bits
    x = x.copy()
    bits = x.view(np.uint32)
    nanpos = np.isnan(x)
    alt = rng.integers(0, 3, size=x.shape)
    bits[nanpos & (alt == 1)] = 0xFFC00001
    bits[nanpos & (alt == 2)] = 0x7F800001
    return x


def pin_bruteforce_tiny(orc, seed=0):
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        for cols in (1, 2, 3, 5, 8, 10):
            x = _tiny_rows(rng, 12, cols, dtype)
            vals = decode(x)
            row_end = rng.integers(-2, cols + 3, size=12).astype(np.int32)
            for k in range(1, cols + 3):
                for sorted_index in (False, True):
                    v, idx, flag = orc.topk(x, k, row_end=row_end, sorted_index=sorted_index,
                                            return_value=True)
                    for i in range(x.shape[0]):
                        n = valid_len(row_end, i, cols)
                        sel = check_row_contract(vals[i], raw_bits(x[i]), n, k, idx[i],
                                                 raw_bits(v[i]), sorted_index, dtype == "bf16")
                        want = brute_force_select(list(vals[i]), n, k)
                        assert sorted(sel) == want, (dtype, cols, k, i, sel, want)
                        assert flag[i] == expected_flag(vals[i], n, k)


# ---------------------------------------------------------------------------
# pairwise dominance on larger rows
# ---------------------------------------------------------------------------

def _rank_arrays(vals):
    """(is_nan, value-with-nan-zeroed) for vectorised comparisons."""
    isn = np.isnan(vals)
    v = np.where(isn, 0.0, vals)
    return isn, v


def check_pairwise(vals, n, sel):
    """Every selected beats every unselected valid element, or ties it with a lower index."""
    if n == 0:
        return
    isn, v = _rank_arrays(vals[:n])
    selm = np.zeros(n, dtype=bool)
    selm[sel] = True
    s_idx = np.nonzero(selm)[0]
    u_idx = np.nonzero(~selm)[0]
    if len(s_idx) == 0 or len(u_idx) == 0:
        return
    sn, sv = isn[s_idx][:, None], v[s_idx][:, None]
    un, uv = isn[u_idx][None, :], v[u_idx][None, :]
    s_beats = (sn & ~un) | (~sn & ~un & (sv > uv))
    s_same = (sn & un) | (~sn & ~un & (sv == uv))
    lower = s_idx[:, None] < u_idx[None, :]
    ok = s_beats | (s_same & lower)
    assert ok.all(), "a selected element does not dominate an unselected one"


def pin_pairwise(orc, seed=1):
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        for dist in ("ties", "normal", "special"):
            rows, cols = 6, 300
            if dist == "ties":
                base = rng.integers(-5, 5, size=(rows, cols)).astype(np.float32)
            elif dist == "normal":
                base = rng.standard_normal((rows, cols)).astype(np.float32)
            else:
                base = rng.standard_normal((rows, cols)).astype(np.float32)
                pick = rng.integers(0, 12, size=base.shape)
                base[pick == 0] = np.nan
                base[pick == 1] = -0.0
                base[pick == 2] = 0.0
                base[pick == 3] = np.inf
                base[pick == 4] = -np.inf
            x = bf16_bits(torch.from_numpy(base).to(torch.bfloat16)).copy() if dtype == "bf16" else base
            vals = decode(x)
            row_end = rng.integers(0, cols + 1, size=rows).astype(np.int32)
            for k in (1, 7, 64, 150, 299, 300, 400):
                v, idx, flag = orc.topk(x, k, row_end=row_end, sorted_index=False)
                for i in range(rows):
                    n = valid_len(row_end, i, cols)
                    sel = check_row_contract(vals[i], raw_bits(x[i]), n, k, idx[i],
                                             raw_bits(v[i]), False, dtype == "bf16")
                    check_pairwise(vals[i], n, sel)
                    assert flag[i] == expected_flag(vals[i], n, k)


# ---------------------------------------------------------------------------
# library special cases
# ---------------------------------------------------------------------------

def pin_numpy_stable_argsort(orc, seed=2):
    """Rows without NaN: the set is numpy's stable argsort of -x, truncated."""
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        base = rng.integers(-20, 20, size=(5, 1000)).astype(np.float32) * 0.5
        base[base == 0.0] = -0.0  # both zeros present
        base[:, ::7] = 0.0
        x = bf16_bits(torch.from_numpy(base).to(torch.bfloat16)).copy() if dtype == "bf16" else base
        vals = decode(x)
        for k in (1, 10, 333, 1000, 1200):
            for srt in (False, True):
                v, idx, _ = orc.topk(x, k, sorted_index=srt)
                for i in range(x.shape[0]):
                    c = min(k, 1000)
                    want = np.argsort(-vals[i], kind="stable")[:c]
                    got = idx[i, :c].astype(np.int64)
                    assert sorted(got.tolist()) == sorted(want.tolist())
                    if srt:
                        assert got.tolist() == sorted(want.tolist())


def _ranks_before(a_val, a_idx, b_val, b_idx) -> bool:
    """(a_val, a_idx) comes before (b_val, b_idx) in value order: NaN above
    everything, NaNs equal, -0 equal to +0, equal values by ascending index."""
    an, bn = bool(np.isnan(a_val)), bool(np.isnan(b_val))
    if an != bn:
        return an
    if not an and a_val != b_val:
        return a_val > b_val
    return a_idx < b_idx


def pin_value_order(orc, seed=9):
    """sorted_index=2: rows without NaN equal numpy's stable argsort of -x
    position by position; every row (NaN, +-0, ties included) is in value
    order with ties by ascending index; the set matches the unsorted call."""
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        base = rng.integers(-20, 20, size=(5, 1000)).astype(np.float32) * 0.5
        base[base == 0.0] = -0.0
        base[:, ::7] = 0.0
        x = bf16_bits(torch.from_numpy(base).to(torch.bfloat16)).copy() if dtype == "bf16" else base
        vals = decode(x)
        for k in (1, 10, 333, 1000, 1200):
            _, idx, _ = orc.topk(x, k, sorted_index=2)
            for i in range(x.shape[0]):
                c = min(k, 1000)
                want = np.argsort(-vals[i], kind="stable")[:c]
                assert idx[i, :c].astype(np.int64).tolist() == want.tolist()
                assert (idx[i, c:] == -1).all()
        xs = _tiny_rows(rng, 12, 40, dtype)
        vs = decode(xs)
        row_end = rng.integers(0, 45, size=12).astype(np.int32)
        for k in (1, 3, 17, 40, 50):
            v, idx, _ = orc.topk(xs, k, row_end=row_end, sorted_index=2)
            _, idx0, _ = orc.topk(xs, k, row_end=row_end, sorted_index=0)
            for i in range(xs.shape[0]):
                n = valid_len(row_end, i, 40)
                sel = check_row_contract(vs[i], raw_bits(xs[i]), n, k, idx[i], raw_bits(v[i]),
                                         False, dtype == "bf16")
                assert sorted(sel) == sorted(int(t) for t in idx0[i, :min(k, n)])
                for a, b in zip(sel, sel[1:]):
                    assert _ranks_before(vs[i][a], a, vs[i][b], b), (dtype, k, i, a, b)


def pin_custom_fills(orc, seed=10):
    """Rows shorter than k: slots [n, k) hold the given fill index and the
    given fill value bits, and slots [0, n) are the row's columns in order
    (the closed form of a short row), whatever the fills."""
    rng = np.random.default_rng(seed)
    for dtype, bits in (("bf16", 0x7FC0), ("f32", 0x3F800000)):
        x = _tiny_rows(rng, 6, 30, dtype)
        row_end = np.array([0, 1, 7, 19, 30, 29], dtype=np.int32)
        for itype, fill in ((np.int32, -7), (np.int64, 2 ** 40)):
            v, idx, _ = orc.topk(x, 32, row_end=row_end, sorted_index=True, indices_type=itype,
                                 idx_fill=fill, val_fill_bits=bits)
            for i in range(6):
                n = int(row_end[i])
                assert idx[i, :n].tolist() == list(range(n))
                assert (idx[i, n:] == fill).all()
                assert (raw_bits(v[i])[:n] == raw_bits(x[i])[:n]).all()
                assert (raw_bits(v[i])[n:] == bits).all()


def pin_torch_topk_distinct(orc, seed=3):
    """Rows of distinct values: the set and values equal torch.topk's."""
    g = torch.Generator().manual_seed(seed)
    x = torch.stack([torch.randperm(5000, generator=g) for _ in range(8)]).float() * 0.37 - 900.0
    for r in range(x.shape[0]):
        assert torch.unique(x[r]).numel() == x.shape[1]
    xn = x.numpy()
    for k in (1, 100, 4096):
        v, idx, _ = orc.topk(xn, k, sorted_index=False, indices_type=np.int64)
        tv, ti = torch.topk(x, k, dim=1, largest=True, sorted=True)
        for r in range(x.shape[0]):
            assert set(idx[r].tolist()) == set(ti[r].tolist())
            order = np.argsort(idx[r])
            torder = torch.argsort(ti[r])
            assert np.array_equal(v[r][order], tv[r][torder].numpy())


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_closed_forms(orc):
    for dtype in ("bf16", "f32"):
        def mk(a):
            a = np.asarray(a, dtype=np.float32)
            if dtype == "bf16":
                return bf16_bits(torch.from_numpy(a).to(torch.bfloat16)).copy()
            return a
        n = 200  # integers < 256 are exact in bf16
        # all equal -> 0..c-1
        x = mk(np.full((2, n), 1.5))
        for k in (1, 50, 200, 300):
            _, idx, _ = orc.topk(x, k, sorted_index=True)
            c = min(k, n)
            assert idx[0, :c].tolist() == list(range(c))
            assert (idx[0, c:] == -1).all()
        # ascending -> n-c..n-1
        x = mk(np.tile(np.arange(n), (2, 1)))
        for k in (1, 50, 200):
            _, idx, _ = orc.topk(x, k, sorted_index=True)
            assert idx[1, :k].tolist() == list(range(n - k, n))
        # descending -> 0..c-1
        x = mk(np.tile(-np.arange(n), (2, 1)))
        for k in (1, 50, 200):
            _, idx, _ = orc.topk(x, k, sorted_index=True)
            assert idx[0, :k].tolist() == list(range(k))
        # end bounds: ascending row, end e -> e-c..e-1 ; e <= 0 -> all padding
        x = mk(np.tile(np.arange(n), (4, 1)))
        re = np.array([0, -5, 17, 500], dtype=np.int32)
        v, idx, flag = orc.topk(x, 10, row_end=re, sorted_index=True)
        assert (idx[0] == -1).all() and (idx[1] == -1).all()
        assert idx[2].tolist() == list(range(7, 17))
        assert idx[3].tolist() == list(range(190, 200))
        pad = BF16_NEG_INF if dtype == "bf16" else F32_NEG_INF_BITS
        assert (raw_bits(v[0]) == pad).all()
        # NaNs rank first: every NaN position is selected when k >= count
        row = np.arange(n, dtype=np.float32)
        row[[3, 50, 120]] = np.nan
        x = mk(row[None, :])
        _, idx, flag = orc.topk(x, 5, sorted_index=True)
        assert idx[0].tolist() == [3, 50, 120, 198, 199]
        assert flag[0] == 1
        # +-0 are equal: the lower index wins among zeros
        row = np.array([-0.0, 0.0, -0.0, 0.0, -1.0], dtype=np.float32)
        _, idx, _ = orc.topk(mk(row[None, :]), 2, sorted_index=True)
        assert idx[0].tolist() == [0, 1]
        # -inf is a real value that outranks the padding
        row = np.array([-np.inf, -np.inf, 3.0], dtype=np.float32)
        _, idx, _ = orc.topk(mk(row[None, :]), 3, sorted_index=True)
        assert idx[0].tolist() == [0, 1, 2]


def pin_nan_flag_rule(orc):
    """DeepSelect tutorial, NaN section: rows of valid length <= k are not checked."""
    for dtype in ("bf16", "f32"):
        base = np.arange(64, dtype=np.float32)[None, :].repeat(6, axis=0)
        base[0, 10] = np.nan        # long row, NaN in range  -> flagged
        base[1, 60] = np.nan        # NaN beyond end (end 40) -> not flagged
        base[2, 5] = np.nan         # short row (end 8 <= k)  -> not flagged
        base[3, 8] = np.nan         # end 9 = k+1, NaN at 8   -> flagged
        # row 4: no NaN -> not flagged; row 5: NaN at column 0, full row -> flagged
        base[5, 0] = np.nan
        x = bf16_bits(torch.from_numpy(base).to(torch.bfloat16)).copy() if dtype == "bf16" else base
        re = np.array([64, 40, 8, 9, 64, 64], dtype=np.int32)
        _, _, flag = orc.topk(x, 8, row_end=re)
        assert flag.tolist() == [1, 0, 0, 1, 0, 1]


def pin_row_stride_and_index_types(orc, seed=4):
    """A padded-stride view equals its contiguous copy; int64 equals int32."""
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        base = rng.standard_normal((7, 520)).astype(np.float32)
        full = bf16_bits(torch.from_numpy(base).to(torch.bfloat16)).copy() if dtype == "bf16" else base
        view = full[:, :500]
        cont = np.ascontiguousarray(view)
        for k in (3, 100, 500):
            a = orc.topk(view, k, sorted_index=True)
            b = orc.topk(cont, k, sorted_index=True)
            c = orc.topk(cont, k, sorted_index=True, indices_type=np.int64)
            assert np.array_equal(a[1], b[1])
            assert np.array_equal(raw_bits(a[0]), raw_bits(b[0]))
            assert np.array_equal(b[1].astype(np.int64), c[1])


def pin_values_are_copies(orc, seed=5):
    rng = np.random.default_rng(seed)
    x = _tiny_rows(rng, 16, 40, "bf16")
    v, idx, _ = orc.topk(x, 12)
    for i in range(x.shape[0]):
        for j in range(12):
            assert raw_bits(v[i])[j] == raw_bits(x[i])[idx[i, j]]
    x = _tiny_rows(rng, 16, 40, "f32")
    v, idx, _ = orc.topk(x, 12)
    for i in range(x.shape[0]):
        for j in range(12):
            assert raw_bits(v[i])[j] == raw_bits(x[i])[idx[i, j]]


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------

def _np_key(t: torch.Tensor) -> np.ndarray:
    return bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


def pin_gather_library(orc, seed=6):
    """Equal to torch advanced indexing and to index_select over b*L + pos."""
    g = torch.Generator().manual_seed(seed)
    for dtype in (torch.bfloat16, torch.float32):
        for B in (1, 3):
            L, D, R, P = 37, 16, 5, 9
            key = torch.randn(B, L, D, generator=g).to(dtype)
            pos = torch.randint(-2, L + 2, (B, R, P), generator=g).to(torch.int32)
            out = orc.gather(_np_key(key), pos.numpy())
            safe = pos.long().clamp(0, L - 1)
            bidx = torch.arange(B).view(B, 1, 1).expand(B, R, P)
            want_adv = key[bidx, safe]
            flat = (bidx * L + safe).reshape(-1)
            want_sel = key.reshape(B * L, D).index_select(0, flat).view(B, R, P, D)
            assert out.shape == (B, R, P, D) and out.dtype == _np_key(key).dtype
            assert np.array_equal(out, _np_key(want_adv))
            assert np.array_equal(out, _np_key(want_sel))


def pin_gather_batches_do_not_mix(orc):
    """Batch b reads only key[b]: key[b] filled with b, output row equals b."""
    B, L, D = 4, 10, 8
    key = torch.arange(B, dtype=torch.float32).view(B, 1, 1).expand(B, L, D).contiguous()
    pos = torch.randint(0, L, (B, 3, 5), generator=torch.Generator().manual_seed(7)).to(torch.int64)
    out = orc.gather(key.numpy(), pos.numpy())
    for b in range(B):
        assert (out[b] == b).all()


def pin_gather_noncontiguous_and_repeats(orc, seed=8):
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(40, 2, 16, generator=g).to(torch.bfloat16)
    key = base.transpose(0, 1)          # [2, 40, 16], strides (16, 32, 1)
    pos = torch.randint(0, 40, (2, 3, 6), generator=g).to(torch.int32)
    pos[:, :, ::2] = pos[:, :, :1]       # repeated positions within a row
    out = orc.gather(_np_key(key), pos.numpy())
    want = _np_key(key.contiguous())
    for b in range(2):
        for r in range(3):
            for j in range(6):
                assert np.array_equal(out[b, r, j], want[b, int(pos[b, r, j])])


def pin_gather_masked_fill(orc, seed=11):
    """The masked fill: rows at positions inside [0, L) equal the clamped
    gather's, every other row is zero; by brute force over a tiny key whose
    rows are all non-zero, with positions -3 .. L + 2 (L itself included)."""
    g = torch.Generator().manual_seed(seed)
    for dtype in (torch.bfloat16, torch.float32):
        B, L, D, R = 2, 6, 8, 3
        key = (torch.rand(B, L, D, generator=g) + 0.5).to(dtype)   # no zero element
        pos = torch.arange(-3, L + 3, dtype=torch.int32).repeat(B, R, 1)
        P = pos.shape[2]
        got = orc.gather(_np_key(key), pos.numpy(), pad="zero")
        kz = _np_key(key)
        for b in range(B):
            for r in range(R):
                for j in range(P):
                    p = int(pos[b, r, j])
                    if 0 <= p < L:
                        assert np.array_equal(got[b, r, j], kz[b, p])
                    else:
                        assert not got[b, r, j].any()
        clamp = orc.gather(_np_key(key), pos.numpy())
        inside = ((pos >= 0) & (pos < L)).numpy()
        assert np.array_equal(got[inside], clamp[inside])


ALL_PINS = [
    pin_bruteforce_tiny,
    pin_pairwise,
    pin_numpy_stable_argsort,
    pin_value_order,
    pin_custom_fills,
    pin_torch_topk_distinct,
    pin_closed_forms,
    pin_nan_flag_rule,
    pin_row_stride_and_index_types,
    pin_values_are_copies,
    pin_gather_library,
    pin_gather_batches_do_not_mix,
    pin_gather_noncontiguous_and_repeats,
    pin_gather_masked_fill,
]
