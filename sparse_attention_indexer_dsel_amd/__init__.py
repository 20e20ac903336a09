"""Row-wise top-k and compressed-key gather on MI355X, over the ``libdsel.so`` C ABI.

This module only marshals tensors into the C entry points of
``include/dsel.h`` (same names without the ``dsel_`` prefix); every step of
the computation runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.  Importing fails loudly when the library has
not been built (``python sparse_attention_indexer_dsel_amd/build_lib.py``).

Call shapes follow the DeepSelect tutorial ("Sheshisa Imisebenzi ye-PyTorch
TopK nge-DeepSelect"): ``topk(x, k, sorted_index=..., indices_type=...,
return_value=..., end=..., output_idx=...)`` on a 2-D input whose last dim is
contiguous and whose row stride is a multiple of ``stride_requirement()[0]``
bytes; the outputs' row strides are aligned to ``stride_requirement()[1]``
bytes, so they may be non-contiguous views.  The gather follows MindSpore
hyper-parallel PR #1094: ``gather_rows(key, pos)`` equals
``key[batch_ids, pos.clamp(0, L-1)]``, and ``topk_gather`` runs that
page's chain tail (top-k, then the gather of one or more keys at the selected
positions, clamped or zero-filled) in one call.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["stride_requirement", "topk", "gather_rows", "topk_gather", "check_workspaces",
           "read_floor", "DselError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsel.so")

DSEL_OK, DSEL_ERR_ARG, DSEL_ERR_K, DSEL_ERR_ALIGN, DSEL_ERR_WORKSPACE, DSEL_ERR_DEVICE, \
    DSEL_ERR_SPLIT = 0, -1, -2, -3, -4, -5, -6
DSEL_BF16, DSEL_F32 = 0, 1
DSEL_I32, DSEL_I64 = 0, 1
DSEL_ROWS_AUTO, DSEL_ROWS_NATURAL, DSEL_ROWS_DUAL_CHUNK = 0, 1, 2
_ROW_ORDERS = {None: DSEL_ROWS_AUTO, "auto": DSEL_ROWS_AUTO, "natural": DSEL_ROWS_NATURAL,
               "dual_chunk": DSEL_ROWS_DUAL_CHUNK}
_NAMES = {DSEL_ERR_ARG: "DSEL_ERR_ARG", DSEL_ERR_K: "DSEL_ERR_K", DSEL_ERR_ALIGN: "DSEL_ERR_ALIGN",
          DSEL_ERR_WORKSPACE: "DSEL_ERR_WORKSPACE", DSEL_ERR_DEVICE: "DSEL_ERR_DEVICE",
          DSEL_ERR_SPLIT: "DSEL_ERR_SPLIT (a split row's workgroups did not all meet; "
                          "its output is undefined and the workspace was reset)"}


class DselError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {_NAMES.get(code, code)}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python sparse_attention_indexer_dsel_amd/build_lib.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32, szp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
    lib.dsel_stride_requirement.restype = i32
    lib.dsel_stride_requirement.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.dsel_topk.restype = i32
    lib.dsel_topk.argtypes = [vp, i32, i64, i64, i64, i64, vp, i32, i32, i32, vp, i64, vp, i64,
                              vp, vp, szp, vp]
    lib.dsel_topk_ex.restype = i32
    lib.dsel_topk_ex.argtypes = [vp, i32, i64, i64, i64, i64, vp, i32, i32, i32, vp, i64, vp,
                                 i64, vp, vp, szp, vp, i64, ctypes.c_uint32, i32]
    lib.dsel_topk_check.restype = i32
    lib.dsel_topk_check.argtypes = [vp, ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.dsel_topk_gather.restype = i32
    lib.dsel_topk_gather.argtypes = [vp, i32, i64, i64, i64, i64, vp, i32, i32, vp, i64, vp, i64,
                                     vp, i32, i32, vp, szp, vp]
    lib.dsel_gather_rows.restype = i32
    lib.dsel_gather_rows.argtypes = [vp, i32, i64, i64, i64, i64, i64, vp, i32, i64, i64, i64,
                                     vp, vp]
    lib.dsel_read_floor.restype = i32
    lib.dsel_read_floor.argtypes = [vp, i64, vp, vp]
    return lib


_lib = _load()


def _check(code: int, what: str) -> None:
    if code != DSEL_OK:
        raise DselError(code, what)


def stride_requirement() -> Tuple[int, int]:
    """(input row-stride alignment, output row-stride alignment) in bytes."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.dsel_stride_requirement(ctypes.byref(a), ctypes.byref(b)), "dsel_stride_requirement")
    return int(a.value), int(b.value)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DSEL_BF16
    if dt == torch.float32:
        return DSEL_F32
    raise TypeError(f"unsupported value dtype {dt} (bf16 or fp32)")


def _index_code(dt: torch.dtype) -> int:
    if dt == torch.int32:
        return DSEL_I32
    if dt == torch.int64:
        return DSEL_I64
    raise TypeError(f"unsupported index dtype {dt} (int32 or int64)")


def _aligned_empty(rows: int, k: int, dtype: torch.dtype, device) -> torch.Tensor:
    """[rows, k] view of a buffer whose row stride is aligned to the output alignment."""
    _, out_align = stride_requirement()
    esz = torch.empty((), dtype=dtype).element_size()
    stride = -(-k * esz // out_align) * out_align // esz
    return torch.empty(rows, stride, dtype=dtype, device=device)[:, :k]


# Zero-initialised scratch per (device, stream), for split rows; the library
# leaves it zeroed after every call.  A bigger one replaces it when a call
# needs more, but every buffer ever handed out stays alive in _RETIRED: a
# HIP graph captured with an older one keeps using its address on replay.
_WORKSPACES = {}
_RETIRED = []


def _workspace(device: torch.device, stream_ptr: int, nbytes: int) -> torch.Tensor:
    """The (device, stream)'s workspace of at least nbytes, zero-filled on
    the current stream (the caller makes that the stream the kernels run on)."""
    key = (device.index, stream_ptr)
    ws = _WORKSPACES.get(key)
    need = max(int(nbytes), 256)
    if ws is None or ws.numel() < need:
        if ws is not None:
            _RETIRED.append(ws)
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def check_workspaces() -> None:
    """Raise DselError(DSEL_ERR_SPLIT) if a split-row rendezvous gave up on any
    workspace since the last check (that call's split rows hold undefined
    output; the workspace is reset).  Synchronises each workspace's stream."""
    for (dev, sptr), ws in list(_WORKSPACES.items()):
        _check_one(ws, sptr)


def _check_one(ws: torch.Tensor, sptr: int) -> None:
    bits = ctypes.c_uint32(0)
    with torch.cuda.device(ws.device):
        _check(_lib.dsel_topk_check(ws.data_ptr(), ws.numel(), sptr, ctypes.byref(bits)),
               f"dsel_topk (error bits {bits.value:#x})")


def _row_stride(t: torch.Tensor) -> int:
    """Row stride in elements; a one-row tensor's stride is never used for
    addressing, so report the smallest aligned stride covering its row."""
    if t.shape[0] > 1:
        return int(t.stride(0))
    per = 16 // t.element_size()
    return -(-max(int(t.shape[1]), 1) // per) * per


def _fill_bits(value, dtype: torch.dtype) -> int:
    """Raw bits of `value` in the value dtype (None: -inf)."""
    v = float("-inf") if value is None else float(value)
    t = torch.tensor([v], dtype=dtype)
    return int(t.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).item()) & (
        0xFFFF if dtype == torch.bfloat16 else 0xFFFFFFFF)


def _topk_call(x, k, end, order, itype, return_value, idx, val, flag, ws_ptr, ws_bytes, sptr,
               idx_fill=-1, val_fill=None, row_order=0):
    return _lib.dsel_topk_ex(
        x.data_ptr(), _dtype_code(x.dtype), x.shape[0], x.shape[1], _row_stride(x),
        int(k), end.data_ptr() if end is not None else None,
        int(order), _index_code(itype), int(bool(return_value)),
        idx.data_ptr(), _row_stride(idx),
        val.data_ptr() if val is not None else None, _row_stride(val) if val is not None else 0,
        flag.data_ptr(), ws_ptr, ctypes.byref(ws_bytes), sptr, int(idx_fill),
        _fill_bits(val_fill, x.dtype), int(row_order))


def _check_input(x: torch.Tensor) -> None:
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, cols)")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("the last dim of x must be contiguous")


def topk(x: torch.Tensor, topk: int, *, end: Optional[torch.Tensor] = None,
         sorted_index: bool = False, sorted: Optional[bool] = None,
         indices_type: torch.dtype = torch.int32, return_value: bool = True,
         output_idx: Optional[torch.Tensor] = None, by_value: bool = False,
         idx_oob_fill_value: int = -1, value_oob_fill_value: Optional[float] = None,
         abort_when_nan_found: bool = False, check: bool = False, stream=None,
         row_order: Optional[str] = None
         ) -> Tuple[Optional[torch.Tensor], torch.Tensor, torch.Tensor]:
    """Row-wise top-k of ``x`` [rows, cols] (bf16 or fp32), 1 <= topk <= 4096.

    Returns ``(values or None, indices, nan_flag)``: indices [rows, topk] of
    ``indices_type`` (ascending per row; -1 past a short row's length),
    values [rows, topk] of x's dtype (bit copies; -inf padding), and a uint8
    [rows] NaN flag (set for rows longer than topk holding a NaN in range).
    ``end`` (int32 [rows]) is each row's exclusive end.  ``sorted`` is
    accepted as another name for ``sorted_index``.  ``output_idx`` is a
    caller-owned [rows, >= topk] index buffer with an aligned row stride.
    ``by_value=True`` orders each row's selection by value instead (largest
    first, equal values by ascending column; NaN first, -0 equal to +0);
    it takes precedence over ``sorted_index``.  ``idx_oob_fill_value`` and
    ``value_oob_fill_value`` (default -1 and -inf) fill the slots past a
    short row's length.  ``abort_when_nan_found=True`` raises
    FloatingPointError when a row longer than ``topk`` holds a NaN (this
    waits for the call to finish); by default the flag is only returned.
    ``check=True`` waits for the call and raises DselError (DSEL_ERR_SPLIT)
    if the workgroups of a split row (rows over 16384 columns) could not all
    run at once, so that its output is undefined; see ``check_workspaces``.
    With ``stream`` given, the outputs and workspace are allocated and zeroed
    on that stream and the kernels run there; ordering against other streams
    (the producer of ``x``, the consumers of the outputs) is the caller's.
    ``row_order`` ("natural", "dual_chunk", or None/"auto": dual chunk when
    ``end`` is given) is the order in which the workers take rows; it
    changes timing only, never the output.
    """
    _check_input(x)
    if row_order not in _ROW_ORDERS:
        raise ValueError(f"row_order must be one of {sorted(k for k in _ROW_ORDERS if k)} or None")
    ro = _ROW_ORDERS[row_order]
    if sorted is not None:
        sorted_index = bool(sorted)
    order = 2 if by_value else int(bool(sorted_index))
    rows = x.shape[0]
    dev = x.device
    if end is not None:
        if end.dtype != torch.int32 or end.shape != (rows,) or end.device != dev:
            raise ValueError("end must be an int32 [rows] tensor on x's device")
        end = end.contiguous()
    if output_idx is not None:
        if output_idx.dtype != indices_type:
            raise ValueError("output_idx dtype must equal indices_type")
        if output_idx.dim() != 2 or output_idx.shape[0] != rows or output_idx.shape[1] < topk:
            raise ValueError("output_idx must be [rows, >= topk]")
        if output_idx.shape[1] > 1 and output_idx.stride(1) != 1:
            raise ValueError("output_idx's last dim must be contiguous")
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream(dev) if stream is None else stream
        with torch.cuda.stream(s):
            # allocated (and the workspace zeroed) on the stream the kernels run on
            idx = output_idx if output_idx is not None else _aligned_empty(rows, topk,
                                                                          indices_type, dev)
            val = _aligned_empty(rows, topk, x.dtype, dev) if return_value else None
            flag = torch.empty(rows, dtype=torch.uint8, device=dev)
            sptr = int(s.cuda_stream)
            nb = ctypes.c_size_t(0)
            _check(_topk_call(x, topk, end, order, indices_type, return_value, idx, val, flag,
                              None, nb, sptr, idx_oob_fill_value, value_oob_fill_value, ro),
                   "dsel_topk (size query)")
            ws = _workspace(dev, sptr, nb.value)
            nb = ctypes.c_size_t(ws.numel())
            _check(_topk_call(x, topk, end, order, indices_type, return_value, idx, val, flag,
                              ws.data_ptr(), nb, sptr, idx_oob_fill_value, value_oob_fill_value, ro),
                   "dsel_topk")
            if check:
                _check_one(ws, sptr)
    if output_idx is not None:
        idx = output_idx[:, :topk]
    if abort_when_nan_found and bool(flag.any()):
        rows_hit = torch.nonzero(flag).flatten()[:8].tolist()
        raise FloatingPointError(f"NaN in rows longer than topk (first rows: {rows_hit})")
    return val, idx, flag


def gather_rows(key: torch.Tensor, pos: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """out[b, r, j, :] = key[b, clamp(pos[b, r, j], 0, L-1), :].

    key: [B, L, D] bf16/fp32 with a contiguous last dim (any batch and row
    strides).  pos: [B, R, P] int32/int64 with a contiguous last dim and
    pos.stride(0) == R * pos.stride(1) (a [B*R, k] top-k index buffer viewed
    as [B, R, k] qualifies).  Returns a contiguous [B, R, P, D] tensor.
    """
    if key.dim() != 3 or pos.dim() != 3:
        raise ValueError("key must be [B, L, D] and pos [B, R, P]")
    B, L, D = key.shape
    Bp, R, P = pos.shape
    if Bp != B:
        raise ValueError("pos and key disagree on the batch size")
    if D > 1 and key.stride(2) != 1:
        raise ValueError("key's last dim must be contiguous")
    if P > 1 and pos.stride(2) != 1:
        raise ValueError("pos's last dim must be contiguous")
    prs = pos.stride(1) if R > 1 else max(P, pos.stride(1))
    if B > 1 and R > 0 and pos.stride(0) != R * prs:
        raise ValueError("pos batch stride must equal R * row stride")
    if key.device != pos.device or not key.is_cuda:
        raise ValueError("key and pos must be GPU tensors on one device")
    if out is not None and (out.shape != (B, R, P, D) or not out.is_contiguous()
                            or out.dtype != key.dtype):
        raise ValueError("out must be a contiguous [B, R, P, D] tensor of key's dtype")
    with torch.cuda.device(key.device):
        s = torch.cuda.current_stream(key.device) if stream is None else stream
        with torch.cuda.stream(s):
            if out is None:
                out = torch.empty(B, R, P, D, dtype=key.dtype, device=key.device)
        sptr = int(s.cuda_stream)
        _check(_lib.dsel_gather_rows(
            key.data_ptr(), _dtype_code(key.dtype), B, L, D,
            key.stride(0), key.stride(1), pos.data_ptr(), _index_code(pos.dtype), R, P, prs,
            out.data_ptr(), sptr), "dsel_gather_rows")
    return out


def read_floor(x: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The streaming-read floor (a measurement helper): one launch reads all
    of the contiguous GPU tensor x once with the select's load form and
    returns int32 words, word b the XOR of the 32-bit words of x's b-th
    64 KiB block.  x's size in bytes must be a multiple of 16."""
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    nbytes = x.numel() * x.element_size()
    words = -(-nbytes // 65536)
    with torch.cuda.device(x.device):
        s = torch.cuda.current_stream(x.device) if stream is None else stream
        if out is None:
            with torch.cuda.stream(s):
                out = torch.empty(max(words, 1), dtype=torch.int32, device=x.device)
        elif out.dtype != torch.int32 or out.numel() < words or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous int32 tensor of at least {words} words")
        _check(_lib.dsel_read_floor(x.data_ptr(), nbytes, out.data_ptr(), int(s.cuda_stream)),
               "dsel_read_floor")
    return out[:words]


class _GatherKey(ctypes.Structure):
    """DselGatherKey of dsel.h."""
    _fields_ = [("key", ctypes.c_void_p), ("dtype", ctypes.c_int), ("len", ctypes.c_int64),
                ("dim", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("out", ctypes.c_void_p)]


_PADS = {"clamp": 0, "zero": 1}


def topk_gather(x: torch.Tensor, topk: int, keys, *, rows_per_batch: int,
                end: Optional[torch.Tensor] = None, sorted_index: bool = False,
                by_value: bool = False, indices_type: torch.dtype = torch.int32,
                pad: str = "clamp", check: bool = False, stream=None, out=None,
                output_idx: Optional[torch.Tensor] = None):
    """Row-wise top-k of ``x`` and the gather of each key at the selected
    positions, in one call (dsel_topk_gather).

    ``keys``: a list of 1..4 tensors [B, L, D] (bf16/fp32, last dim
    contiguous, any batch and row strides) with B = rows / rows_per_batch.
    Returns ``(indices, nan_flag, outs)``: indices and flag as ``topk`` (no
    values), and for each key a contiguous [rows, topk, D] tensor with
    ``outs[g][r, j] = keys[g][r // rows_per_batch, p]``, p = indices[r, j];
    a position outside [0, L) (a short row's -1 padding) is clamped into it
    (``pad="clamp"``) or gives a zero row (``pad="zero"``).  ``out`` (a list
    of contiguous [rows, topk, D] tensors, one per key) and ``output_idx``
    (as in ``topk``) take caller-owned outputs.
    """
    _check_input(x)
    if pad not in _PADS:
        raise ValueError("pad must be 'clamp' or 'zero'")
    keys = list(keys)
    if not 1 <= len(keys) <= 4:
        raise ValueError("between one and four keys")
    rows = x.shape[0]
    dev = x.device
    if rows_per_batch < 1 or rows % rows_per_batch:
        raise ValueError("rows must be a multiple of rows_per_batch")
    B = rows // rows_per_batch
    for kt in keys:
        if kt.dim() != 3 or kt.shape[0] != B or kt.device != dev:
            raise ValueError("each key must be [rows // rows_per_batch, L, D] on x's device")
        if kt.shape[2] > 1 and kt.stride(2) != 1:
            raise ValueError("a key's last dim must be contiguous")
    if end is not None:
        if end.dtype != torch.int32 or end.shape != (rows,) or end.device != dev:
            raise ValueError("end must be an int32 [rows] tensor on x's device")
        end = end.contiguous()
    order = 2 if by_value else int(bool(sorted_index))
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream(dev) if stream is None else stream
        with torch.cuda.stream(s):
            if output_idx is not None:
                if (output_idx.dtype != indices_type or output_idx.dim() != 2
                        or output_idx.shape[0] != rows or output_idx.shape[1] < topk
                        or (output_idx.shape[1] > 1 and output_idx.stride(1) != 1)):
                    raise ValueError("output_idx must be [rows, >= topk] of indices_type")
                idx = output_idx
            else:
                idx = _aligned_empty(rows, topk, indices_type, dev)
            flag = torch.empty(rows, dtype=torch.uint8, device=dev)
            if out is not None:
                outs = list(out)
                if len(outs) != len(keys) or any(
                        o.shape != (rows, topk, kt.shape[2]) or o.dtype != kt.dtype
                        or not o.is_contiguous() for o, kt in zip(outs, keys)):
                    raise ValueError("out must hold a contiguous [rows, topk, D] tensor per key")
            else:
                outs = [torch.empty(rows, topk, kt.shape[2], dtype=kt.dtype, device=dev)
                        for kt in keys]
            desc = (_GatherKey * len(keys))(*[
                _GatherKey(kt.data_ptr(), _dtype_code(kt.dtype), kt.shape[1], kt.shape[2],
                           kt.stride(0), kt.stride(1), o.data_ptr()) for kt, o in zip(keys, outs)])
            sptr = int(s.cuda_stream)

            def call(ws_ptr, nb):
                return _lib.dsel_topk_gather(
                    x.data_ptr(), _dtype_code(x.dtype), rows, x.shape[1], _row_stride(x), int(topk),
                    end.data_ptr() if end is not None else None, order, _index_code(indices_type),
                    idx.data_ptr(), _row_stride(idx), flag.data_ptr(), int(rows_per_batch), desc,
                    len(keys), _PADS[pad], ws_ptr, ctypes.byref(nb), sptr)

            nb = ctypes.c_size_t(0)
            _check(call(None, nb), "dsel_topk_gather (size query)")
            ws = _workspace(dev, sptr, nb.value)
            nb = ctypes.c_size_t(ws.numel())
            _check(call(ws.data_ptr(), nb), "dsel_topk_gather")
            if check:
                _check_one(ws, sptr)
    return idx[:, :topk], flag, outs
