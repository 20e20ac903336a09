"""Per-phase timestamps of the top-k kernels on a named workload.

    python -m sparse_attention_indexer_dsel_amd.phase_stamps build
    python -m sparse_attention_indexer_dsel_amd.phase_stamps run {wave,wx,whole} cfgN

``build`` (no GPU needed) compiles an instrumented copy of the library,
``libdsel_stamps.so`` beside ``libdsel.so``, with ``DSEL_PHASE_STAMPS``
defined: at each phase boundary of the one-wave rows' kernel (per row), the
fp32 window-exchange kernel (per workgroup) and the whole-row kernel (per
row) one thread records the GPU's 100 MHz real-time clock.  A stamp does
not wait for memory: it marks when the thread's instructions reach the
boundary (a phase that ends in a workgroup barrier ends when every wave is
there), so the kernel's loads still overlap its work as in the product
build, and a phase that starts with loads shows when they were issued, the
next one when their data was used.  ``run`` loads that build, warms it up
on the workload, clears the stamps, runs one top-k call and prints each
phase's duration (mean, percentiles, max) in nanoseconds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
STAMPS_LIB = os.path.join(HERE, "libdsel_stamps.so")
UNITS, PER_UNIT = 4096, 24


def build(verbose: bool = False) -> str:
    """Compile the instrumented library (hipcc for gfx950)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_dsel_build_lib", os.path.join(HERE, "build_lib.py"))
    bl = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bl)
    out = os.path.join(bl.BUILD, "stamps")
    os.makedirs(out, exist_ok=True)
    objs = []
    for name in ("topk", "api", "gather", "floor"):
        o = os.path.join(out, name + ".o")
        cmd = [bl._hipcc(), *bl.HIPCC_FLAGS, "-DDSEL_PHASE_STAMPS", "-I", os.path.join(ROOT, "include"),
               "-c", os.path.join(bl.CSRC, name + ".hip"), "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(o)
    subprocess.run([bl._hipcc(), "-shared", "-fPIC", f"--offload-arch={bl.ARCH}", *objs, "-o", STAMPS_LIB],
                   check=True)
    return STAMPS_LIB


def _stats(name: str, v) -> str:
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0:
        return f"  {name:26s} (none)"
    return (f"  {name:26s} mean {v.mean():8.0f} p10 {np.percentile(v, 10):8.0f} "
            f"p50 {np.percentile(v, 50):8.0f} p90 {np.percentile(v, 90):8.0f} max {v.max():8.0f}")


def collect(cfg: int):
    """Stamps of one top-k call on workload cfg, as an int64 array [units, 24]
    of nanoseconds from the earliest stamp (0 where nothing was stamped)."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import workloads as W
    import sparse_attention_indexer_dsel_amd as dsel
    if not os.path.exists(STAMPS_LIB):
        raise SystemExit(f"{STAMPS_LIB} is missing: run the build step first")
    dsel.LIB_PATH = STAMPS_LIB
    dsel._lib = dsel._load()
    lib = dsel._lib
    lib.dsel_stamps_read.argtypes = [ctypes.c_void_p]
    lib.dsel_stamps_read.restype = ctypes.c_int
    lib.dsel_stamps_clear.restype = ctypes.c_int
    case = W.make_config(cfg)
    dev = torch.device("cuda:0")
    copies = [case.x.to(dev) for _ in range(6)]
    end = case.row_end.to(dev) if case.row_end is not None else None
    s = torch.cuda.Stream()
    kw = dict(end=end, sorted_index=case.sorted_index, indices_type=case.indices_type,
              return_value=case.return_value, stream=s)
    with torch.cuda.stream(s):
        for i in range(10):
            dsel.topk(copies[i % 5], case.k, **kw)
    torch.cuda.synchronize()
    assert lib.dsel_stamps_clear() == 0
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dsel.topk(copies[5], case.k, **kw)
    torch.cuda.synchronize()
    buf = np.zeros(UNITS * PER_UNIT, dtype=np.uint64)
    assert lib.dsel_stamps_read(buf.ctypes.data) == 0
    raw = buf.reshape(UNITS, PER_UNIT).astype(np.int64)
    return raw, case


def report(kernel: str, cfg: int) -> str:
    raw, case = collect(cfg)
    used = raw[:, 0] > 0
    base = raw[used, 0].min()
    ns = lambda i: (raw[:, i] - base) * 10
    lines = [f"{case.name}: {kernel} kernel, {int(used.sum())} units stamped"]
    if kernel == "wave":  # per row: 0 start, 1 keys+histogram, 2 digit, 3 refine, 4 end; 7 = n
        n = raw[:, 7]
        long_ = used & (n > case.k)
        short = used & (n <= case.k)
        lines.append(f"rows longer than k: {int(long_.sum())}, at most k: {int(short.sum())}")
        lines.append("long rows:")
        lines.append(_stats("start", ns(0)[long_]))
        lines.append(_stats("loads, keys, histogram", (ns(1) - ns(0))[long_]))
        lines.append(_stats("first digit", (ns(2) - ns(1))[long_]))
        lines.append(_stats("second digit, cut", (ns(3) - ns(2))[long_]))
        lines.append(_stats("write", (ns(4) - ns(3))[long_]))
        lines.append(_stats("total", (ns(4) - ns(0))[long_]))
        lines.append(_stats("end", ns(4)[long_]))
        lines.append("rows of at most k:")
        lines.append(_stats("start", ns(0)[short]))
        lines.append(_stats("total", (ns(4) - ns(0))[short]))
        lines.append(_stats("end", ns(4)[short]))
    elif kernel == "wx":  # per workgroup; 7 = exchange held
        ok = used & (raw[:, 7] == 1)
        lines.append(f"the exchange held in {int(ok.sum())} of {int(used.sum())} workgroups")
        for name, a, b in (("loads issued, hist zeroed", 0, 13), ("keys, sampled histogram", 13, 1),
                           ("window digit", 1, 8), ("candidate list", 8, 9),
                           ("window keys published", 9, 14), ("header", 14, 2), ("rendezvous wait", 2, 6),
                           ("headers, boundary bin", 6, 10),
                           ("gather keys, 1st digit", 10, 11),
                           ("select, earlier counts", 11, 3),
                           ("write", 3, 4), ("finish", 4, 5)):
            lines.append(_stats(name, (ns(b) - ns(a))[ok]))
        lines.append(_stats("end", ns(5)[ok]))
    elif kernel == "whole":  # per row (list path)
        lst = used & (raw[:, 7] > 0)
        lines.append(f"rows that took the list path: {int(lst.sum())} of {int(used.sum())}")
        for name, a, b in (("loads issued", 0, 1), ("keys, zero histogram", 1, 2), ("histogram", 2, 3),
                           ("first digit", 3, 4), ("candidate list", 4, 5), ("later digits", 5, 6),
                           ("write", 6, 7), ("finish", 7, 8), ("total", 0, 8)):
            lines.append(_stats(name, (ns(b) - ns(a))[lst]))
        lines.append(_stats("start", ns(0)[lst]))
        lines.append(_stats("end", ns(8)[lst]))
    else:
        raise SystemExit(f"unknown kernel {kernel!r}: wave, wx or whole")
    return "\n".join(lines)


def main(argv=None):
    argv = list(sys.argv[1:] if argv is None else argv)
    if argv[:1] == ["build"]:
        print(build(verbose="-v" in argv))
        return 0
    if len(argv) == 3 and argv[0] == "run":
        print(report(argv[1], int(argv[2].replace("cfg", ""))), flush=True)
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main())
