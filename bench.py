"""Benchmark of the selection step (row-wise top-k, then key gather) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2]
                    [--no-per-config] [--no-cpu-baseline] [--copy-calibration]
    python bench.py --traffic-from FETCH.csv WRITE.csv   # no GPU: writes profiles/traffic.json

Prints ONE JSON line.  The headline workload is the 4 x 204800 bf16 top-k
(k = 1024, ascending int32 indices plus values); a step is one top-k call
over one batch.  ``per_config`` adds the same measurement for the five named
workloads (top-k and, where they have one, the gather), and for two of them
(the 4 x 204800 headline and the 128 x 129280 sampling rows) the top-k with
the selection ordered by value (``topk_by_value``: the select, then the
radix value-order sort).  The causal prefill rows are also timed with values
returned (``topk_with_values``).

Timing protocol
  * inputs are generated on the host from fixed seeds and copied to HBM
    before timing; each step reads a different copy of the input, and the
    copies together exceed twice the 256 MB Infinity Cache, so top-k reads
    come from HBM rather than from cache;
  * the K timed steps are captured once in a HIP graph and replayed, so the
    timed region holds no Python launch overhead; the region is bracketed
    by torch.cuda.synchronize() on both sides and wall-clock timed;
  * a HIP event pair on the kernels' stream brackets the same replay: each
    step is one top-k kernel, so events / K is that kernel's mean duration
    back to back (the roofline figure), comparable with rocprofv3's.

Byte accounting (algorithmic bytes: what the method must move)
  top-k  = sum over rows of the valid-prefix read (a row of valid length
           n <= k is read only when values are returned), + 4*rows for
           row_end, + rows*k*index bytes, + rows*k*value bytes when values
           are returned, + rows bytes of NaN flag;
  gather = written bytes + position bytes read + one compulsory read of each
           distinct key row touched.
The gather is also reported in the pages' convention (gathered output bytes
over time; MindSpore hyper-parallel PR #1094, mechanism check).

HBM traffic (roofline "traffic")
  Two rocprofv3 counter runs of this script with --copy-calibration give
  FETCH_SIZE and WRITE_SIZE per dispatch for the dominant top-k kernel and
  for a plain streaming copy of known size (torch.neg, 256 MiB in, 256 MiB
  out).  --traffic-from turns them into bytes per launch (counter value x
  known copy bytes / copy counter value) and stores them in
  profiles/traffic.json with a hash of the kernel sources; the bench reports
  them only while that hash still matches, and null otherwise.
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
COPY_CAL_BYTES = 256 << 20
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_attention_indexer_dsel_amd", "csrc", f)
                  for f in ("topk.hip", "dsel_internal.h", "api.hip")]
METRIC = "top-k rows/s and achieved HBM GB/s (% of peak) per config; gather GB/s"
# workloads also timed with the selection ordered by value (the sampling
# workload, where that order is the natural one, and the headline)
VALUE_ORDER_CONFIGS = (2, 4)
# index-only workloads also timed with values returned (the causal prefill
# rows: half of them are shorter than k, so this times the short-row value
# copy)
WITH_VALUES_CONFIGS = (3,)


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


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
# ---------------------------------------------------------------------------

def _code_only(text: str) -> str:
    """Source text without comments and whitespace: what the compiler sees."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources' code (comments and whitespace ignored), so
    that stored counter figures stay valid across comment edits only."""
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def copy_calibration(torch, stream, launches: int = 3) -> None:
    """A plain streaming copy of known size for the counter calibration:
    COPY_CAL_BYTES read and COPY_CAL_BYTES written per launch."""
    n = COPY_CAL_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(launches):
            torch.neg(src, out=dst)
    stream.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _counter_means(path: str, counter: str):
    """Mean per dispatch of `counter`, per kernel name, from a rocprofv3
    counter_collection.csv."""
    per = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {name: (float(np.mean(v)), len(v)) for name, v in out.items()}


def traffic_from(fetch_csv: str, write_csv: str, out_path: str = TRAFFIC_JSON) -> dict:
    """Per-launch HBM bytes of the top-k kernel, scaled by the copy kernel's
    reading of the same counters (counter x known bytes / copy counter)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")

    def pick(table, pat):
        names = [n for n in table if pat in n]
        if not names:
            raise SystemExit(f"no kernel matching {pat!r} in the counter file")
        return max(names, key=lambda n: table[n][1])

    copy_f, copy_w = pick(fetch, "neg"), pick(write, "neg")
    tk_f, tk_w = pick(fetch, "topk_rows"), pick(write, "topk_rows")
    f_fac = COPY_CAL_BYTES / fetch[copy_f][0]
    w_fac = COPY_CAL_BYTES / write[copy_w][0]
    rec = {
        "kernel": tk_f,
        "source_hash": kernel_source_hash(),
        "fetch_counter_per_launch": fetch[tk_f][0],
        "write_counter_per_launch": write[tk_w][0],
        "launches_sampled": [fetch[tk_f][1], write[tk_w][1]],
        "copy_fetch_counter": fetch[copy_f][0],
        "copy_write_counter": write[copy_w][0],
        "copy_bytes": COPY_CAL_BYTES,
        "fetch_factor": f_fac,
        "write_factor": w_fac,
        "fetch_bytes": fetch[tk_f][0] * f_fac,
        "write_bytes": write[tk_w][0] * w_fac,
    }
    rec["traffic_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def load_traffic():
    """The stored traffic record, or None when the kernel sources changed since."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_hash") == kernel_source_hash() else None


# ---------------------------------------------------------------------------
# GPU measurement helpers
# ---------------------------------------------------------------------------

def _valid_lengths(case):
    rows, cols = case.x.shape
    if case.row_end is None:
        return np.full(rows, cols, dtype=np.int64)
    return np.clip(case.row_end.numpy().astype(np.int64), 0, cols)


def _copies_for(nbytes: int, cap: int = 4096) -> int:
    return int(max(2, min(cap, -(-2 * MALL_BYTES // max(nbytes, 1)))))


class TopkBench:
    """Device-resident inputs (rotating copies) and a reusable top-k call."""

    def __init__(self, dsel, torch, case, stream, by_value=False):
        self.dsel, self.torch, self.case, self.stream = dsel, torch, case, stream
        self.by_value = by_value
        x = case.x
        self.in_bytes = x.numel() * x.element_size()
        self.ncopy = _copies_for(self.in_bytes)
        dev = torch.device("cuda")
        base = x.contiguous().to(dev)
        self.xs = torch.empty((self.ncopy,) + tuple(x.shape), dtype=x.dtype, device=dev)
        self.xs.copy_(base.unsqueeze(0).expand_as(self.xs))
        self.row_end = case.row_end.to(dev) if case.row_end is not None else None
        torch.cuda.synchronize()

    def call(self, i: int):
        c = self.case
        return self.dsel.topk(self.xs[i % self.ncopy], c.k, end=self.row_end,
                              sorted_index=c.sorted_index, indices_type=c.indices_type,
                              return_value=c.return_value, by_value=self.by_value,
                              stream=self.stream)

    def algorithmic_bytes(self) -> int:
        c = self.case
        esz = c.x.element_size()
        isz = 4 if c.indices_type == self.torch.int32 else 8
        return topk_algorithmic_bytes(_valid_lengths(c), c.k, esz, isz, c.return_value,
                                      c.row_end is not None)


def graph_time(torch, stream, fn, steps: int, warmup: int, reps: int = 1):
    """Capture `steps` calls of fn(i) (one kernel each) in one HIP graph and
    replay it; return (wall seconds per call, event seconds per call).  The
    event pair brackets the replay on the stream the kernels run on, so the
    second figure is the kernels' mean duration back to back."""
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):
            fn(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fn(i)
    with torch.cuda.stream(stream):
        g.replay()  # untimed replay: page in the graph
    torch.cuda.synchronize()
    best = best_ev = None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        de = e0.elapsed_time(e1) * 1e-3 / steps
        best = dt if best is None else min(best, dt)
        best_ev = de if best_ev is None else min(best_ev, de)
    del g
    return best, best_ev


def measure_topk(dsel, torch, case, stream, steps, warmup, by_value=False):
    """One top-k call per step (with by_value, the select and then the
    value-order pass: kernel_us covers both)."""
    tb = TopkBench(dsel, torch, case, stream, by_value)
    t_step, t_kern = graph_time(torch, stream, tb.call, steps, warmup, reps=3)
    nbytes = tb.algorithmic_bytes()
    rows = case.x.shape[0]
    res = {
        "rows_per_s": rows / t_step,
        "us_per_call": t_step * 1e6,
        "kernel_us": t_kern * 1e6,
        "algorithmic_bytes": nbytes,
        "gbps": nbytes / t_step / 1e9,
        "pct_peak": 100.0 * nbytes / t_step / 1e9 / HBM_PEAK_GBPS,
        "input_copies": tb.ncopy,
    }
    del tb
    torch.cuda.empty_cache()
    return res


def measure_gather(dsel, torch, case, stream, steps, warmup):
    """Gather(s) of the case's keys at the top-k positions (one call per key)."""
    dev = torch.device("cuda")
    _, idx, _ = dsel.topk(case.x.to(dev), case.k, end=case.row_end.to(dev) if case.row_end is not None else None,
                          indices_type=case.indices_type, return_value=False)
    B = case.gather_batch
    R = case.x.shape[0] // B
    pos = idx.contiguous().view(B, R, case.k)
    out = []
    for ki, key in enumerate(case.keys):
        kd = key.to(dev)
        D = key.shape[2]
        dst = torch.empty(B, R, case.k, D, dtype=key.dtype, device=dev)

        def fn(i, kd=kd, dst=dst):
            return dsel.gather_rows(kd, pos, out=dst, stream=stream)

        t, tk = graph_time(torch, stream, fn, steps, warmup, reps=3)
        safe = pos.long().clamp(0, key.shape[1] - 1)
        distinct = int(sum(torch.unique(safe[b]).numel() for b in range(B)))
        npos = B * R * case.k
        esz = key.element_size()
        psz = pos.element_size()
        alg = gather_algorithmic_bytes(npos, D, esz, psz, distinct)
        out_bytes = npos * D * esz
        out.append({
            "key": "contiguous" if key.is_contiguous() else "strided view",
            "us_per_call": t * 1e6,
            "kernel_us": tk * 1e6,
            "algorithmic_bytes": alg,
            "gbps": alg / t / 1e9,
            "pct_peak": 100.0 * alg / t / 1e9 / HBM_PEAK_GBPS,
            "output_convention_gbps": output_convention_gbps(out_bytes, t),
        })
        del dst, kd
    torch.cuda.empty_cache()
    return out


def cpu_baseline(case, budget_s: float = 10.0):
    """The oracle on the host cores, repeated over the same workload for ~budget_s."""
    import torch
    import oracle
    orc = oracle.Oracle()
    x = case.x
    xh = x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()
    it = np.int32 if str(case.indices_type).endswith("int32") else np.int64
    re = case.row_end.numpy() if case.row_end is not None else None
    threads = min(oracle.host_threads(), x.shape[0])
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.topk(xh, case.k, row_end=re, sorted_index=case.sorted_index, indices_type=it,
                 return_value=case.return_value, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": reps * x.shape[0] / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full passes of the {case.name} top-k ({x.shape[0]} rows x "
                      f"{x.shape[1]}) in {dt:.1f} s, {threads} threads"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg2")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the plain copy kernel the traffic counters are scaled by")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter files into profiles/traffic.json")
    args = ap.parse_args(argv)
    if args.traffic_from:
        print(json.dumps(traffic_from(*args.traffic_from)))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU (run with --gpus 1): the selection step shards by "
              "rows with no exchange, so N GPUs run N independent row slices", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import sparse_attention_indexer_dsel_amd as dsel

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    cfg_id = int(args.workload.replace("cfg", ""))
    case = W.make_config(cfg_id)
    if args.copy_calibration:
        copy_calibration(torch, stream)

    # ---- headline: K steps of the workload's top-k -------------------------
    tb = TopkBench(dsel, torch, case, stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            tb.call(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(args.steps):
            tb.call(i)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    # the timed region: one replay of the K steps, HIP events on the kernels'
    # stream inside the host clock
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_kern = e0.elapsed_time(e1) * 1e-3 / args.steps
    del g
    t_step = elapsed / args.steps
    nbytes = tb.algorithmic_bytes()
    rows = case.x.shape[0]
    achieved = nbytes / t_kern / 1e9
    traffic = load_traffic() if cfg_id == 2 else None
    del tb
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": rows / t_step,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.x.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded host generator; no datasets or weights)",
        "config": {"workload": f"{case.name}: top-k {rows}x{case.x.shape[1]} "
                               f"{'bf16' if case.x.dtype == torch.bfloat16 else 'fp32'}, "
                               f"k={case.k}, sorted_index={case.sorted_index}, "
                               f"{str(case.indices_type).split('.')[-1]} indices, "
                               f"values={case.return_value}",
                   "global_batch": rows, "seq_len": int(case.x.shape[1]), "parallelism": "none"},
        "gbps": nbytes / t_step / 1e9,
        "pct_peak": 100.0 * nbytes / t_step / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "kernel": traffic["kernel"] if traffic else "dsel_topk (one kernel per call)",
                     "kernel_us": t_kern * 1e6,
                     "algorithmic_bytes_per_launch": nbytes},
    }

    if not args.no_per_config:
        per = {}
        for i in sorted(W.CONFIGS):
            c = case if i == cfg_id else W.make_config(i)
            entry = {"topk": measure_topk(dsel, torch, c, stream, 20, 3)}
            if i in VALUE_ORDER_CONFIGS:
                entry["topk_by_value"] = measure_topk(dsel, torch, c, stream, 20, 3, by_value=True)
            if i in WITH_VALUES_CONFIGS and not c.return_value:
                entry["topk_with_values"] = measure_topk(
                    dsel, torch, dataclasses.replace(c, return_value=True), stream, 20, 3)
            if c.keys:
                entry["gather"] = measure_gather(dsel, torch, c, stream, 10, 2)
            per[c.name] = entry
            print(f"# {c.name}: {json.dumps(entry)}", file=sys.stderr, flush=True)
        line["per_config"] = per

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case)

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
