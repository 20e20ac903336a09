"""Benchmark of the selection step (row-wise top-k, then key gather) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg4]
                    [--no-per-config] [--no-cpu-baseline] [--no-floors] [--no-cold]
    python bench.py --profile-run cfgN      # a few calls of one workload, for counter runs
    python bench.py --traffic-from DIR      # no GPU: counter files -> profiles/traffic.json

Prints ONE JSON line.  The headline workload is the sampling top-k (128 x
129280 fp32, k = 4096, int64 indices plus values): the largest top-k of the
five named workloads, the one whose HBM roofline a single call can reach (the
4 x 8192 and 4 x 204800 top-k move 0.07 and 1.7 MB, below what any launch
can stream in its floor time).  A step is one top-k call over the whole
batch.  ``per_config`` carries the same measurement, with its own roofline
block, for all five workloads (top-k and, where they have one, the gather),
plus the top-k with the selection ordered by value for the 4 x 204800 and
sampling rows and the causal prefill rows with values returned.

Timing protocol
  * inputs are generated on the host from fixed seeds and copied to HBM
    before timing; each step reads a different copy of the input, and the
    copies together exceed twice the 256 MB Infinity Cache, so top-k reads
    come from HBM rather than from cache (warm, back-to-back throughput);
  * the K timed steps are captured once in a HIP graph and replayed, so the
    timed region holds no Python launch overhead; the region is bracketed
    by torch.cuda.synchronize() on both sides and wall-clock timed;
  * a HIP event pair on the kernels' stream brackets the same replay: each
    step is one top-k kernel (two with value order), so events / K is that
    kernel's mean duration back to back (the roofline figure), comparable
    with rocprofv3's kernel trace;
  * ``floors`` gives the launch floor (a graph of empty-work kernels, per
    launch), streaming read, write and copy rates of plain device kernels
    over 1 GiB, and the library's read floor (``dsel_read_floor``: one
    launch reading with the select's own loads) over 1 GiB and at the
    headline input's size, for scale;
  * each workload's top-k and gathers are also timed cold (``cold``): 10
    warm-up calls, then 100 single eager calls, each after 1 GiB is written
    on the call's stream (four times the Infinity Cache), with an event
    pair around the call alone; the median (and p10, p90) is reported.
    It includes the launch latency that graph replay hides.

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
  Two rocprofv3 counter runs per workload of ``--profile-run cfgN`` give
  FETCH_SIZE and WRITE_SIZE per dispatch for its top-k and gather kernels
  and for a plain streaming copy of known size (torch.neg, 256 MiB in,
  256 MiB out).  ``--traffic-from`` turns them into bytes per launch
  (counter value x known copy bytes / copy counter value) and stores them
  in profiles/traffic.json with a hash of the kernel sources; the bench
  reports them only while that hash still matches, and null otherwise.

CPU baseline
  The oracle (plain C, one row at a time) timed on the host's cores for
  every workload's top-k, once with a thread per core (rows split over the
  threads) and once on one thread, and on the gathers; each leg runs a
  bounded number of repetitions.  ``cores`` is the host's core count; each
  entry states the threads it used.
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
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
                  for f in ("topk.hip", "gather.hip", "dsel_internal.h", "api.hip")]
METRIC = "top-k rows/s and achieved HBM GB/s (% of peak) per config; gather GB/s"
HEADLINE = 4
# workloads also timed with the selection ordered by value (the sampling
# workload, where that order is the natural one, and the 4 x 204800 rows)
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


def roofline(alg_bytes: int, kernel_s: float, kernel: str, traffic=None) -> dict:
    achieved = alg_bytes / kernel_s / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "kernel": kernel,
            "kernel_us": kernel_s * 1e6, "algorithmic_bytes_per_launch": alg_bytes}


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


def _find_csv(d: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return hits[0]


def traffic_from(root: str, out_path: str = TRAFFIC_JSON) -> dict:
    """Per-launch HBM bytes of each workload's top-k and gather kernels from
    counter runs under `root` (fetch_cfgN/ and write_cfgN/ directories, one
    --profile-run each), scaled by the copy kernel's reading of the same
    counters (counter x known bytes / copy counter)."""
    rec = {"source_hash": kernel_source_hash(), "copy_bytes": COPY_CAL_BYTES, "configs": {}}
    specs = [f"cfg{c}" for c in range(1, 6)] + [f"cfg{c}v" for c in VALUE_ORDER_CONFIGS]
    for spec in specs:
        fd, wd = os.path.join(root, f"fetch_{spec}"), os.path.join(root, f"write_{spec}")
        if not (os.path.isdir(fd) and os.path.isdir(wd)):
            continue
        fetch = _counter_means(_find_csv(fd), "FETCH_SIZE")
        write = _counter_means(_find_csv(wd), "WRITE_SIZE")

        def pick(table, pat):
            names = [n for n in table if pat in n]
            return max(names, key=lambda n: table[n][1]) if names else None

        cf, cw = pick(fetch, "neg"), pick(write, "neg")
        if cf is None or cw is None:
            raise SystemExit(f"no copy-calibration kernel in the {spec} counter files")
        f_fac, w_fac = COPY_CAL_BYTES / fetch[cf][0], COPY_CAL_BYTES / write[cw][0]
        entry = rec["configs"].setdefault(spec.rstrip("v"), {})
        entry["fetch_factor" + ("_by_value_run" if spec.endswith("v") else "")] = f_fac
        entry["write_factor" + ("_by_value_run" if spec.endswith("v") else "")] = w_fac
        roles = (("value_order", "sort_rows_by_value"),) if spec.endswith("v") else \
            (("topk", "topk_rows"), ("gather", "gather_rows"))
        for role, pat in roles:
            kf, kw = pick(fetch, pat), pick(write, pat)
            if kf is None or kw is None:
                continue
            fb, wb = fetch[kf][0] * f_fac, write[kw][0] * w_fac
            entry[role] = {"kernel": kf, "fetch_bytes": fb, "write_bytes": wb,
                           "traffic_bytes": fb + wb, "dispatches": [fetch[kf][1], write[kw][1]]}
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


def traffic_for(traffic, cfg_name: str, role: str):
    if not traffic:
        return None
    e = traffic.get("configs", {}).get(cfg_name, {}).get(role)
    return e["traffic_bytes"] if e else None


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
    """Capture `steps` calls of fn(i) in one HIP graph and replay it; return
    (wall seconds per call, event seconds per call).  The event pair brackets
    the replay on the stream the kernels run on, so the second figure is the
    kernels' mean duration back to back."""
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


COLD_FLUSH_BYTES = 1 << 30  # written before each cold call: four times the Infinity Cache
_FLUSH = []


def cold_time(torch, stream, fn, reps: int = 100, warmup: int = 10) -> dict:
    """Cold-cache timing: before each call a 1 GiB buffer is written on the
    call's stream (evicting L2 and the Infinity Cache), and a HIP event pair
    brackets the call alone (eager launch, so the launch latency is in).
    `warmup` untimed calls first; the median of `reps` calls is reported."""
    if not _FLUSH:
        _FLUSH.append(torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device="cuda"))
    flush = _FLUSH[0]
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    with torch.cuda.stream(stream):
        for i, (e0, e1) in enumerate(evs):
            flush.fill_(i & 0xFF)
            e0.record(stream)
            fn(i)
            e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    return {"median_us": float(np.median(t)), "p10_us": t[len(t) // 10],
            "p90_us": t[(9 * len(t)) // 10], "reps": reps, "warmup": warmup,
            "how": "1 GiB written on the stream before each call; events around the call only"}


def topk_kernel_name(case, by_value=False) -> str:
    return "dsel_topk" + (" + value order" if by_value else "") + f" ({case.name})"


def measure_topk(dsel, torch, case, stream, steps, warmup, by_value=False, traffic=None,
                 cold=False):
    """One top-k call per step (with by_value, the select and then the
    value-order pass: kernel_us covers both).  cold: also the cold-cache
    median of 100 single calls."""
    tb = TopkBench(dsel, torch, case, stream, by_value)
    steps = min(max(steps, tb.ncopy), 256)  # every input copy read once per replay
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
        "steps": steps,
        "roofline": roofline(nbytes, t_kern, topk_kernel_name(case, by_value), traffic),
    }
    if cold:
        res["cold"] = cold_time(torch, stream, tb.call)
        res["cold"]["pct_peak"] = 100.0 * nbytes / (res["cold"]["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS
    del tb
    torch.cuda.empty_cache()
    return res


def measure_gather(dsel, torch, case, stream, steps, warmup, traffic=None, cold=True):
    """Gather(s) of the case's keys at the top-k positions (one call per key)."""
    dev = torch.device("cuda")
    _, idx, _ = dsel.topk(case.x.to(dev), case.k,
                          end=case.row_end.to(dev) if case.row_end is not None else None,
                          indices_type=case.indices_type, return_value=False)
    B = case.gather_batch
    R = case.x.shape[0] // B
    pos = idx.contiguous().view(B, R, case.k)
    out = []
    for key in case.keys:
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
        cold_t = None
        if cold:
            cold_t = cold_time(torch, stream, fn)
            cold_t["pct_peak"] = 100.0 * alg / (cold_t["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS
        out.append({
            "key": "contiguous" if key.is_contiguous() else "strided view",
            "us_per_call": t * 1e6,
            "kernel_us": tk * 1e6,
            "algorithmic_bytes": alg,
            "gbps": alg / t / 1e9,
            "pct_peak": 100.0 * alg / t / 1e9 / HBM_PEAK_GBPS,
            "output_convention_gbps": output_convention_gbps(out_bytes, t),
            "roofline": roofline(alg, tk, f"dsel_gather_rows ({case.name})", traffic),
        })
        if cold_t is not None:
            out[-1]["cold"] = cold_t
        del dst, kd
    torch.cuda.empty_cache()
    return out


def _event_time(torch, stream, fn, reps: int = 5) -> float:
    """Best event-timed duration of fn() on `stream`, seconds (eager)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        fn()
    stream.synchronize()
    best = None
    for _ in range(reps):
        with torch.cuda.stream(stream):
            e0.record(stream)
            fn()
            e1.record(stream)
        stream.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    return best


def measure_fused(dsel, torch, case, stream, steps, warmup) -> dict:
    """The top-k and the gather of the workload's keys as one call
    (dsel_topk_gather) against the two-call chain (the top-k, then one
    gather launch per key), outputs reused across steps, inputs rotated."""
    tb = TopkBench(dsel, torch, case, stream)
    dev = torch.device("cuda")
    rows = case.x.shape[0]
    B = case.gather_batch
    R = rows // B
    keys = [k.to(dev) for k in case.keys]
    idx = torch.empty(rows, -(-case.k // 4) * 4, dtype=case.indices_type, device=dev)
    outs = [torch.empty(rows, case.k, k.shape[2], dtype=k.dtype, device=dev) for k in keys]
    gouts = [o.view(B, R, case.k, -1) for o in outs]

    def fused(i):
        dsel.topk_gather(tb.xs[i % tb.ncopy], case.k, keys, rows_per_batch=R, end=tb.row_end,
                         indices_type=case.indices_type, stream=stream, out=outs, output_idx=idx)

    def chain(i):
        dsel.topk(tb.xs[i % tb.ncopy], case.k, end=tb.row_end, indices_type=case.indices_type,
                  return_value=False, stream=stream, output_idx=idx)
        pos = idx[:, :case.k].view(B, R, case.k)
        for k, o in zip(keys, gouts):
            dsel.gather_rows(k, pos, out=o, stream=stream)

    steps = min(max(steps, 2), 32)
    t_f, k_f = graph_time(torch, stream, fused, steps, warmup, reps=3)
    t_c, k_c = graph_time(torch, stream, chain, steps, warmup, reps=3)
    n = _valid_lengths(case)
    isz = 4 if case.indices_type == torch.int32 else 8
    read = int(np.where(n > case.k, n, 0).sum()) * case.x.element_size() + 4 * rows
    written = rows * case.k * isz + rows
    # gathered rows written, and each key row the positions can reach read
    # once (rows below the longest valid length, per batch)
    gbytes = sum(rows * case.k * k.shape[2] * k.element_size() for k in case.keys)
    gbytes += sum(int(min(k.shape[1], n.max())) * k.shape[2] * k.element_size() * B
                  for k in case.keys)
    alg = read + written + gbytes
    res = {"fused_us": t_f * 1e6, "fused_kernel_us": k_f * 1e6,
           "chain_us": t_c * 1e6, "chain_kernels_us": k_c * 1e6,
           "fused_vs_chain": t_c / t_f,
           "algorithmic_bytes": alg,
           "roofline": roofline(alg, k_f, f"dsel_topk_gather ({case.name})"),
           "how": "one dsel_topk_gather call (select and gather in the select's kernel) "
                  "against dsel_topk then one dsel_gather_rows per key, same outputs, "
                  "graph replay, inputs rotated"}
    del tb, keys, outs, idx
    torch.cuda.empty_cache()
    return res


def measure_floors(torch, stream, dsel=None, head_bytes: int = 0) -> dict:
    """Launch floor and plain streaming rates of device kernels over 1 GiB
    (torch's own kernels: a reduction for read, a fill for write, a copy),
    and the library's read floor (dsel_read_floor: the select's own load
    form) at the headline input size and at 1 GiB."""
    dev = torch.device("cuda")
    tiny = torch.zeros(1, device=dev)
    _, launch = graph_time(torch, stream, lambda i: tiny.add_(1.0), 200, 5, reps=3)
    n = (1 << 30) // 2
    a = torch.ones(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    acc = torch.zeros((), dtype=torch.float32, device=dev)
    t_read = _event_time(torch, stream, lambda: torch.sum(a, 0, dtype=torch.float32, out=acc))
    t_write = _event_time(torch, stream, lambda: b.fill_(1.0))
    h = n // 2
    t_copy = _event_time(torch, stream, lambda: b[:h].copy_(a[h:]))
    res = {"launch_us": launch * 1e6,
           "read_gbps": (1 << 30) / t_read / 1e9,
           "write_gbps": (1 << 30) / t_write / 1e9,
           "copy_gbps": (1 << 30) / t_copy / 1e9,  # 512 MiB read + 512 MiB written
           "how": "launch: a graph of 200 one-element adds, event time per launch; "
                  "read 1 GiB (torch.sum), write 1 GiB (fill_), copy 512 MiB -> 512 MiB, "
                  "best of 5 event-timed eager calls"}
    if dsel is not None:
        words = torch.empty(-(-(1 << 30) // 65536), dtype=torch.int32, device=dev)
        t_big = _event_time(torch, stream, lambda: dsel.read_floor(a, out=words, stream=stream))
        res["read_floor_1gib_gbps"] = (1 << 30) / t_big / 1e9
        if head_bytes >= 16:
            hb = head_bytes // 16 * 16
            ncopy = max(2, -(-(512 << 20) // hb))  # past twice the Infinity Cache
            copies = [torch.ones(hb // 4, dtype=torch.int32, device=dev) for _ in range(ncopy)]
            _, t_head = graph_time(torch, stream,
                                   lambda i: dsel.read_floor(copies[i % ncopy], out=words, stream=stream),
                                   max(64, ncopy), 5, reps=3)
            res["read_floor_headline"] = {"bytes": hb, "us": t_head * 1e6, "gbps": hb / t_head / 1e9}
            del copies
        res["how_read_floor"] = ("dsel_read_floor: one launch reading the buffer once with the "
                                 "select's loads (16-byte, non-temporal hint, 16 per thread); 1 GiB "
                                 "best of 5 eager calls, the headline input's size back to back in a "
                                 "graph over rotating copies")
        del words
    del a, b
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline (the oracle)
# ---------------------------------------------------------------------------

def _host_x(case):
    import torch
    x = case.x
    return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()


def _time_reps(fn, budget_s: float, max_reps: int):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= max_reps:
            return reps, dt


def cpu_baseline(cases, headline, budget_s: float = 2.0) -> dict:
    """The oracle on the host cores: every workload's top-k with a thread per
    core and with one thread, and the gathers."""
    import torch
    import oracle
    orc = oracle.Oracle()
    cores = oracle.host_threads()
    per = {}
    for c in cases:
        xh = _host_x(c)
        it = np.int32 if c.indices_type == torch.int32 else np.int64
        re = c.row_end.numpy() if c.row_end is not None else None
        rows = c.x.shape[0]
        entry = {}
        for label, threads in (("all_cores", min(cores, rows)), ("one_thread", 1)):
            def run(threads=threads):
                orc.topk(xh, c.k, row_end=re, sorted_index=c.sorted_index, indices_type=it,
                         return_value=c.return_value, threads=threads)
            reps, dt = _time_reps(run, budget_s, 1000)
            entry[label] = {"rows_per_s": reps * rows / dt, "s_per_call": dt / reps,
                            "threads": threads, "calls": reps}
        if c.keys:
            _, idx, _ = orc.topk(xh, c.k, row_end=re, sorted_index=c.sorted_index,
                                 indices_type=it, return_value=False)
            B = c.gather_batch
            pos = idx.reshape(B, rows // B, c.k)
            g = []
            for key in c.keys:
                kh = key.view(torch.int16).numpy().view(np.uint16)
                reps, dt = _time_reps(lambda kh=kh: orc.gather(kh, pos), budget_s, 100)
                out_bytes = pos.size * key.shape[2] * key.element_size()
                g.append({"key": "contiguous" if key.is_contiguous() else "strided view",
                          "s_per_call": dt / reps, "output_convention_gbps": out_bytes * reps / dt / 1e9,
                          "threads": 1, "calls": reps})
            entry["gather"] = g
        per[c.name] = entry
    h = per[headline.name]["all_cores"]
    return {"value": h["rows_per_s"], "unit": "rows/s", "cores": cores, "kind": "oracle",
            "threads": h["threads"],
            "sample": f"{h['calls']} full calls of the {headline.name} top-k "
                      f"({headline.x.shape[0]} rows x {headline.x.shape[1]}) on {h['threads']} "
                      f"threads (rows split over threads; the host has {cores} cores); every "
                      f"workload on all cores and on one thread, and the gathers, in per_config",
            "per_config": per}


# ---------------------------------------------------------------------------

def profile_run(spec: str) -> int:
    """A few calls of one workload's top-k and gathers, plus the counter
    calibration copy: the program the counter runs profile.  ``cfgN`` runs
    the workload as named; ``cfgNv`` runs its top-k ordered by value (the
    select, then the value-order pass) and no gather."""
    import torch
    import workloads as W
    import sparse_attention_indexer_dsel_amd as dsel
    by_value = spec.endswith("v")
    cfg_id = int(spec.replace("cfg", "").rstrip("v"))
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    copy_calibration(torch, stream)
    case = W.make_config(cfg_id)
    dev = torch.device("cuda")
    x = case.x.to(dev)
    re = case.row_end.to(dev) if case.row_end is not None else None
    with torch.cuda.stream(stream):
        for _ in range(3):
            _, idx, _ = dsel.topk(x, case.k, end=re, sorted_index=case.sorted_index,
                                  indices_type=case.indices_type, return_value=case.return_value,
                                  by_value=by_value, stream=stream)
        if case.keys and not by_value:
            B = case.gather_batch
            pos = idx.contiguous().view(B, case.x.shape[0] // B, case.k)
            for key in case.keys:
                kd = key.to(dev)
                for _ in range(3):
                    dsel.gather_rows(kd, pos, stream=stream)
    stream.synchronize()
    print(f"profile run of {case.name}{' by value' if by_value else ''} done", flush=True)
    return 0


# One SQ counter pass (8 SQ counters and GRBM_GUI_ACTIVE, the most one run
# can hold): instruction counts, and rocprofv3's derived occupancy, LDS
# bank-conflict and VALU-busy figures for gfx950 (their inputs are
# SQ_WAVE_CYCLES, SQ_LDS_BANK_CONFLICT, SQ_ACTIVE_INST_VALU and
# GRBM_GUI_ACTIVE).
SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_LDS "
               "SQ_LDS_BANK_CONFLICT OccupancyPercent LDSBankConflict VALUBusy")


def counters_from(d: str) -> str:
    """Markdown table of per-dispatch means per library kernel from one
    rocprofv3 run with SQ_COUNTERS, plus bank-conflict cycles per LDS
    instruction cycle."""
    path = _find_csv(d)
    names = SQ_COUNTERS.split()
    table = {}
    for c in names:
        for kern, (mean, cnt) in _counter_means(path, c).items():
            table.setdefault(kern, {})[c] = (mean, cnt)
    lines = ["| kernel | dispatches | " + " | ".join(names) + " | conflict cycles / LDS cycles |",
             "|---" * (len(names) + 3) + "|"]
    for kern, row in sorted(table.items()):
        if not any(p in kern for p in ("dsel", "topk", "gather", "sort_rows")):
            continue
        get = lambda c: row.get(c, (float("nan"), 0))[0]
        lds = get("SQ_ACTIVE_INST_LDS")
        ratio = get("SQ_LDS_BANK_CONFLICT") / lds if lds else float("nan")
        short = kern.split("(dsel::")[0].replace("dsel::", "").replace("(anonymous namespace)::", "")
        lines.append(f"| `{short}` | {max(v[1] for v in row.values())} | " +
                     " | ".join(f"{get(c):.4g}" for c in names) + f" | {ratio:.3f} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=f"cfg{HEADLINE}")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floors", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache single calls (kernel traces of the warm replay)")
    ap.add_argument("--profile-run", metavar="CFG",
                    help="a few calls of one workload (cfgN, or cfgNv ordered by value) for counter runs")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="no GPU: per-kernel table of an SQ counter run")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="no GPU: turn per-workload counter runs into profiles/traffic.json")
    args = ap.parse_args(argv)
    if args.traffic_from:
        print(json.dumps(traffic_from(args.traffic_from)))
        return 0
    if args.counters_from:
        print(counters_from(args.counters_from))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU (run with --gpus 1): the selection step shards by "
              "rows with no exchange, so N GPUs run N independent row slices", file=sys.stderr)
        return 2
    if args.profile_run:
        return profile_run(args.profile_run)

    import torch
    import workloads as W
    import sparse_attention_indexer_dsel_amd as dsel

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    cfg_id = int(args.workload.replace("cfg", ""))
    case = W.make_config(cfg_id)
    traffic = load_traffic()

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
    dt_name = "bf16" if case.x.dtype == torch.bfloat16 else "f32"
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
        "dtype": dt_name,
        "data": "synthetic (seeded host generator; no datasets or weights)",
        "config": {"workload": f"{case.name}: top-k {rows}x{case.x.shape[1]} {dt_name}, "
                               f"k={case.k}, sorted_index={case.sorted_index}, "
                               f"{str(case.indices_type).split('.')[-1]} indices, "
                               f"values={case.return_value}",
                   "global_batch": rows, "seq_len": int(case.x.shape[1]), "parallelism": "none"},
        "gbps": nbytes / t_step / 1e9,
        "pct_peak": 100.0 * nbytes / t_step / 1e9 / HBM_PEAK_GBPS,
        "roofline": roofline(nbytes, t_kern, topk_kernel_name(case),
                             traffic_for(traffic, case.name, "topk")),
        "timing": "warm back-to-back graph replay over rotating input copies (> 2x the "
                  "Infinity Cache), events on the kernels' stream; per_config entries also "
                  "carry a cold-cache median of 100 single calls ('cold')",
    }

    cases = [case if i == cfg_id else W.make_config(i) for i in sorted(W.CONFIGS)]
    if not args.no_floors:
        line["floors"] = measure_floors(torch, stream, dsel,
                                        case.x.numel() * case.x.element_size())
        print(f"# floors: {json.dumps(line['floors'])}", file=sys.stderr, flush=True)
    if not args.no_per_config:
        per = {}
        for c in cases:
            entry = {"topk": measure_topk(dsel, torch, c, stream, 20, 3,
                                          traffic=traffic_for(traffic, c.name, "topk"),
                                          cold=not args.no_cold)}
            if c.x.shape[0] and c.name == case.name:
                entry["topk"]["headline"] = True
            if int(c.name[3:]) in VALUE_ORDER_CONFIGS:
                entry["topk_by_value"] = measure_topk(dsel, torch, c, stream, 20, 3, by_value=True)
            if int(c.name[3:]) in WITH_VALUES_CONFIGS and not c.return_value:
                entry["topk_with_values"] = measure_topk(
                    dsel, torch, dataclasses.replace(c, return_value=True), stream, 20, 3)
            if c.keys:
                entry["gather"] = measure_gather(dsel, torch, c, stream, 10, 2,
                                                 traffic=traffic_for(traffic, c.name, "gather"),
                                                 cold=not args.no_cold)
                entry["topk_gather"] = measure_fused(dsel, torch, c, stream, 10, 2)
            per[c.name] = entry
            print(f"# {c.name}: {json.dumps(entry)}", file=sys.stderr, flush=True)
        line["per_config"] = per

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cases, case)

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
