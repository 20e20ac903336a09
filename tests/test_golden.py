"""The pages' printed worked examples (tests/golden/deepselect_examples.txt)."""
import os

import numpy as np
import torch

import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepselect_examples.txt")


def load_golden():
    facts = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            facts[key] = val
    return facts


def test_basic_example_shapes(orc):
    f = load_golden()
    b, v, k = int(f["A.batch"]), int(f["A.vocab"]), int(f["A.topk"])
    x = torch.randn(b, v, generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    vals, idx, _ = orc.topk(P.to_host(x), k, sorted_index=True, indices_type=np.int32)
    assert vals.shape == tuple(int(s) for s in f["A.values_shape"].split(","))
    assert idx.shape == tuple(int(s) for s in f["A.indices_shape"].split(","))
    assert idx.dtype == np.int32 and vals.dtype == np.uint16
    assert (np.diff(idx, axis=1) > 0).all()


def test_variable_length_example(orc):
    f = load_golden()
    b, v, k = int(f["B.batch"]), int(f["B.vocab"]), int(f["B.topk"])
    end = np.array([int(s) for s in f["B.end"].split(",")], dtype=np.int32)
    x = torch.randn(b, v, generator=torch.Generator().manual_seed(12)).numpy()
    vals, idx, flag = orc.topk(x, k, row_end=end, sorted_index=True, indices_type=np.int64)
    assert idx.dtype == np.int64 and idx.shape == (b, k)
    assert (idx[1] < end[1]).all()
    assert (idx[0] >= end[1]).any()  # the full row does reach past the second row's end
    assert (np.diff(idx, axis=1) > 0).all()
    assert not flag.any()


def test_gather_bandwidth_convention():
    """The pages count gather GB/s as gathered (output) bytes over time."""
    import bench
    f = load_golden()
    out_bytes = int(f["C.rows"]) * int(f["C.positions"]) * int(f["C.head_dim"]) * int(f["C.elt_bytes"])
    gbps = bench.output_convention_gbps(out_bytes, float(f["C.ms"]) * 1e-3)
    assert abs(gbps - float(f["C.gbps_about"])) / float(f["C.gbps_about"]) < 0.01
