"""The CPU oracle against checks that do not come from the oracle itself."""
import numpy as np
import pytest
import torch

import oracle_pins as P
import workloads


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_prefill_workload_totals(orc):
    """Closed forms for the 4096 x 2048 causal prefill workload (k = 1024).

    row_end[i] = (i+1)//2, so min(k, n_i) summed over rows is 3,145,728, the
    padding count is 4096*1024 - 3,145,728 = 2**20, and exactly the 2047 rows
    with n_i > 1024 are eligible for the NaN flag.
    """
    case = workloads.config3()
    x = P.to_host(case.x)
    re = case.row_end.numpy()
    _, idx, flag = orc.topk(x, case.k, row_end=re, sorted_index=False, return_value=False)
    assert int((idx != -1).sum()) == 3_145_728
    assert int((idx == -1).sum()) == 1 << 20
    n = np.clip(re.astype(np.int64), 0, x.shape[1])
    assert int((n > case.k).sum()) == 2047
    vals = P.decode(x)
    want = np.array([int(n[i] > case.k and np.isnan(vals[i, :n[i]]).any()) for i in range(x.shape[0])])
    assert np.array_equal(flag, want)
    assert 0 < int(flag.sum()) < 41  # some seeded NaN rows are short or out of range


def test_oracle_rejects_bad_k(orc):
    x = np.zeros((2, 8), dtype=np.float32)
    for k in (0, 4097):
        with pytest.raises(RuntimeError):
            orc.topk(x, k)


def test_oracle_empty_rows(orc):
    x = np.zeros((0, 8), dtype=np.float32)
    v, idx, flag = orc.topk(x, 4)
    assert idx.shape == (0, 4) and flag.shape == (0,)
