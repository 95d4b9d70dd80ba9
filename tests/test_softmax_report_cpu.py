"""The Taylor-versus-exact-softmax report (oracle only, CPU).  The pages say the P = 4
truncation is close to float16 resolution but give no metric, so this is reported, not a
parity bar: per-row max_j |y_P - y_softmax| / max_j |y_softmax| on one head of each
workload recipe (bench.py prints the same report at full length).  What is asserted is
what the mathematics fixes: the error falls with every added term, it is smaller at the
smaller input scale of the wide heads, and at P = 4 it sits near fp16 resolution (2^-10)
in the median at the Mid/Long scale."""
import numpy as np
import pytest

import oracle
from constant_cost_self_amd import inputs


@pytest.mark.parametrize("w", [inputs.MID, inputs.WIDE], ids=lambda w: w.name)
def test_report(w):
    n = 1024
    x = inputs.prefill_inputs(w, n=n, B=1, H=1)
    q, k, v = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0]
    ys = oracle.softmax(q, k, v)
    med, mx = [], []
    for P in range(1, 6):
        e = oracle.row_rel_err(oracle.direct(q, k, v, P), ys)
        med.append(float(np.median(e)))
        mx.append(float(np.max(e)))
        print("%s P=%d: max %.2e median %.2e" % (w.name, P, mx[-1], med[-1]))
    assert all(b < a for a, b in zip(med, med[1:])), med
    assert all(b < a for a, b in zip(mx, mx[1:])), mx
    if w is inputs.MID:
        assert 2 ** -12 < med[3] < 2 ** -8
    else:
        assert med[3] < 2 ** -12
