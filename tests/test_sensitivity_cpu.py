"""The inputs of the top-term parity tests (tests/sensitive_cases.py) must make the highest
Taylor term of their P visible: dropping it (the oracle at P-1 against the oracle at P) moves
y on the checked rows by at least 10 x the 2e-2 bar, so a GPU result with that term wrong or
missing cannot pass them.  The denominators must stay well away from zero, so the bar is
not met or missed by cancellation.  Oracle only, on the CPU."""
import numpy as np
import pytest

import oracle
import sensitive_cases as sc

TOL_BF16 = 2e-2
MIN_GAP = 10 * TOL_BF16
MIN_DEN = 0.15          # min over rows of D_T / T


def _gap(x, P, rows=slice(None)):
    y_lo = oracle.direct(x["q"], x["k"], x["v"], P - 1)
    y, den = oracle.direct(x["q"], x["k"], x["v"], P, return_den=True)
    n = x["q"].shape[-2]
    gap = float(np.max(oracle.row_rel_err(y_lo[..., rows, :], y[..., rows, :])))
    cond = float(np.min(den / np.arange(1, n + 1)))
    return gap, cond


@pytest.mark.parametrize("d,P,n,seed", sc.ONE_LEVEL)
def test_one_level_cases(d, P, n, seed):
    gap, cond = _gap(sc.draw(d, P, 1, 2, n, seed), P)
    assert gap >= MIN_GAP and cond >= MIN_DEN, (gap, cond)


@pytest.mark.parametrize("d,P,n,seed,nsub", sc.TWO_LEVEL)
def test_two_level_cases(d, P, n, seed, nsub):
    gap, cond = _gap(sc.draw(d, P, 1, 2, n, seed), P)
    assert gap >= MIN_GAP and cond >= MIN_DEN, (gap, cond)


@pytest.mark.parametrize("d,P,n1,n2,seed", sc.CONTINUE)
def test_continue_cases(d, P, n1, n2, seed):
    gap, cond = _gap(sc.draw(d, P, 1, 2, n1 + n2, seed), P, slice(n1, None))
    assert gap >= MIN_GAP and cond >= MIN_DEN, (gap, cond)


@pytest.mark.parametrize("d,P,n1,steps,seed,sigma", sc.DECODE)
def test_decode_cases(d, P, n1, steps, seed, sigma):
    gap, cond = _gap(sc.draw(d, P, 1, 2, n1 + steps, seed, sigma), P, slice(n1, None))
    assert gap >= MIN_GAP and cond >= MIN_DEN, (gap, cond)


def test_mid_shape_case():
    B, H, n, d, P, seed = sc.MID_SHAPE
    gap, cond = _gap(sc.draw(d, P, B, H, n, seed), P)
    assert gap >= MIN_GAP and cond >= MIN_DEN, (gap, cond)


def test_long_shape_case_on_its_sampled_rows():
    """The Long shape's test checks sampled rows; the top term must be visible on them."""
    B, H, n, d, P, seed = sc.LONG_SHAPE
    x = sc.draw(d, P, B, H, n, seed, sc.LONG_SIGMA)
    flat = {c: x[c].reshape(B * H, n, d) for c in ("q", "k", "v")}
    heads, rows = sc.long_rows(n, seed)
    y_lo = oracle.direct_rows(flat["q"], flat["k"], flat["v"], P - 1, heads, rows)
    y = oracle.direct_rows(flat["q"], flat["k"], flat["v"], P, heads, rows)
    gap = float(np.max(oracle.row_rel_err(y_lo, y)))
    assert gap >= MIN_GAP, gap


def test_workload_scales_are_insensitive():
    """Why these cases exist: at the benchmark workloads' own scale (q, k ~ N(0, 0.5^2),
    d = 64) dropping the cubic term moves y by well under 10 x the bar."""
    from constant_cost_self_amd import inputs
    x = inputs.draw((1, 2, 700, 64), (1, 2, 700, 64), "bf16", 0.5, 1.0, 72)
    gap, _ = _gap(x, 4)
    assert gap < MIN_GAP
