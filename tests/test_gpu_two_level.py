"""GPU parity of the two-level prefill (sub-segments of the sequence scanned in parallel
from prefix-summed starting states) against the fp64 oracle, and against the one-level
scan.  Bars as in test_gpu_parity: y within 2e-2 (bf16 inputs, fp32 state) as max over
rows of max_j |y - y_ref| / max_j |y_ref|; the final state per degree block and column (gpu_helpers.state_col_err)."""
import time

import numpy as np
import pytest

from gpu_helpers import (TOL_BF16, inputs, max_row_err, new_state, oracle, prefill, sample_feature_rows,
                         sampled_state_err, say, sata, state_col_err, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _draw(n, d, H, seed):
    return inputs.draw((1, H, n, d), (1, H, n, d), "bf16", 0.5, 1.0, seed)


@pytest.mark.parametrize("d,nsub,n", [(64, 2, 2000), (64, 3, 2000), (64, 5, 1234), (64, 8, 300),
                                      (128, 3, 700), (128, 2, 129)])
def test_two_level_matches_oracle(torch_cuda, d, nsub, n):
    """Forced sub-segments (ragged last chunk, a last sub-segment shorter than the others,
    more sub-segments asked for than the sequence has windows): y and the final state."""
    say("two-level d=%d nsub=%d n=%d" % (d, nsub, n))
    x = _draw(n, d, 2, 40 + nsub + d)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, 4)
    t.set_prefill_split(nsub)
    S = new_state(1, 2, d, d, 4)
    y = prefill(t, q, k, v, 64, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y.cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    M = oracle.feature_dim(d, 4)
    rows = sample_feature_rows(d, 4, 200, n)
    S_ref = oracle.state_rows(x["k"][0, 1], x["v"][0, 1], 4, rows)
    Sg = S[0, 1].cpu().numpy()
    serr = sampled_state_err(Sg, S_ref, rows, d, 4)
    say("  state err %.3e" % serr)
    assert serr <= TOL_BF16
    assert np.all(Sg[:, M:] == 0.0), "padding of the state must stay zero"
    t.close()


@pytest.mark.parametrize("P", [2, 3, 5])
def test_two_level_term_counts(torch_cuda, P):
    """Other term counts (another parent depth in the scan's operand building)."""
    n = 1100
    say("two-level d=64 P=%d nsub=3 n=%d" % (P, n))
    x = _draw(n, 64, 1, 80 + P)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(64, P)
    t.set_prefill_split(3)
    y = prefill(t, q, k, v, 64)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    err = max_row_err(y.cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    t.close()


def test_two_level_continue_from_state(torch_cuda):
    """The first sub-segment starts from the caller's state (prefix of 700 tokens)."""
    say("two-level prefill(700) + prefill(1300, continue, nsub=3)")
    n1, n2 = 700, 1300
    x = _draw(n1 + n2, 64, 1, 50)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(64, 4)
    S = new_state(1, 1, 64, 64, 4)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), 64, S)
    t.set_prefill_split(3)
    y2 = prefill(t, q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(),
                 64, S, continue_state=True)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y2.cpu().numpy(), ref[:, :, n1:])
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    _, S_ref = oracle.feature_form(None, x["k"][0, 0], x["v"][0, 0], 4, want_y=False)
    M = S_ref.shape[1]
    assert state_col_err(S[0, 0].cpu().numpy()[:, :M], S_ref, 64, 4) <= TOL_BF16
    t.close()


def test_two_level_equals_one_level(torch_cuda):
    """Same sums in another order: the two forms agree far inside the oracle bar."""
    say("two-level vs one-level, d=64 n=3000")
    n = 3000
    x = _draw(n, 64, 1, 60)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(64, 4)
    t.set_prefill_split(1)
    S1 = new_state(1, 1, 64, 64, 4)
    y1 = prefill(t, q, k, v, 64, S1)
    t.set_prefill_split(4)
    S2 = new_state(1, 1, 64, 64, 4)
    y2 = prefill(t, q, k, v, 64, S2)
    torch_cuda.cuda.synchronize()
    dy = max_row_err(y2.cpu().numpy(), y1.cpu().numpy().astype(np.float64))
    a, b = S1[0, 0].cpu().numpy().astype(np.float64), S2[0, 0].cpu().numpy()
    ds = state_col_err(b, a, 64, 4)
    say("  y diff %.3e state diff %.3e" % (dy, ds))
    assert dy <= 2e-3 and ds <= 1e-5
    t.close()


@pytest.mark.parametrize("n", [16384, 65536])
def test_two_level_automatic_long_single_head(torch_cuda, n):
    """One head leaves most compute units idle: the automatic choice takes the two-level form
    (n = 65536 is the benchmark's two-level workload, drawn as the benchmark draws it).
    Sampled rows of y and of the state against the oracle; the time of both forms is printed."""
    say("automatic two-level, B=H=1 n=%d d=64" % n)
    x = _draw(n, 64, 1, 70) if n != 65536 else inputs.draw((1, 1, n, 64), (1, 1, n, 64), "bf16", 0.5, 1.0, 0)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(64, 4)
    S = new_state(1, 1, 64, 64, 4)
    times = {}
    for split in (1, 0):
        t.set_prefill_split(split)
        prefill(t, q, k, v, 64, S)                     # warm-up
        torch_cuda.cuda.synchronize()
        t0 = time.perf_counter()
        y = prefill(t, q, k, v, 64, S)
        torch_cuda.cuda.synchronize()
        times[split] = (time.perf_counter() - t0) * 1e3
    say("  one-level %.2f ms, automatic %.2f ms" % (times[1], times[0]))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, 8191, 8192, n // 2 - 1, n // 2, n - 1],
                                     np.random.default_rng(1).choice(n, 40, replace=False)]))
    ref = oracle.direct_rows(x["q"], x["k"], x["v"], 4, np.zeros_like(rows), rows)
    err = max_row_err(y[0, 0].cpu().numpy()[rows], ref)
    say("  sampled y err %.3e" % err)
    assert err <= TOL_BF16
    M = oracle.feature_dim(64, 4)
    frows = sample_feature_rows(64, 4, 100, 2)
    S_ref = oracle.state_rows(x["k"][0, 0], x["v"][0, 0], 4, frows)
    serr = sampled_state_err(S[0, 0].cpu().numpy(), S_ref, frows, 64, 4)
    say("  sampled state err %.3e" % serr)
    assert serr <= TOL_BF16
    t.close()


def test_two_level_falls_back_under_a_small_workspace_cap(torch_cuda):
    """The two-level form needs the whole sequence's partials: under a small cap the one-level
    scan runs in segments instead, with the same results."""
    n = 2000
    say("two-level asked for under an 8 MiB workspace cap, n=%d" % n)
    x = _draw(n, 64, 1, 90)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(64, 4)
    t.set_prefill_split(4)
    t.set_workspace_limit(8 << 20)
    S = new_state(1, 1, 64, 64, 4)
    y = prefill(t, q, k, v, 64, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y.cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    _, S_ref = oracle.feature_form(None, x["k"][0, 0], x["v"][0, 0], 4, want_y=False)
    M = S_ref.shape[1]
    assert state_col_err(S[0, 0].cpu().numpy()[:, :M], S_ref, 64, 4) <= TOL_BF16
    t.close()


@pytest.mark.parametrize("case", range(8))
def test_two_level_sweep_against_one_level(torch_cuda, case):
    """Seeded awkward shapes (sequence lengths around window boundaries, sub-segment counts
    that do not divide the windows): the two forms agree on y and the final state."""
    rng = np.random.default_rng(1000 + case)
    d = int(rng.choice([64, 128]))
    win = 4 if d == 64 else 2
    n = int(64 * win * rng.integers(2, 9) + rng.integers(-70, 70))
    nsub = int(rng.integers(2, 7))
    say("two-level sweep: d=%d n=%d nsub=%d" % (d, n, nsub))
    x = _draw(n, d, 1, 2000 + case)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, 4)
    out = []
    for split in (1, nsub):
        t.set_prefill_split(split)
        S = new_state(1, 1, d, d, 4)
        y = prefill(t, q, k, v, 64, S)
        torch_cuda.cuda.synchronize()
        out.append((y[0, 0].cpu().numpy().astype(np.float64), S[0, 0].cpu().numpy().astype(np.float64)))
    t.close()
    dy = max_row_err(out[1][0], out[0][0])
    ds = state_col_err(out[1][1], out[0][1], d, 4)
    say("  y diff %.3e state diff %.3e" % (dy, ds))
    assert np.all(np.isfinite(out[1][0]))
    assert dy <= 2e-3 and ds <= 1e-5
