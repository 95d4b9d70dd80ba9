"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one sata_prefill over all heads, chunk 64, default workspace;
sata_decode_step over all sequences and heads).

The oracle cannot redo a whole workload, so each test checks what it can compute
one by one: full outputs of one head over a prefix, sampled output rows across
heads and positions (oracle.direct_rows, O(T (d_K + d_V)) each), and sampled rows
of final states (oracle.state_rows).  Bars as in the small parity tests: y within
2e-2 per row normalised by max_j |y_ref| (bf16 inputs, fp32 state); states within
2e-2 per degree block and column, normalised by the largest sampled |S_ref| of that
degree's rows in the column.
"""
import numpy as np
import pytest

from gpu_helpers import (TOL_BF16, inputs, max_row_err, oracle, sample_feature_rows,
                         sampled_state_err, sata, say, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _sample_positions(n, count, seed, lo=0):
    rng = np.random.default_rng(seed)
    fixed = [lo, n - 1, (lo + n) // 2]
    return np.unique(np.concatenate([fixed, rng.integers(lo, n, size=count)]))


def _check_rows(y_gpu_flat, x, P, heads, rows, label):
    """y_gpu_flat: [heads, n, d_V] on the host; compares the listed (head, row)."""
    ref = oracle.direct_rows(x["q"], x["k"], x["v"], P, heads, rows)
    got = y_gpu_flat[heads, rows].astype(np.float64)
    err = max_row_err(got, ref)
    say("  %s: %d sampled rows, y err %.3e" % (label, len(rows), err))
    assert err <= TOL_BF16


def _full_prefill(torch, w, with_state=True):
    say("%s: generating inputs B=%d H=%d n=%d d_K=%d d_V=%d" % (w.name, w.B, w.H, w.n, w.d_K, w.d_V))
    x = inputs.prefill_inputs(w)
    q, k, v = upload(x, w.dtype)
    t = sata.sata_tables_build(w.d_K, w.P)
    Mp = sata.sata_state_stride(w.d_K, w.P)
    S = (torch.zeros((w.B, w.H, w.d_V + 1, Mp), device="cuda:0", dtype=torch.float32)
         if with_state else None)
    y = torch.full((w.B, w.H, w.n, w.d_V), float("nan"), device="cuda:0", dtype=torch.float32)
    say("%s: prefill" % w.name)
    sata.sata_prefill(t, q, k, v, y, S, chunk=w.chunk)
    torch.cuda.synchronize()
    return x, t, S, y


def test_long_prefill_full_size(torch_cuda):
    """B=4, H=16, n=65536, d=64, P=4: head (0, 0) over its first 4096 tokens in
    full, sampled rows of every batch row and head, sampled final-state rows."""
    w = inputs.LONG
    x, t, S, y = _full_prefill(torch_cuda, w)
    yh = y.cpu().numpy()
    assert not np.isnan(yh).any()
    ref = oracle.direct(x["q"][0, 0, :4096], x["k"][0, 0, :4096], x["v"][0, 0, :4096], w.P)
    err = max_row_err(yh[0, 0, :4096], ref)
    say("  head (0,0) first 4096 tokens: y err %.3e" % err)
    assert err <= TOL_BF16
    flat = {s: x[s].reshape(w.B * w.H, w.n, -1) for s in ("q", "k", "v")}
    heads = np.arange(w.B * w.H)
    pos = _sample_positions(w.n, 2, 5, lo=4096)
    hs = np.repeat(heads, pos.size)
    ts = np.tile(pos, heads.size)
    _check_rows(yh.reshape(w.B * w.H, w.n, w.d_V), flat, w.P, hs, ts, "long, all heads")
    for (b, h), seed in (((0, 0), 1), ((3, 15), 2)):
        M = oracle.feature_dim(w.d_K, w.P)
        rows = sample_feature_rows(w.d_K, w.P, 80, seed)
        ref_rows = oracle.state_rows(x["k"][b, h], x["v"][b, h], w.P, rows)
        Sg = S[b, h].cpu().numpy()
        err = sampled_state_err(Sg, ref_rows, rows, w.d_K, w.P)
        say("  final state (%d,%d): err %.3e on %d rows" % (b, h, err, rows.size))
        assert err <= TOL_BF16
        assert Sg[w.d_V, 0] == w.n
        assert np.all(Sg[:, M:] == 0.0)
    t.close()


def test_decode_full_size(torch_cuda):
    """16 sequences x 32 heads, d=64, P=4: prefill 1024 tokens, then the decode
    steps over all sequences and heads; sampled heads checked at every step and
    on sampled rows of their final state."""
    torch = torch_cuda
    w = inputs.DECODE
    x, t, S, _ = _full_prefill(torch, w)
    steps = inputs.DECODE_STEPS
    s = inputs.decode_inputs(w, steps, seed=1)
    qs, ks, vs = upload(s, w.dtype)
    yd = torch.empty((steps, w.B, w.H, w.d_V), device="cuda:0", dtype=torch.float32)
    say("decode: %d steps over %dx%d heads" % (steps, w.B, w.H))
    for i in range(steps):
        sata.sata_decode_step(t, S, qs[i], ks[i], vs[i], yd[i])
    torch.cuda.synchronize()
    ydh = yd.cpu().numpy()
    assert not np.isnan(ydh).any()
    rng = np.random.default_rng(9)
    picks = [(0, 0), (w.B - 1, w.H - 1)] + [tuple(p) for p in
                                           zip(rng.integers(0, w.B, 6), rng.integers(0, w.H, 6))]
    for (b, h) in picks:
        cat = {c: np.concatenate([x[c][b, h], s[c][:, b, h]], axis=0) for c in ("q", "k", "v")}
        n_all = w.n + steps
        rows = np.arange(w.n, n_all)
        ref = oracle.direct_rows(cat["q"][None], cat["k"][None], cat["v"][None], w.P,
                                 np.zeros_like(rows), rows)
        err = max_row_err(ydh[:, b, h], ref)
        say("  decode (%d,%d): y err %.3e over %d steps" % (b, h, err, steps))
        assert err <= TOL_BF16
    for (b, h) in picks[:2]:
        cat_k = np.concatenate([x["k"][b, h], s["k"][:, b, h]], axis=0)
        cat_v = np.concatenate([x["v"][b, h], s["v"][:, b, h]], axis=0)
        M = oracle.feature_dim(w.d_K, w.P)
        rows = sample_feature_rows(w.d_K, w.P, 80, 3 + b)
        ref_rows = oracle.state_rows(cat_k, cat_v, w.P, rows)
        Sg = S[b, h].cpu().numpy()
        err = sampled_state_err(Sg, ref_rows, rows, w.d_K, w.P)
        say("  final state (%d,%d): err %.3e" % (b, h, err))
        assert err <= TOL_BF16
        assert Sg[w.d_V, 0] == w.n + steps
    t.close()


def test_wide_prefill_and_decode_full_size(torch_cuda):
    """B=1, H=32, n=16384, d_K=d_V=128, P=4: chunked prefill, then the decode
    steps; head 0 in full over its first 2048 tokens, sampled rows of every head,
    every decode step of sampled heads, sampled final-state rows."""
    torch = torch_cuda
    w = inputs.WIDE
    x, t, S, y = _full_prefill(torch, w)
    yh = y.cpu().numpy().reshape(w.H, w.n, w.d_V)
    assert not np.isnan(yh).any()
    ref = oracle.direct(x["q"][0, 0, :2048], x["k"][0, 0, :2048], x["v"][0, 0, :2048], w.P)
    err = max_row_err(yh[0, :2048], ref)
    say("  head 0 first 2048 tokens: y err %.3e" % err)
    assert err <= TOL_BF16
    flat = {c: x[c].reshape(w.H, w.n, -1) for c in ("q", "k", "v")}
    pos = _sample_positions(w.n, 2, 6, lo=2048)
    hs = np.repeat(np.arange(w.H), pos.size)
    ts = np.tile(pos, w.H)
    _check_rows(yh, flat, w.P, hs, ts, "wide, all heads")

    steps = inputs.WIDE_DECODE_STEPS
    s = inputs.decode_inputs(w, steps, seed=1)
    qs, ks, vs = upload(s, w.dtype)
    yd = torch.empty((steps, w.B, w.H, w.d_V), device="cuda:0", dtype=torch.float32)
    say("wide decode: %d steps" % steps)
    for i in range(steps):
        sata.sata_decode_step(t, S, qs[i], ks[i], vs[i], yd[i])
    torch.cuda.synchronize()
    ydh = yd.cpu().numpy()
    for h in (0, 17, w.H - 1):
        cat = {c: np.concatenate([x[c][0, h], s[c][:, 0, h]], axis=0) for c in ("q", "k", "v")}
        rows = np.arange(w.n, w.n + steps)
        ref = oracle.direct_rows(cat["q"][None], cat["k"][None], cat["v"][None], w.P,
                                 np.zeros_like(rows), rows)
        err = max_row_err(ydh[:, 0, h], ref)
        say("  wide decode head %d: y err %.3e" % (h, err))
        assert err <= TOL_BF16
    for h in (0, w.H - 1):
        cat_k = np.concatenate([x["k"][0, h], s["k"][:, 0, h]], axis=0)
        cat_v = np.concatenate([x["v"][0, h], s["v"][:, 0, h]], axis=0)
        M = oracle.feature_dim(w.d_K, w.P)
        rows = sample_feature_rows(w.d_K, w.P, 60, 11 + h)
        ref_rows = oracle.state_rows(cat_k, cat_v, w.P, rows)
        Sg = S[0, h].cpu().numpy()
        err = sampled_state_err(Sg, ref_rows, rows, w.d_K, w.P)
        say("  wide final state head %d: err %.3e" % (h, err))
        assert err <= TOL_BF16
        assert Sg[w.d_V, 0] == w.n + steps
    t.close()
