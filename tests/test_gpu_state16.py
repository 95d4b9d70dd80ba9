"""GPU parity of the half-precision state (include/sata.h "Half-precision state"): the
prefill writing it, the conversions, the decode step over it (dense and pool), a prefill
continued from it, its range, and the decode workloads at full size.

Bars: y within 2e-2 of the oracle per row (max_j |y - y_ref| / max_j |y_ref|), states within
2e-2 per degree block and column (gpu_helpers.state_col_err / sampled_state_err), as for the
fp32 state.  The stored form itself is checked exactly where it is fixed: the fp32
normaliser column equals the fp32 state's, every value entry is the fp32 entry rounded to
fp16 at its block's exponent (error at most 2^-11 of the entry, or half an fp16 subnormal
step), the exponents and bounds follow the documented rule.  The state is read on the host
from the documented byte layout (gpu_helpers.state16_read).

After more than one write (decode steps, a continued prefill) each entry carries the fp16
rounding of every write, relative to the entry's size at that write; an entry that later
cancels toward zero then has an error relative to its earlier size.  There the value
columns of a degree block share one scale in the state bar (the largest |S_ref| over the
block's rows and value columns; gpu_helpers joint_values), and the fp32 normaliser column
keeps its own."""
import numpy as np
import pytest

import sensitive_cases as sc
from gpu_helpers import (TOL_BF16, TOL_F32, feature_degrees, inputs, max_row_err, new_state, new_state16, oracle,
                         prefill, sample_feature_rows, sampled_state_err, sata, say,
                         state16_read, state_col_err, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _prefill16(t, q, k, v, S16, continue_state=False):
    import torch
    B, H, n, _ = q.shape
    y = torch.full((B, H, n, v.shape[-1]), float("nan"), device="cuda:0", dtype=torch.float32)
    sata.sata_prefill(t, q, k, v, y, S16, continue_state=continue_state, state16=True)
    return y


def _oracle_state_err(Sd, k, v, d, P, seed, joint_values=False):
    """Per-degree-block error of a host state [d_V + 1, M] against the oracle (every row at
    d_K <= 64, sampled rows above)."""
    if d <= 64:
        _, S_ref = oracle.feature_form(None, k, v, P, want_y=False)
        return state_col_err(Sd, S_ref, d, P, joint_values)
    rows = sample_feature_rows(d, P, 240, seed)
    return sampled_state_err(Sd, oracle.state_rows(k, v, P, rows), rows, d, P, joint_values)


def _check_stored_form(raw, S32, d_K, d_V, P, exact_bound=True):
    """raw: one head's half-precision state; S32: the same head's fp32 state [cols, M_pad].
    Checks the stored form against the fp32 entries (see the module docstring)."""
    M = oracle.feature_dim(d_K, P)
    S, expo, bound, pads_zero = state16_read(raw, d_K, d_V, P)
    ref = np.asarray(S32, dtype=np.float64)[:, :M]
    assert pads_zero, "rows past m_p of a block must be zero"
    assert np.array_equal(S[d_V], ref[d_V]), "the normaliser column is kept in fp32"
    degs = feature_degrees(d_K, P)
    for p in range(P):
        blk = degs == p
        e = expo[p].astype(np.int64)[:, None]
        tol = np.abs(ref[:d_V, blk]) * 2.0 ** -11 + np.ldexp(1.0, e - 24)
        assert np.all(np.abs(S[:d_V, blk] - ref[:d_V, blk]) <= tol), "fp16 rounding of degree %d" % p
        mx = np.max(np.abs(ref[:d_V, blk]), axis=1)
        if exact_bound:
            assert np.array_equal(bound[p].astype(np.float64), mx), "bound = largest |entry| of the block"
        nz = bound[p] > 0
        if nz.any():
            _, ex = np.frexp(bound[p][nz].astype(np.float64))
            assert np.array_equal(expo[p][nz], ex - 1 - 14), "exponent = floor(log2 bound) - 14"
        assert np.all(np.abs(S[:d_V, blk]) * np.ldexp(1.0, -e) < 2.0 ** 15 * (1 + 2.0 ** -10))


# (d_K, d_V, P, n, dtype, seed, sigma): the matrix-core path (bf16, d = 64 / 128) at the
# scales where the top term shows, and the fp32 path at odd sizes (d_K = 7 puts every degree
# block in one 64-row group, so waves span several degrees)
PREFILL_CASES = [(64, 64, 4, 700, "bf16", 301, 0.75), (64, 64, 5, 700, "bf16", 302, 0.9),
                 (128, 128, 4, 300, "bf16", 303, 0.8), (64, 64, 3, 200, "f32", 304, 0.5),
                 (7, 20, 5, 150, "f32", 305, 0.7)]


@pytest.mark.parametrize("d_K,d_V,P,n,dtype,seed,sigma", PREFILL_CASES)
def test_prefill_state16(torch_cuda, d_K, d_V, P, n, dtype, seed, sigma):
    """Prefill into a half-precision state: y bit-identical to the fp32-state prefill, the
    stored form matches the fp32 state entry by entry, and the state matches the oracle."""
    torch = torch_cuda
    say("state16 prefill d_K=%d d_V=%d P=%d n=%d %s" % (d_K, d_V, P, n, dtype))
    x = inputs.draw((1, 2, n, d_K), (1, 2, n, d_V), dtype, sigma, 1.0, seed)
    q, k, v = upload(x, dtype)
    t = sata.sata_tables_build(d_K, P)
    S32 = new_state(1, 2, d_K, d_V, P)
    y32 = prefill(t, q, k, v, 64, S32)
    S16 = new_state16(1, 2, d_K, d_V, P)
    y16 = _prefill16(t, q, k, v, S16)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32), "y must not depend on the state's storage form"
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    err = max_row_err(y16.cpu().numpy(), oracle.direct(x["q"], x["k"], x["v"], P))
    say("  y err %.3e" % err)
    assert err <= tol
    raw = S16.cpu().numpy()
    for h in range(2):
        _check_stored_form(raw[0, h], S32[0, h].cpu().numpy(), d_K, d_V, P)
        Sd = state16_read(raw[0, h], d_K, d_V, P)[0]
        assert Sd[d_V, 0] == n
        serr = _oracle_state_err(Sd, x["k"][0, h], x["v"][0, h], d_K, P, seed)
        say("  head %d state err %.3e" % (h, serr))
        assert serr <= TOL_BF16
    t.close()


def test_state16_conversions(torch_cuda):
    """pack(fp32 state) gives the bytes the prefill wrote; unpack gives back exactly the
    stored values in fp32 (padding rows zero)."""
    torch = torch_cuda
    d, P, n = 64, 4, 500
    x = sc.draw(d, P, 2, 3, n, 311)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    S32 = new_state(2, 3, d, d, P)
    prefill(t, q, k, v, 64, S32)
    S16 = new_state16(2, 3, d, d, P)
    _prefill16(t, q, k, v, S16)
    P16 = torch.full_like(S16, 0xAB)
    sata.sata_state_pack_f16(t, S32, P16, d)
    U = torch.full_like(S32, float("nan"))
    sata.sata_state_unpack_f16(t, S16, U, d)
    torch.cuda.synchronize()
    raw16 = S16.cpu().numpy()
    assert np.array_equal(P16.cpu().numpy(), raw16), "pack must write the bytes the prefill wrote"
    M = oracle.feature_dim(d, P)
    Un = U.cpu().numpy()
    for b in range(2):
        for h in range(3):
            Sd = state16_read(raw16[b, h], d, d, P)[0]
            assert np.array_equal(Un[b, h, :, :M].astype(np.float64), Sd)
            assert not Un[b, h, :, M:].any()
    t.close()


@pytest.mark.parametrize("d,P,n1,steps,seed,sigma", sc.DECODE)
def test_decode_state16_top_term(torch_cuda, d, P, n1, steps, seed, sigma):
    """Prefill into a half-precision state, then decode steps on it, at the scales where the
    top Taylor term shows; y at every step and the final state against the oracle; the
    header after the steps (bounds are the blocks' largest entries up to their fp16
    rounding)."""
    torch = torch_cuda
    say("state16 decode: prefill(%d) + %d steps, d=%d P=%d" % (n1, steps, d, P))
    x = sc.draw(d, P, 1, 2, n1 + steps, seed, sigma)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    S16 = new_state16(1, 2, d, d, P)
    _prefill16(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), S16)
    ys = []
    for T in range(n1, n1 + steps):
        y = torch.empty((1, 2, d), device="cuda:0")
        sata.sata_decode_step_f16(t, S16, q[:, :, T].contiguous(), k[:, :, T].contiguous(),
                                  v[:, :, T].contiguous(), y)
        ys.append(y.cpu().numpy())
    torch.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    err = max_row_err(np.stack(ys, axis=2), ref[:, :, n1:])
    say("  decode y err %.3e" % err)
    assert err <= TOL_BF16
    raw = S16.cpu().numpy()
    for h in range(2):
        Sd, expo, bound, pads_zero = state16_read(raw[0, h], d, d, P)
        assert pads_zero
        assert Sd[d, 0] == n1 + steps
        serr = _oracle_state_err(Sd, x["k"][0, h], x["v"][0, h], d, P, seed, joint_values=True)
        say("  head %d state err %.3e" % (h, serr))
        assert serr <= TOL_BF16
        degs = feature_degrees(d, P)
        for p in range(P):
            mx = np.max(np.abs(Sd[:d, degs == p]), axis=1)
            b = bound[p].astype(np.float64)
            assert np.all(mx <= b * (1 + 2.0 ** -11)) and np.all(mx >= b * (1 - 2.0 ** -11))
    t.close()


def test_decode_state16_matches_fp32_state(torch_cuda):
    """The same decode steps on the fp32 and the half-precision state: both within the bar of
    the oracle, and within fp16 rounding of each other."""
    torch = torch_cuda
    d, P, n1, steps = 64, 4, 1000, 24
    x = inputs.draw((2, 4, n1 + steps, d), (2, 4, n1 + steps, d), "bf16", 0.5, 1.0, 321)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    S32 = new_state(2, 4, d, d, P)
    S16 = new_state16(2, 4, d, d, P)
    qa, ka, va = (z[:, :, :n1].contiguous() for z in (q, k, v))
    prefill(t, qa, ka, va, 64, S32)
    _prefill16(t, qa, ka, va, S16)
    y32, y16 = [], []
    for T in range(n1, n1 + steps):
        a = torch.empty((2, 4, d), device="cuda:0")
        b = torch.empty((2, 4, d), device="cuda:0")
        qs, ks, vs = q[:, :, T].contiguous(), k[:, :, T].contiguous(), v[:, :, T].contiguous()
        sata.sata_decode_step(t, S32, qs, ks, vs, a)
        sata.sata_decode_step_f16(t, S16, qs, ks, vs, b)
        y32.append(a.cpu().numpy())
        y16.append(b.cpu().numpy())
    torch.cuda.synchronize()
    y32, y16 = np.stack(y32, axis=2), np.stack(y16, axis=2)
    ref = oracle.direct(x["q"], x["k"], x["v"], P)[:, :, n1:]
    e32, e16, e_between = max_row_err(y32, ref), max_row_err(y16, ref), max_row_err(y16, y32.astype(np.float64))
    say("  fp32 state %.3e, fp16 state %.3e, between %.3e" % (e32, e16, e_between))
    assert e32 <= TOL_BF16 and e16 <= TOL_BF16
    assert e_between <= 5e-3
    t.close()


@pytest.mark.parametrize("d_K,d_V,P,seed", [(7, 20, 5, 361), (64, 64, 2, 362), (16, 3, 3, 363)])
def test_decode_state16_fp32_inputs_odd_sizes(torch_cuda, d_K, d_V, P, seed):
    """fp32 inputs and odd sizes (a partial group of value columns, several degree blocks inside
    one wave's rows, P from 2 to 5): a prefill into the half-precision state and decode steps
    on it, against the oracle (the bar of the half-precision state) and against the same steps
    on the fp32 state (which meets the fp32 bar)."""
    torch = torch_cuda
    n1, steps = 150, 6
    say("state16 decode, fp32 inputs: d_K=%d d_V=%d P=%d" % (d_K, d_V, P))
    x = inputs.draw((2, 3, n1 + steps, d_K), (2, 3, n1 + steps, d_V), "f32", 0.7, 1.0, seed)
    q, k, v = upload(x, "f32")
    t = sata.sata_tables_build(d_K, P)
    S32 = new_state(2, 3, d_K, d_V, P)
    S16 = new_state16(2, 3, d_K, d_V, P)
    qa, ka, va = (z[:, :, :n1].contiguous() for z in (q, k, v))
    prefill(t, qa, ka, va, 64, S32)
    _prefill16(t, qa, ka, va, S16)
    y32, y16 = [], []
    for T in range(n1, n1 + steps):
        a = torch.empty((2, 3, d_V), device="cuda:0")
        b = torch.empty((2, 3, d_V), device="cuda:0")
        qs, ks, vs = q[:, :, T].contiguous(), k[:, :, T].contiguous(), v[:, :, T].contiguous()
        sata.sata_decode_step(t, S32, qs, ks, vs, a)
        sata.sata_decode_step_f16(t, S16, qs, ks, vs, b)
        y32.append(a.cpu().numpy())
        y16.append(b.cpu().numpy())
    torch.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)[:, :, n1:]
    e32 = max_row_err(np.stack(y32, axis=2), ref)
    e16 = max_row_err(np.stack(y16, axis=2), ref)
    say("  fp32 state %.3e, half-precision state %.3e" % (e32, e16))
    assert e32 <= TOL_F32 and e16 <= TOL_BF16
    raw = S16.cpu().numpy()
    for b_, h in ((0, 0), (1, 2)):
        Sd, expo, bound, pads_zero = state16_read(raw[b_, h], d_K, d_V, P)
        assert pads_zero and Sd[d_V, 0] == n1 + steps
        cat_k = x["k"][b_, h]
        cat_v = x["v"][b_, h]
        serr = _oracle_state_err(Sd, cat_k, cat_v, d_K, P, seed, joint_values=True)
        say("  state (%d,%d) err %.3e" % (b_, h, serr))
        assert serr <= TOL_BF16
    t.close()


def test_decode_state16_pool_equals_dense(torch_cuda):
    """The pool form on half-precision states: bit-identical y and state bytes to the dense
    step; an entry with a slot outside the pool reads out NaN and leaves the pool alone."""
    torch = torch_cuda
    d, P, H, n1 = 64, 3, 2, 300
    x = inputs.draw((3, H, n1 + 2, d), (3, H, n1 + 2, d), "bf16", 0.6, 1.0, 331)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    dense = new_state16(3, H, d, d, P)
    _prefill16(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), dense)
    pool = torch.zeros((5,) + tuple(dense.shape[1:]), device="cuda:0", dtype=torch.uint8)
    slots_list = [4, 1, 2]
    for i, s in enumerate(slots_list):
        pool[s].copy_(dense[i])
    pool[0].fill_(7)
    pool[3].fill_(9)
    before = pool.clone()
    for T in range(n1, n1 + 2):
        qs, ks, vs = q[:, :, T].contiguous(), k[:, :, T].contiguous(), v[:, :, T].contiguous()
        yd = torch.empty((3, H, d), device="cuda:0")
        yp = torch.empty((3, H, d), device="cuda:0")
        sata.sata_decode_step_f16(t, dense, qs, ks, vs, yd)
        slots = torch.tensor(slots_list, dtype=torch.int32, device="cuda:0")
        sata.sata_decode_step_pool_f16(t, pool, slots, qs, ks, vs, yp)
        torch.cuda.synchronize()
        assert torch.equal(yd, yp)
    for i, s in enumerate(slots_list):
        assert torch.equal(pool[s], dense[i])
    assert torch.equal(pool[0], before[0]) and torch.equal(pool[3], before[3])
    # an entry outside the pool: NaN row, pool unchanged
    bad = torch.tensor([1, 5, 2], dtype=torch.int32, device="cuda:0")
    snap = pool.clone()
    yp = torch.zeros((3, H, d), device="cuda:0")
    sata.sata_decode_step_pool_f16(t, pool, bad, q[:, :, 0].contiguous(), k[:, :, 0].contiguous(),
                                   v[:, :, 0].contiguous(), yp)
    torch.cuda.synchronize()
    assert torch.isnan(yp[1]).all() and not torch.isnan(yp[0]).any()
    assert torch.equal(pool[4], snap[4]) and torch.equal(pool[0], snap[0])
    t.close()


@pytest.mark.parametrize("d,P,n1,n2,seed", sc.CONTINUE)
def test_continued_prefill_state16(torch_cuda, d, P, n1, n2, seed):
    """A prefill continued from a half-precision state (unpacked, scanned, packed again)."""
    say("state16 continued prefill d=%d P=%d %d + %d" % (d, P, n1, n2))
    x = sc.draw(d, P, 1, 2, n1 + n2, seed)
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    S16 = new_state16(1, 2, d, d, P)
    _prefill16(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), S16)
    y2 = _prefill16(t, q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(),
                    S16, continue_state=True)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    err = max_row_err(y2.cpu().numpy(), ref[:, :, n1:])
    say("  continued y err %.3e" % err)
    assert err <= TOL_BF16
    Sd = state16_read(S16.cpu().numpy()[0, 1], d, d, P)[0]
    assert Sd[d, 0] == n1 + n2
    serr = _oracle_state_err(Sd, x["k"][0, 1], x["v"][0, 1], d, P, seed, joint_values=True)
    say("  state err %.3e" % serr)
    assert serr <= TOL_BF16
    t.close()


def test_state16_range(torch_cuda):
    """Values far outside fp16's range: v x 2^20 and k x 4 (q / 4, so the weights are those
    of the unscaled inputs), a prefill of 2500 tokens (past fp16's exact integers: the token
    count lives in the fp32 normaliser) and decode steps; y against the oracle, finite."""
    torch = torch_cuda
    d, P, n1, steps = 64, 4, 2500, 8
    x = inputs.draw((1, 2, n1 + steps, d), (1, 2, n1 + steps, d), "bf16", 0.5, 1.0, 341)
    x = {"q": x["q"] / 4, "k": x["k"] * 4, "v": x["v"] * 2.0 ** 20}
    q, k, v = upload(x, "bf16")
    t = sata.sata_tables_build(d, P)
    S16 = new_state16(1, 2, d, d, P)
    y1 = _prefill16(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), S16)
    ys = []
    for T in range(n1, n1 + steps):
        y = torch.empty((1, 2, d), device="cuda:0")
        sata.sata_decode_step_f16(t, S16, q[:, :, T].contiguous(), k[:, :, T].contiguous(),
                                  v[:, :, T].contiguous(), y)
        ys.append(y.cpu().numpy())
    torch.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    yd = np.stack(ys, axis=2)
    assert np.isfinite(yd).all()
    e1 = max_row_err(y1.cpu().numpy(), ref[:, :, :n1])
    e2 = max_row_err(yd, ref[:, :, n1:])
    say("  prefill y err %.3e, decode y err %.3e (|y| ~ %.1e)" % (e1, e2, np.max(np.abs(ref))))
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16
    Sd, expo, bound, _ = state16_read(S16.cpu().numpy()[0, 0], d, d, P)
    assert Sd[d, 0] == n1 + steps
    assert expo.max() > 0, "the value columns need exponents past fp16's range here"
    t.close()


def test_state16_long_prefix(torch_cuda):
    """A prefix of n_p = 3e7 identical tokens (k0, v0) given as its fp32 state n_p phi(k0)
    [v0 | 1]^T, packed to half precision (value entries ~3e7 |v0|, far past fp16's range),
    then decode steps: y_T = (n_p w(q_T . k0) v0 + N_T) / (n_p w(q_T . k0) + D_T), with N_T,
    D_T the new tokens' numerator and normaliser; every piece from the oracle."""
    torch = torch_cuda
    n_p, steps, d, P = 30_000_000, 6, 64, 4
    x = inputs.draw((1, 1, steps + 1, d), (1, 1, steps + 1, d), "bf16", 0.5, 1.0, 351)
    k0, v0 = x["k"][0, 0, steps], x["v"][0, 0, steps]
    _, S1 = oracle.feature_form(None, k0[None], v0[None], P, want_y=False)
    Mp = sata.sata_state_stride(d, P)
    S0 = np.zeros((1, 1, d + 1, Mp), dtype=np.float32)
    S0[0, 0, :, :S1.shape[1]] = n_p * S1
    t = sata.sata_tables_build(d, P)
    S16 = new_state16(1, 1, d, d, P)
    sata.sata_state_pack_f16(t, torch.from_numpy(S0).cuda(), S16, d)
    q, k, v = upload({c: x[c][:, :, :steps] for c in ("q", "k", "v")}, "bf16")
    ys = []
    for T in range(steps):
        y = torch.empty((1, 1, d), device="cuda:0")
        sata.sata_decode_step_f16(t, S16, q[:, :, T].contiguous(), k[:, :, T].contiguous(),
                                  v[:, :, T].contiguous(), y)
        ys.append(y[0, 0].cpu().numpy())
    torch.cuda.synchronize()
    qn, kn, vn = (x[c][0, 0, :steps] for c in ("q", "k", "v"))
    y_new, den_new = oracle.direct(qn, kn, vn, P, return_den=True)
    _, w0 = oracle.direct(qn[:, None, :], np.broadcast_to(k0, (steps, 1, d)), np.zeros((steps, 1, d)),
                          P, return_den=True)
    num = n_p * w0[:, 0, None] * v0[None, :].astype(np.float64) + y_new * den_new[:, None]
    ref = num / (n_p * w0[:, 0] + den_new)[:, None]
    got = np.stack(ys)
    assert np.isfinite(got).all()
    err = max_row_err(got, ref)
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    t.close()


def _decode_full(torch, w, steps):
    """Prefill w into half-precision states, then `steps` decode steps over all heads; sampled
    heads checked at every step against the oracle and on sampled rows of their final state."""
    say("%s state16: prefill B=%d H=%d n=%d, %d decode steps" % (w.name, w.B, w.H, w.n, steps))
    x = inputs.prefill_inputs(w)
    q, k, v = upload(x, w.dtype)
    t = sata.sata_tables_build(w.d_K, w.P)
    S16 = new_state16(w.B, w.H, w.d_K, w.d_V, w.P)
    _prefill16(t, q, k, v, S16)
    s = inputs.decode_inputs(w, steps, seed=1)
    qs, ks, vs = upload(s, w.dtype)
    yd = torch.empty((steps, w.B, w.H, w.d_V), device="cuda:0", dtype=torch.float32)
    for i in range(steps):
        sata.sata_decode_step_f16(t, S16, qs[i], ks[i], vs[i], yd[i])
    torch.cuda.synchronize()
    ydh = yd.cpu().numpy()
    assert not np.isnan(ydh).any()
    rng = np.random.default_rng(19)
    picks = [(0, 0), (w.B - 1, w.H - 1)] + [tuple(p) for p in zip(rng.integers(0, w.B, 4), rng.integers(0, w.H, 4))]
    for (b, h) in picks:
        cat = {c: np.concatenate([x[c][b, h], s[c][:, b, h]], axis=0) for c in ("q", "k", "v")}
        rows = np.arange(w.n, w.n + steps)
        ref = oracle.direct_rows(cat["q"][None], cat["k"][None], cat["v"][None], w.P, np.zeros_like(rows), rows)
        err = max_row_err(ydh[:, b, h], ref)
        say("  decode (%d,%d): y err %.3e" % (b, h, err))
        assert err <= TOL_BF16
    raw = S16.cpu().numpy()
    for (b, h) in picks[:2]:
        cat_k = np.concatenate([x["k"][b, h], s["k"][:, b, h]], axis=0)
        cat_v = np.concatenate([x["v"][b, h], s["v"][:, b, h]], axis=0)
        rows = sample_feature_rows(w.d_K, w.P, 60, 23 + b)
        Sd = state16_read(raw[b, h], w.d_K, w.d_V, w.P)[0]
        err = sampled_state_err(Sd, oracle.state_rows(cat_k, cat_v, w.P, rows), rows, w.d_K, w.P,
                                joint_values=True)
        say("  final state (%d,%d): err %.3e" % (b, h, err))
        assert err <= TOL_BF16
        assert Sd[w.d_V, 0] == w.n + steps
    t.close()


def test_decode_state16_full_size(torch_cuda):
    """16 sequences x 32 heads, d = 64, P = 4: the decode workload on half-precision states."""
    _decode_full(torch_cuda, inputs.DECODE, inputs.DECODE_STEPS)


def test_wide_decode_state16_full_size(torch_cuda):
    """32 heads, d_K = d_V = 128, P = 4, a 16384-token prefill: the wide decode workload on
    half-precision states."""
    _decode_full(torch_cuda, inputs.WIDE, inputs.WIDE_DECODE_STEPS)
