"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars (written in each test): tables bit-exact; y within 2e-2 for bf16 inputs
with an fp32 state and 1e-5 for the fp32 path, as max over rows of
max_j |y - y_ref| / max_j |y_ref|; the final state per Taylor term: for every degree block
and column, max |dS| over the block's rows / max |S_ref| over them.
"""
import numpy as np
import pytest

from gpu_helpers import (TOL_BF16, TOL_F32, inputs, max_row_err, new_state, oracle, prefill,
                         say, sata, state_col_err, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _tables(d_K, P):
    return sata.sata_tables_build(d_K, P)


# --------------------------------------------------------------------------
# Tiny: d = 8, P = 4, fp32, chunk 16
# --------------------------------------------------------------------------

def test_tiny_prefill_y_and_state(torch_cuda):
    w = inputs.TINY
    say("tiny prefill n=%d chunk=%d fp32" % (w.n, w.chunk))
    x = inputs.prefill_inputs(w)
    q, k, v = upload(x, w.dtype)
    t = _tables(w.d_K, w.P)
    S = new_state(1, 1, w.d_K, w.d_V, w.P)
    y = prefill(t, q, k, v, w.chunk, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], w.P)
    err = max_row_err(y[0, 0].cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= TOL_F32
    _, S_ref = oracle.feature_form(None, x["k"][0, 0], x["v"][0, 0], w.P, want_y=False)
    M = S_ref.shape[1]
    S_gpu = S[0, 0].cpu().numpy()
    assert state_col_err(S_gpu[:, :M], S_ref, w.d_K, w.P) <= TOL_F32
    assert np.all(S_gpu[:, M:] == 0.0), "padding of the state must stay zero"
    assert S_gpu[w.d_V, 0] == w.n          # Z of the p = 0 feature counts the tokens
    t.close()


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_chunk_invariance_ragged(torch_cuda, chunk):
    w = inputs.TINY
    n = 300                                  # not a multiple of any chunk size
    say("tiny ragged n=%d chunk=%d" % (n, chunk))
    x = inputs.prefill_inputs(w, n=n, seed=3)
    q, k, v = upload(x, "f32")
    t = _tables(w.d_K, w.P)
    y = prefill(t, q, k, v, chunk)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], w.P)
    assert max_row_err(y[0, 0].cpu().numpy(), ref) <= TOL_F32
    t.close()


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 47])
def test_short_sequences(torch_cuda, n):
    w = inputs.TINY
    say("tiny short n=%d" % n)
    x = inputs.prefill_inputs(w, n=n, B=2, H=3, seed=4)
    q, k, v = upload(x, "f32")
    t = _tables(w.d_K, w.P)
    y = prefill(t, q, k, v, 16)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], w.P)
    assert max_row_err(y.cpu().numpy(), ref) <= TOL_F32
    if n == 1:
        assert np.allclose(y.cpu().numpy(), x["v"], rtol=1e-6, atol=1e-6)
    t.close()


@pytest.mark.parametrize("P", [1, 2, 3, 5])
def test_other_term_counts(torch_cuda, P):
    say("d=8 P=%d prefill" % P)
    w = inputs.TINY
    x = inputs.prefill_inputs(w, n=130, B=1, H=2, seed=5)
    q, k, v = upload(x, "f32")
    t = _tables(8, P)
    y = prefill(t, q, k, v, 32)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    assert max_row_err(y.cpu().numpy(), ref) <= TOL_F32
    if P == 1:
        cm = np.cumsum(x["v"], axis=2) / np.arange(1, 131)[None, None, :, None]
        assert np.allclose(y.cpu().numpy(), cm, rtol=1e-5, atol=1e-6)
    t.close()


def test_unequal_key_value_dims(torch_cuda):
    say("d_K=16 d_V=5 prefill and decode")
    x = inputs.draw((1, 2, 90, 16), (1, 2, 90, 5), "f32", 0.6, 1.0, 6)
    q, k, v = upload(x, "f32")
    t = _tables(16, 4)
    S = new_state(1, 2, 16, 5, 4)
    y = prefill(t, q, k, v, 32, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    assert max_row_err(y.cpu().numpy(), ref) <= TOL_F32
    t.close()


# --------------------------------------------------------------------------
# Decode: state recurrence one token at a time
# --------------------------------------------------------------------------

def test_decode_from_empty_state_tiny(torch_cuda):
    w = inputs.TINY
    n = 64
    say("tiny decode from empty state, %d steps" % n)
    x = inputs.prefill_inputs(w, n=n, B=2, H=2, seed=7)
    t = _tables(w.d_K, w.P)
    S = new_state(2, 2, w.d_K, w.d_V, w.P)
    ys = []
    torch = torch_cuda
    for T in range(n):
        q = torch.from_numpy(np.ascontiguousarray(x["q"][:, :, T])).cuda()
        k = torch.from_numpy(np.ascontiguousarray(x["k"][:, :, T])).cuda()
        v = torch.from_numpy(np.ascontiguousarray(x["v"][:, :, T])).cuda()
        y = torch.empty((2, 2, w.d_V), device="cuda:0")
        sata.sata_decode_step(t, S, q, k, v, y)
        ys.append(y.cpu().numpy())
    y = np.stack(ys, axis=2)
    ref = oracle.direct(x["q"], x["k"], x["v"], w.P)
    assert max_row_err(y, ref) <= TOL_F32
    _, S_ref = oracle.feature_form(None, x["k"][1, 0], x["v"][1, 0], w.P, want_y=False)
    M = S_ref.shape[1]
    Sg = S[1, 0].cpu().numpy()
    assert state_col_err(Sg[:, :M], S_ref, w.d_K, w.P) <= TOL_F32
    assert np.all(Sg[:, M:] == 0.0)
    t.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode_equals_longer_prefill(torch_cuda, dtype):
    torch = torch_cuda
    d, P, n1, steps = 16, 4, 77, 9
    say("prefill(%d) + %d decode steps, d=%d %s" % (n1, steps, d, dtype))
    x = inputs.draw((2, 3, n1 + steps, d), (2, 3, n1 + steps, d), dtype, 0.5, 1.0, 8)
    t = _tables(d, P)
    q, k, v = upload(x, dtype)
    S = new_state(2, 3, d, d, P)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(),
            32, S)
    ys = []
    for T in range(n1, n1 + steps):
        y = torch.empty((2, 3, d), device="cuda:0")
        sata.sata_decode_step(t, S, q[:, :, T].contiguous(), k[:, :, T].contiguous(),
                              v[:, :, T].contiguous(), y)
        ys.append(y.cpu().numpy())
    S2 = new_state(2, 3, d, d, P)
    yfull = prefill(t, q, k, v, 32, S2)
    torch.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert max_row_err(np.stack(ys, axis=2), ref[:, :, n1:]) <= tol
    assert max_row_err(yfull.cpu().numpy(), ref) <= tol
    M = sata.sata_feature_dim(d, P)
    Sa = S.cpu().numpy()[..., :M]
    Sb = S2.cpu().numpy()[..., :M]
    rel = np.max(np.abs(Sa - Sb)) / np.max(np.abs(Sb))
    assert rel <= 1e-5
    t.close()


def test_prefill_continue_equals_one_prefill(torch_cuda):
    say("prefill(n1) + prefill(n2, continue) == prefill(n1 + n2)")
    d, P, n1, n2 = 8, 4, 96, 70
    x = inputs.draw((1, 2, n1 + n2, d), (1, 2, n1 + n2, d), "f32", 1.0, 1.0, 9)
    t = _tables(d, P)
    q, k, v = upload(x, "f32")
    S = new_state(1, 2, d, d, P)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(),
            16, S)
    y2 = prefill(t, q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(),
                 v[:, :, n1:].contiguous(), 16, S, continue_state=True)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    assert max_row_err(y2.cpu().numpy(), ref[:, :, n1:]) <= TOL_F32
    _, S_ref = oracle.feature_form(None, x["k"][0, 1], x["v"][0, 1], P, want_y=False)
    M = S_ref.shape[1]
    assert state_col_err(S[0, 1].cpu().numpy()[:, :M], S_ref, d, P) <= TOL_F32
    t.close()


def test_segmented_prefill_is_bit_identical(torch_cuda):
    """A workspace cap that forces many segments changes nothing in the result."""
    say("segmented prefill vs one segment")
    d, P, n = 8, 4, 500
    x = inputs.draw((2, 2, n, d), (2, 2, n, d), "f32", 1.0, 1.0, 10)
    q, k, v = upload(x, "f32")
    t = _tables(d, P)
    S1 = new_state(2, 2, d, d, P)
    y1 = prefill(t, q, k, v, 16, S1)
    t.set_workspace_limit(64 * 1024)
    y2 = prefill(t, q, k, v, 16)            # no caller state: the library carries it
    S3 = new_state(2, 2, d, d, P)
    y3 = prefill(t, q, k, v, 16, S3)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(y1, y2) and torch_cuda.equal(y1, y3)
    assert torch_cuda.equal(S1, S3)
    t.close()


# --------------------------------------------------------------------------
# d = 64, P = 4 (the Mid workload: B=1, H=8, n=4096)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mid_parity(torch_cuda, dtype):
    w = inputs.MID
    say("mid prefill B=%d H=%d n=%d d=%d %s" % (w.B, w.H, w.n, w.d_K, dtype))
    x = inputs.prefill_inputs(w)
    q, k, v = upload(x, dtype)
    t = _tables(w.d_K, w.P)
    S = new_state(w.B, w.H, w.d_K, w.d_V, w.P)
    y = prefill(t, q, k, v, w.chunk, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], w.P)
    err = max_row_err(y.cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    # final state of head (0, 3) against the literal feature sum
    _, S_ref = oracle.feature_form(None, x["k"][0, 3], x["v"][0, 3], w.P, want_y=False)
    M = S_ref.shape[1]
    Sg = S[0, 3].cpu().numpy()
    serr = state_col_err(Sg[:, :M], S_ref, w.d_K, w.P)
    say("  state err %.3e" % serr)
    assert serr <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    assert np.all(Sg[:, M:] == 0.0)
    assert Sg[w.d_V, 0] == w.n
    t.close()


# --------------------------------------------------------------------------
# bf16 MFMA scan (d_K = d_V = 64, P = 4, chunk 64): ragged, continued, segmented
# --------------------------------------------------------------------------

def _bf16_64(n, B, H, seed):
    return inputs.draw((B, H, n, 64), (B, H, n, 64), "bf16", 0.5, 1.0, seed)


def test_mfma_ragged_and_short(torch_cuda):
    for n in (1, 63, 64, 65, 1000):
        say("mfma bf16 d=64 n=%d" % n)
        x = _bf16_64(n, 1, 3, 20 + n)
        q, k, v = upload(x, "bf16")
        t = _tables(64, 4)
        S = new_state(1, 3, 64, 64, 4)
        y = prefill(t, q, k, v, 64, S)
        torch_cuda.cuda.synchronize()
        ref = oracle.direct(x["q"], x["k"], x["v"], 4)
        err = max_row_err(y.cpu().numpy(), ref)
        say("  y err %.3e" % err)
        assert err <= TOL_BF16
        _, S_ref = oracle.feature_form(None, x["k"][0, 2], x["v"][0, 2], 4, want_y=False)
        M = S_ref.shape[1]
        Sg = S[0, 2].cpu().numpy()
        assert state_col_err(Sg[:, :M], S_ref, 64, 4) <= TOL_BF16
        assert np.all(Sg[:, M:] == 0.0)
        t.close()


def test_mfma_continue_from_state(torch_cuda):
    say("mfma prefill(700) + prefill(500, continue) vs oracle")
    n1, n2 = 700, 500
    x = _bf16_64(n1 + n2, 1, 2, 30)
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    S = new_state(1, 2, 64, 64, 4)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(),
            64, S)
    y2 = prefill(t, q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(),
                 v[:, :, n1:].contiguous(), 64, S, continue_state=True)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y2.cpu().numpy(), ref[:, :, n1:])
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    _, S_ref = oracle.feature_form(None, x["k"][0, 1], x["v"][0, 1], 4, want_y=False)
    M = S_ref.shape[1]
    assert state_col_err(S[0, 1].cpu().numpy()[:, :M], S_ref, 64, 4) <= TOL_BF16
    t.close()


def test_mfma_segmented_matches_single_segment(torch_cuda):
    """Segments carry the state through fp32 memory with the key-side factors
    divided out and back in: equal to one segment to fp32 rounding."""
    say("mfma segmented vs one segment")
    n = 64 * 20 + 17
    x = _bf16_64(n, 2, 2, 31)
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    S1 = new_state(2, 2, 64, 64, 4)
    y1 = prefill(t, q, k, v, 64, S1)
    t.set_workspace_limit(4 << 20)
    S2 = new_state(2, 2, 64, 64, 4)
    y2 = prefill(t, q, k, v, 64, S2)
    y3 = prefill(t, q, k, v, 64)
    torch_cuda.cuda.synchronize()
    d12 = float((y1 - y2).abs().max() / y1.abs().max())
    d13 = float((y1 - y3).abs().max() / y1.abs().max())
    dS = float((S1 - S2).abs().max() / S1.abs().max())
    say("  rel diffs y %.2e %.2e state %.2e" % (d12, d13, dS))
    assert d12 <= 1e-5 and d13 <= 1e-5 and dS <= 1e-5
    t.close()


# --------------------------------------------------------------------------
# bf16 MFMA scan with 128-wide heads: two column groups (d_V = 128) and the
# 17-slot raw rows of d_K = 128; state checked on sampled rows
# --------------------------------------------------------------------------

def _state_check(S_head, x_k, x_v, P, n_rows, seed, tol):
    from gpu_helpers import sample_feature_rows, sampled_state_err
    d_K = x_k.shape[-1]
    M = oracle.feature_dim(d_K, P)
    rows = sample_feature_rows(d_K, P, n_rows, seed)
    ref = oracle.state_rows(x_k, x_v, P, rows)
    Sg = S_head.cpu().numpy()
    err = sampled_state_err(Sg, ref, rows, d_K, P)
    say("  state err %.3e on %d sampled rows" % (err, rows.size))
    assert err <= tol
    assert np.all(Sg[:, M:] == 0.0), "padding of the state must stay zero"


@pytest.mark.parametrize("dK,dV,n", [(128, 128, 200), (128, 64, 130), (64, 128, 129)])
def test_mfma_wide_heads(torch_cuda, dK, dV, n):
    say("mfma bf16 d_K=%d d_V=%d n=%d" % (dK, dV, n))
    x = inputs.draw((1, 2, n, dK), (1, 2, n, dV), "bf16", 0.35, 1.0, 50 + dK + dV)
    q, k, v = upload(x, "bf16")
    t = _tables(dK, 4)
    S = new_state(1, 2, dK, dV, 4)
    y = prefill(t, q, k, v, 64, S)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y.cpu().numpy(), ref)
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    for h in (0, 1):
        _state_check(S[0, h], x["k"][0, h], x["v"][0, h], 4, 150, h, TOL_BF16)
    assert float(S[0, 1, dV, 0]) == n
    t.close()


def test_mfma_wide_continue_and_segmented(torch_cuda):
    """d = 128: a continued prefill reaches the oracle, and a run cut into segments
    by a small workspace equals one segment to fp32 rounding."""
    say("mfma d=128 continue + segmented")
    n1, n2 = 150, 190
    x = inputs.draw((1, 2, n1 + n2, 128), (1, 2, n1 + n2, 128), "bf16", 0.35, 1.0, 61)
    q, k, v = upload(x, "bf16")
    t = _tables(128, 4)
    S = new_state(1, 2, 128, 128, 4)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(),
            64, S)
    y2 = prefill(t, q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(),
                 v[:, :, n1:].contiguous(), 64, S, continue_state=True)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y2.cpu().numpy(), ref[:, :, n1:])
    say("  continued y err %.3e" % err)
    assert err <= TOL_BF16
    _state_check(S[0, 0], x["k"][0, 0], x["v"][0, 0], 4, 100, 7, TOL_BF16)

    S1 = new_state(1, 2, 128, 128, 4)
    y1 = prefill(t, q, k, v, 64, S1)
    t.set_workspace_limit(64 << 20)          # a few chunks per segment at d = 128
    S2 = new_state(1, 2, 128, 128, 4)
    y3 = prefill(t, q, k, v, 64, S2)
    torch_cuda.cuda.synchronize()
    d13 = float((y1 - y3).abs().max() / y1.abs().max())
    dS = float((S1 - S2).abs().max() / S1.abs().max())
    say("  segmented rel diffs y %.2e state %.2e" % (d13, dS))
    assert d13 <= 1e-5 and dS <= 1e-5
    t.close()


def test_mfma_large_values_stay_finite(torch_cuda):
    """v = 8192 for every token (the constant feature's row of the state reaches n max|v| =
    3.4e7, past fp16's range): the per-head value scale and the per-window exponents keep
    every fp16 operand in range.  The exact y is v, for all 4096 rows."""
    n = 4096
    say("mfma large values: v = 8192, n = %d" % n)
    x = _bf16_64(n, 1, 1, 50)
    x["v"][...] = 8192.0
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    y = prefill(t, q, k, v, 64)
    torch_cuda.cuda.synchronize()
    yn = y[0, 0].cpu().numpy()
    assert np.isfinite(yn).all()
    err = np.max(np.abs(yn - 8192.0)) / 8192.0
    say("  max |y - 8192| / 8192 = %.3e" % err)
    assert err <= TOL_BF16
    t.close()


@pytest.mark.parametrize("d", [64, 128])
def test_mfma_power_of_two_rescaled_inputs(torch_cuda, d):
    """q 2^10, k 2^-10 and v 2^13 leave q.k unchanged and scale y by 2^13 exactly (the bf16
    values scale exactly).  The operand magnitudes (|q| up to ~2000, |k| down to ~1e-6)
    are far outside fp16's comfortable range; the per-head power-of-two input scales make
    the fp16 operands identical, so y / 2^13 equals the unscaled run, which meets the oracle."""
    n = 700
    say("mfma power-of-two rescaled inputs, d=%d n=%d" % (d, n))
    x = inputs.draw((1, 2, n, d), (1, 2, n, d), "bf16", 0.5 if d == 64 else 0.35, 1.0, 51)
    q, k, v = upload(x, "bf16")
    t = _tables(d, 4)
    y1 = prefill(t, q, k, v, 64)
    y2 = prefill(t, q * 1024.0, k * (1.0 / 1024.0), v * 8192.0, 64)
    torch_cuda.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], 4)
    err = max_row_err(y1.cpu().numpy(), ref)
    rel = float((y2 / 8192.0 - y1).abs().max() / y1.abs().max())
    say("  y err %.3e; rescaled run vs plain %.3e" % (err, rel))
    assert err <= TOL_BF16
    assert torch_cuda.isfinite(y2).all() and rel <= 1e-6
    t.close()


def test_mfma_chained_continue_large_context_values(torch_cuda):
    """Eight prefills of 2048 tokens, each continuing the previous state, with v ~ N(0, 4096^2):
    n max|v| reaches about 3e8 (the fp16 state copy of the first matrix-core design overflowed
    at 1.6e7).  Sampled rows of every continued prefill and sampled rows of the final state
    against the oracle over the whole 16384-token sequence."""
    from gpu_helpers import sample_feature_rows, sampled_state_err
    torch = torch_cuda
    n1, parts = 2048, 8
    n = n1 * parts
    say("mfma chained continue: %d x %d tokens, v ~ N(0, 4096^2)" % (parts, n1))
    x = inputs.draw((1, 1, n, 64), (1, 1, n, 64), "bf16", 0.5, 4096.0, 52)
    say("  n max|v| = %.2e" % (n * np.max(np.abs(x["v"]))))
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    S = new_state(1, 1, 64, 64, 4)
    ys = []
    for i in range(parts):
        sl = slice(i * n1, (i + 1) * n1)
        ys.append(prefill(t, q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                          64, S, continue_state=i > 0))
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2)[0, 0].cpu().numpy()
    assert np.isfinite(y).all()
    rows = np.unique(np.concatenate([np.arange(0, n, 997), [n1 - 1, n1, n - 2, n - 1]]))
    ref = oracle.direct_rows(x["q"][0], x["k"][0], x["v"][0], 4, np.zeros_like(rows), rows)
    err = max_row_err(y[rows], ref)
    say("  %d sampled rows: y err %.3e" % (rows.size, err))
    assert err <= TOL_BF16
    frows = sample_feature_rows(64, 4, 120, 5)
    serr = sampled_state_err(S[0, 0].cpu().numpy(), oracle.state_rows(x["k"][0, 0], x["v"][0, 0], 4, frows),
                             frows, 64, 4)
    say("  final state err %.3e (per degree block)" % serr)
    assert serr <= TOL_BF16
    t.close()


def test_mfma_continue_past_2_24_tokens(torch_cuda):
    """A prefix of n_p = 3e7 identical tokens (k0, v0 = 0), given as its state n_p phi(k0)
    [v0 | 1]^T (its p = 0 normaliser entry, the token count, is past fp32's exact integers
    and far past fp16's range), then 4096 new tokens continued from it.  With the prefix in
    the state, y_T = N_T / (n_p w(q_T . k0) + D_T), N_T and D_T the new tokens' numerator and
    normaliser; every piece comes from the oracle."""
    torch = torch_cuda
    n_p, n = 30_000_000, 4096
    say("mfma continue after a %d-token prefix state" % n_p)
    x = inputs.draw((1, 1, n + 1, 64), (1, 1, n + 1, 64), "bf16", 0.5, 1.0, 53)
    k0 = x["k"][0, 0, n]
    v0 = np.zeros(64, dtype=np.float32)
    _, S1 = oracle.feature_form(None, k0[None], v0[None], 4, want_y=False)
    Mp = sata.sata_state_stride(64, 4)
    S0 = np.zeros((1, 1, 65, Mp), dtype=np.float32)
    S0[0, 0, :, :S1.shape[1]] = n_p * S1
    S = torch.from_numpy(S0).cuda()
    q, k, v = upload({c: x[c][:, :, :n] for c in ("q", "k", "v")}, "bf16")
    t = _tables(64, 4)
    y = prefill(t, q, k, v, 64, S, continue_state=True)
    torch.cuda.synchronize()
    y_new, den_new = oracle.direct(x["q"][0, 0, :n], x["k"][0, 0, :n], x["v"][0, 0, :n], 4, return_den=True)
    # w(q_T . k0): the normaliser of a one-token sequence (q_T, k0), one head per row T
    _, w0 = oracle.direct(x["q"][0, 0, :n, None, :], np.broadcast_to(k0, (n, 1, 64)),
                          np.zeros((n, 1, 64)), 4, return_den=True)
    ref = y_new * den_new[:, None] / (n_p * w0[:, 0] + den_new)[:, None]
    yn = y[0, 0].cpu().numpy()
    assert np.isfinite(yn).all()
    err = max_row_err(yn, ref)
    say("  y err %.3e (|y| ~ %.1e)" % (err, np.max(np.abs(ref))))
    assert err <= TOL_BF16
    t.close()


@pytest.mark.parametrize("d,P", [(64, 2), (64, 3), (64, 5), (128, 3)])
def test_mfma_term_counts_prefill_then_decode(torch_cuda, d, P):
    """The matrix-core prefill (one level) at other term counts (another parent depth in the
    operand building), then decode steps on its state, against the oracle."""
    torch = torch_cuda
    n1, steps = 700, 3
    say("mfma bf16 d=%d P=%d: prefill(%d) + %d decode steps" % (d, P, n1, steps))
    x = inputs.draw((1, 2, n1 + steps, d), (1, 2, n1 + steps, d), "bf16", 0.5 if d == 64 else 0.35, 1.0, 60 + P)
    q, k, v = upload(x, "bf16")
    t = _tables(d, P)
    t.set_prefill_split(1)
    S = new_state(1, 2, d, d, P)
    y1 = prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), 64, S)
    ys = []
    for T in range(n1, n1 + steps):
        y = torch.empty((1, 2, d), device="cuda:0")
        sata.sata_decode_step(t, S, q[:, :, T].contiguous(), k[:, :, T].contiguous(), v[:, :, T].contiguous(), y)
        ys.append(y.cpu().numpy())
    torch.cuda.synchronize()
    ref = oracle.direct(x["q"], x["k"], x["v"], P)
    e1 = max_row_err(y1.cpu().numpy(), ref[:, :, :n1])
    e2 = max_row_err(np.stack(ys, axis=2), ref[:, :, n1:])
    say("  prefill y err %.3e, decode y err %.3e" % (e1, e2))
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16
    t.close()


def test_mfma_odd_chunk_count_under_small_cap(torch_cuda):
    """n = 560 (9 chunks, not a whole number of readout windows) under a 4 MiB workspace cap:
    the segment length is rounded to whole windows (it once rounded down to zero and divided
    by it); the result matches the oracle and the single-segment run."""
    n = 560
    say("mfma n=%d under a 4 MiB cap" % n)
    x = _bf16_64(n, 1, 1, 33)
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    t.set_prefill_split(1)
    S1 = new_state(1, 1, 64, 64, 4)
    y1 = prefill(t, q, k, v, 64, S1)
    t.set_workspace_limit(4 << 20)
    nbytes, nseg, _ = t.prefill_workspace(1, 1, n, 64, with_state=True)
    say("  plan: %d segments, %d bytes" % (nseg, nbytes))
    assert nseg >= 2
    S2 = new_state(1, 1, 64, 64, 4)
    y2 = prefill(t, q, k, v, 64, S2)
    torch_cuda.cuda.synchronize()
    err = max_row_err(y2.cpu().numpy(), oracle.direct(x["q"], x["k"], x["v"], 4))
    say("  y err %.3e" % err)
    assert err <= TOL_BF16
    assert float((y1 - y2).abs().max() / y1.abs().max()) <= 1e-5
    assert float((S1 - S2).abs().max() / S1.abs().max()) <= 1e-5
    t.close()


def test_bf16_prefill_is_reproducible(torch_cuda):
    """Two identical bf16 prefills (matrix-core scan, the finalize's fixed-order sums) give
    bit-identical y and final states."""
    say("bf16 prefill run twice, d=64 n=3000 H=3")
    x = _bf16_64(3000, 1, 3, 34)
    q, k, v = upload(x, "bf16")
    t = _tables(64, 4)
    outs = []
    for _ in range(2):
        S = new_state(1, 3, 64, 64, 4)
        y = prefill(t, q, k, v, 64, S)
        torch_cuda.cuda.synchronize()
        outs.append((y.cpu().numpy(), S.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
    t.close()
