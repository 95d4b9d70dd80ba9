"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each check ties the oracle to something other than itself: numbers the pages
print (tests/golden/), closed forms, brute force in exact integer arithmetic,
special cases that reduce to a textbook or library routine, and invariants.
Chosen so that a dropped term, a wrong sign, index, factorial, scale or
multiplicity anywhere in the oracle fails at least one of them
(tests/test_oracle_mutations.py plants such mistakes to show it).

Pages: "self-attention-constant-cost-taylor-approximation" ([TA]) and
"constant-cost-attention-hardware-optimization" ([HW]) on blog.hotdry.top.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from constant_cost_self_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Tables  ([TA Taylor], [TA Features])
# --------------------------------------------------------------------------

def test_worked_example_d2_p2():
    g = _gold("worked_example_d2_p2.json")
    M, C = oracle.tables(g["d"], g["p"])
    assert M.tolist() == g["M_p"]
    assert C.tolist() == g["C_p"]


@pytest.mark.parametrize("d", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("p", [0, 1, 2, 3, 4])
def test_table_counts_and_order(d, p):
    M, C = oracle.tables(d, p)
    # basis size binom(d+p-1, p)  [TA Taylor]
    assert M.shape == (math.comb(d + p - 1, p), p)
    # every ordered tuple is counted once: sum C_p = d^p (multinomial theorem)
    assert int(C.sum()) == d ** p
    if p > 0:
        assert np.all(np.diff(M, axis=1) >= 0), "rows must be non-decreasing"
        rows = [tuple(r) for r in M.tolist()]
        assert rows == sorted(set(rows)), "rows must be unique and in lex order"
        assert M.min() >= 0 and M.max() < d
    # C_p is the multinomial coefficient p! / prod(count_i!)
    for r in range(M.shape[0]):
        _, counts = np.unique(M[r], return_counts=True)
        expect = math.factorial(p)
        for c in counts:
            expect //= math.factorial(int(c))
        assert C[r] == expect


def test_page_basis_sizes():
    g = _gold("page_numbers.json")
    m64 = [oracle.tables(64, p)[0].shape[0] for p in range(4)]
    assert m64 == [1, 64, 2080, 45760]
    assert sum(m64) == g["basis_size_d64_P4"]["value"]
    assert oracle.feature_dim(64, 4) == 47905
    assert oracle.feature_dim(8, 4) == 165
    assert oracle.feature_dim(128, 4) == 366145


@pytest.mark.parametrize("d", [2, 3, 4])
@pytest.mark.parametrize("p", [0, 1, 2, 3])
def test_symmetric_identity_exact(d, p):
    """(q.k)^p = <phi_p(q), phi_p(k)>_{C_p}, exact, on small integer vectors."""
    rng = np.random.default_rng(100 + 10 * d + p)
    M, C = oracle.tables(d, p)
    for _ in range(20):
        q = rng.integers(-3, 4, size=d)
        k = rng.integers(-3, 4, size=d)
        lhs = int(np.dot(q, k)) ** p
        # the full expansion over all d^p ordered tuples, in Python integers
        full = sum(math.prod(int(q[i]) * int(k[i]) for i in tup)
                   for tup in itertools.product(range(d), repeat=p))
        fq = oracle.features(p, M, q.astype(np.float64))
        fk = oracle.features(p, M, k.astype(np.float64))
        sym = sum(int(C[r]) * int(round(fq[r])) * int(round(fk[r])) for r in range(len(C)))
        assert lhs == full == sym


def test_features_literal_product():
    """phi_p on a vector of distinct primes factorises uniquely back to the row."""
    primes = np.array([2.0, 3.0, 5.0, 7.0, 11.0])
    for p in range(4):
        M, _ = oracle.tables(5, p)
        f = oracle.features(p, M, primes)
        for r in range(M.shape[0]):
            assert f[r] == math.prod(primes[i] for i in M[r])


# --------------------------------------------------------------------------
# Direct form  ([TA Features]: truncated kernel, causal sums t <= T)
# --------------------------------------------------------------------------

def _np_attention(q, k, v, kernel):
    """Causal attention with an elementwise kernel of the scores, plain numpy."""
    n = q.shape[0]
    A = kernel(q @ k.T)
    A = A * np.tril(np.ones((n, n)))
    return (A @ v) / A.sum(axis=1, keepdims=True)


def _rand(n, dK, dV, sigma, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, dK)) * sigma, rng.standard_normal((n, dK)) * sigma,
            rng.standard_normal((n, dV)))


def test_P1_is_cumulative_mean():
    q, k, v = _rand(50, 6, 5, 1.0, 1)
    y = oracle.direct(q, k, v, 1)
    expect = np.cumsum(v, axis=0) / np.arange(1, 51)[:, None]
    np.testing.assert_allclose(y, expect, rtol=1e-13, atol=1e-13)


def test_first_row_is_v0():
    q, k, v = _rand(8, 4, 3, 1.0, 2)
    for P in (1, 2, 3, 4, 6):
        y = oracle.direct(q, k, v, P)
        np.testing.assert_allclose(y[0], v[0], rtol=1e-14, atol=1e-14)


def test_P2_is_linear_kernel():
    """P = 2: w = 1 + q.k/sqrt(d)."""
    q, k, v = _rand(40, 8, 4, 0.5, 3)
    c = math.sqrt(8)
    y = oracle.direct(q, k, v, 2)
    expect = _np_attention(q, k, v, lambda s: 1.0 + s / c)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_P3_is_quadratic_kernel():
    q, k, v = _rand(40, 8, 4, 0.5, 4)
    c = math.sqrt(8)
    y = oracle.direct(q, k, v, 3)
    expect = _np_attention(q, k, v, lambda s: 1.0 + s / c + (s / c) ** 2 / 2.0)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_direct_rows_sampled():
    """Sampled rows across heads equal the P = 3 quadratic kernel written with
    numpy, and oracle.direct's rows at P = 4."""
    c = math.sqrt(8)
    heads = [_rand(60, 8, 4, 0.5, 40 + h) for h in range(3)]
    q = np.stack([x[0] for x in heads]); k = np.stack([x[1] for x in heads])
    v = np.stack([x[2] for x in heads])
    hs = np.array([0, 2, 1, 1, 2, 0, 2])
    ts = np.array([0, 59, 17, 1, 33, 58, 0])
    got = oracle.direct_rows(q, k, v, 3, hs, ts)
    for r, (h, t) in enumerate(zip(hs, ts)):
        expect = _np_attention(q[h], k[h], v[h], lambda s: 1.0 + s / c + (s / c) ** 2 / 2.0)
        np.testing.assert_allclose(got[r], expect[t], rtol=1e-12, atol=1e-12)
    full = oracle.direct(q, k, v, 4)
    np.testing.assert_allclose(oracle.direct_rows(q, k, v, 4, hs, ts), full[hs, ts],
                               rtol=1e-14, atol=1e-14)


def test_large_P_converges_to_softmax():
    """The Taylor series of exp(q.k/c) converges to exp: at large P the direct
    form is softmax attention (scipy.special.softmax over the causal row)."""
    q, k, v = _rand(48, 8, 5, 0.4, 5)
    c = math.sqrt(8)
    s = q @ k.T / c
    ref = np.zeros_like(v)
    for T in range(48):
        ref[T] = scipy.special.softmax(s[T, :T + 1]) @ v[:T + 1]
    y = oracle.direct(q, k, v, 20)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.softmax(q, k, v), ref, rtol=1e-12, atol=1e-12)
    errs = [np.max(np.abs(oracle.direct(q, k, v, P) - ref)) for P in range(1, 9)]
    assert all(b < a for a, b in zip(errs, errs[1:])), errs


def test_softmax_rows_against_scipy_and_the_full_form():
    """Sampled softmax rows: scipy.special.softmax over each sampled causal row (several
    heads, first and last rows included), and the same rows of oracle.softmax."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((3, 40, 6)) * 0.7
    k = rng.standard_normal((3, 40, 6)) * 0.7
    v = rng.standard_normal((3, 40, 4))
    hs = np.array([0, 0, 1, 2, 2, 1])
    ts = np.array([0, 39, 17, 5, 39, 38])
    got = oracle.softmax_rows(q, k, v, hs, ts)
    c = math.sqrt(6)
    for r, (h, t) in enumerate(zip(hs, ts)):
        s = q[h, t] @ k[h, :t + 1].T / c
        np.testing.assert_allclose(got[r], scipy.special.softmax(s) @ v[h, :t + 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, oracle.softmax(q, k, v)[hs, ts], rtol=1e-14, atol=1e-14)


def test_affine_equivariance_in_v():
    q, k, v = _rand(30, 8, 4, 0.5, 6)
    y = oracle.direct(q, k, v, 4)
    y2 = oracle.direct(q, k, 2.5 * v - 1.25, 4)
    np.testing.assert_allclose(y2, 2.5 * y - 1.25, rtol=1e-12, atol=1e-12)


def test_joint_coordinate_permutation():
    q, k, v = _rand(30, 8, 4, 0.5, 7)
    perm = np.random.default_rng(8).permutation(8)
    np.testing.assert_allclose(oracle.direct(q[:, perm], k[:, perm], v, 4),
                               oracle.direct(q, k, v, 4), rtol=1e-12, atol=1e-12)


def test_batched_heads_independent():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 3, 20, 4)) * 0.5
    k = rng.standard_normal((2, 3, 20, 4)) * 0.5
    v = rng.standard_normal((2, 3, 20, 5))
    y = oracle.direct(q, k, v, 4)
    for b in range(2):
        for h in range(3):
            np.testing.assert_array_equal(y[b, h], oracle.direct(q[b, h], k[b, h], v[b, h], 4))


# --------------------------------------------------------------------------
# Feature form and state  ([TA Features], [TA Size])
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dK,dV,P,n,sigma", [(2, 3, 4, 30, 1.0), (3, 2, 3, 25, 1.0),
                                             (8, 8, 4, 64, 1.0), (8, 5, 5, 40, 0.7),
                                             (16, 16, 4, 48, 0.5), (64, 64, 4, 40, 0.5)])
def test_feature_form_equals_direct(dK, dV, P, n, sigma):
    q, k, v = _rand(n, dK, dV, sigma, 10 + dK + P)
    y_dir = oracle.direct(q, k, v, P)
    y_feat, S = oracle.feature_form(q, k, v, P)
    assert np.max(oracle.row_rel_err(y_feat, y_dir)) < 1e-12
    assert S.shape == (dV + 1, oracle.feature_dim(dK, P))


def test_state_invariants():
    """Z[p=0] = n; Z over p=1 rows = sum_t k_t; S[p=0 row] = sum_t v_t;
    the p=2 rows hold sum_t k_i k_j [v|1] for i <= j."""
    n, dK, dV, P = 37, 6, 4, 4
    q, k, v = _rand(n, dK, dV, 0.8, 11)
    _, S = oracle.feature_form(q, k, v, P, want_y=False)
    assert S[dV, 0] == n
    np.testing.assert_allclose(S[:dV, 0], v.sum(axis=0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S[dV, 1:1 + dK], k.sum(axis=0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S[:dV, 1:1 + dK], v.T @ k, rtol=1e-12, atol=1e-12)
    M2, _ = oracle.tables(dK, 2)
    off = 1 + dK
    for r, (i, j) in enumerate(M2.tolist()):
        np.testing.assert_allclose(S[dV, off + r], np.sum(k[:, i] * k[:, j]), rtol=1e-12)
        np.testing.assert_allclose(S[:dV, off + r], (k[:, i] * k[:, j]) @ v, rtol=1e-12,
                                   atol=1e-12)


def test_state_rows_match_feature_form():
    n, dK, dV, P = 29, 5, 3, 4
    q, k, v = _rand(n, dK, dV, 0.8, 12)
    _, S = oracle.feature_form(q, k, v, P, want_y=False)
    rows = np.array([0, 1, 4, 7, 20, S.shape[1] - 1])
    np.testing.assert_allclose(oracle.state_rows(k, v, P, rows), S[:, rows].T,
                               rtol=1e-13, atol=1e-13)


def test_state_is_additive_over_a_split():
    """The state after n1 + n2 tokens is the sum of the two parts' states."""
    q, k, v = _rand(40, 4, 3, 0.8, 13)
    _, S = oracle.feature_form(q, k, v, 4, want_y=False)
    _, S1 = oracle.feature_form(q[:17], k[:17], v[:17], 4, want_y=False)
    _, S2 = oracle.feature_form(q[17:], k[17:], v[17:], 4, want_y=False)
    np.testing.assert_allclose(S, S1 + S2, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms  ([TA Size], [HW State])
# --------------------------------------------------------------------------

def test_closed_forms_against_pages():
    g = _gold("page_numbers.json")
    s64 = oracle.state_elems(64, 64, 4)
    assert s64 == 3113825
    assert abs(s64 / g["state_elems_d64_P4_approx"]["value"] - 1) < 0.01
    assert abs(2 * s64 / 1e6 / g["state_mb_fp16_d64_P4_approx"]["value"] - 1) < 0.01
    s128 = oracle.state_elems(128, 128, 4)
    assert s128 == 47232705
    assert abs(s128 / g["state_elems_d128_P4_approx"]["value"] - 1) < 0.01
    assert 1.0 / oracle.alpha(4, 64) == pytest.approx(g["alpha4_d64"]["value_inverse"],
                                                      rel=1e-15)


@pytest.mark.parametrize("dK,dV,P", [(8, 8, 4), (64, 64, 4), (128, 128, 4), (16, 7, 5),
                                     (3, 2, 2), (32, 32, 1)])
def test_closed_forms_are_sums_over_terms(dK, dV, P):
    assert oracle.state_elems(dK, dV, P) == sum(
        oracle.state_elems_term(dK, dV, p) for p in range(P))
    assert oracle.state_elems(dK, dV, P) == (dV + 1) * oracle.feature_dim(dK, P)
    total = sum(oracle.flops_term(dK, dV, p) for p in range(P))
    assert oracle.flops_per_token(dK, dV, P) == pytest.approx(total, rel=1e-14)


def test_flops_values():
    assert round(oracle.flops_per_token(64, 64, 4)) == 12738308
    assert round(oracle.flops_per_token(128, 128, 4)) == 191110660
    assert round(oracle.flops_per_token(8, 8, 4)) == 6820


# --------------------------------------------------------------------------
# Inputs: the stored bf16 values round-trip exactly
# --------------------------------------------------------------------------

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3, 0.0], dtype=np.float32)
    bits, vals = inputs.bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert vals[0] == 1.0 and vals[1] == 1.0
    assert vals[2] == np.float32(1.0078125)
    assert vals[3] == -2.5 and vals[5] == 0.0
    assert abs(vals[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8
    assert np.all((vals.view(np.uint32) & 0xFFFF) == 0)


# --------------------------------------------------------------------------
# Gradients of the direct form (the chain rule through y = N / D)
# --------------------------------------------------------------------------

def _loss(q, k, v, dy, P):
    return float(np.sum(dy * oracle.direct(q, k, v, P)))


@pytest.mark.parametrize("P,seed", [(2, 0), (3, 1), (4, 2), (5, 3)])
def test_grad_matches_finite_differences(P, seed):
    """Every coordinate of dq, dk, dv against central differences of L = sum dy . y,
    computed with the forward oracle only (step 1e-5, fp64)."""
    rng = np.random.default_rng(40 + seed)
    n, dK, dV = 6, 3, 2
    q, k = rng.standard_normal((n, dK)), rng.standard_normal((n, dK))
    v, dy = rng.standard_normal((n, dV)), rng.standard_normal((n, dV))
    dq, dk, dv = oracle.direct_grad(q, k, v, dy, P)
    eps = 1e-5
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        for idx in np.ndindex(g.shape):
            args = {"q": q, "k": k, "v": v}
            plus, minus = dict(args), dict(args)
            plus[name] = args[name].copy()
            plus[name][idx] += eps
            minus[name] = args[name].copy()
            minus[name][idx] -= eps
            fd = (_loss(plus["q"], plus["k"], plus["v"], dy, P) -
                  _loss(minus["q"], minus["k"], minus["v"], dy, P)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


def test_grad_P1_closed_form():
    """P = 1: w = 1, y_T is the mean of v_0..v_T, so dq = dk = 0 and
    dv_t = sum_{T>=t} dy_T / (T + 1)."""
    rng = np.random.default_rng(50)
    n, dK, dV = 9, 4, 3
    q, k = rng.standard_normal((n, dK)), rng.standard_normal((n, dK))
    v, dy = rng.standard_normal((n, dV)), rng.standard_normal((n, dV))
    dq, dk, dv = oracle.direct_grad(q, k, v, dy, 1)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    ref = np.array([sum(dy[T] / (T + 1) for T in range(t, n)) for t in range(n)])
    np.testing.assert_allclose(dv, ref, rtol=1e-13, atol=1e-14)


def test_grad_invariant_under_value_shift():
    """Adding one vector to every v_t shifts every y_T by it, so no gradient changes."""
    rng = np.random.default_rng(51)
    n, dK, dV = 12, 3, 4
    q, k = rng.standard_normal((n, dK)), rng.standard_normal((n, dK))
    v, dy = rng.standard_normal((n, dV)), rng.standard_normal((n, dV))
    g0 = oracle.direct_grad(q, k, v, dy, 4)
    g1 = oracle.direct_grad(q, k, v + np.array([0.7, -1.3, 2.0, 0.25]), dy, 4)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-11)


def test_grad_batched_heads_independent():
    rng = np.random.default_rng(52)
    q, k = rng.standard_normal((2, 3, 7, 4)), rng.standard_normal((2, 3, 7, 4))
    v, dy = rng.standard_normal((2, 3, 7, 5)), rng.standard_normal((2, 3, 7, 5))
    g = oracle.direct_grad(q, k, v, dy, 3)
    gh = oracle.direct_grad(q[1, 2], k[1, 2], v[1, 2], dy[1, 2], 3)
    for a, b in zip(g, gh):
        np.testing.assert_array_equal(a[1, 2], b)
