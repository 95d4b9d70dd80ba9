"""fp64 CPU oracle for SATA causal self-attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
outputs); this module only compiles it, loads it with ctypes and converts
arrays.  Closed forms from the pages are written out here in Python.

Pages: Heinsen & Kozachkov, "Self-Attention at Constant Cost per Token via
Symmetry-Aware Taylor Approximation", as described on the blog.hotdry.top post
"self-attention-constant-cost-taylor-approximation" ([TA]), section
"Hidden-state size and compute analysis" ([TA Size]) for the closed forms.

Parity status of each function (what pins it is in tests/test_oracle_pins.py):
  tables, features, direct, feature_form, state_rows, direct_grad, closed forms: pinned;
  softmax, softmax_rows: pinned against scipy.special.softmax (a library routine); the
  Taylor-versus-softmax error it is used to report has no metric on the pages
  and is reported, not gated (parity unpinned for that report only).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, fp64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_tables.restype = ctypes.c_int64
    lib.oracle_tables.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i64p]
    lib.oracle_features.restype = None
    lib.oracle_features.argtypes = [ctypes.c_int, i32p, ctypes.c_int64, dp, dp]
    lib.oracle_alpha.restype = ctypes.c_double
    lib.oracle_alpha.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_direct.restype = None
    lib.oracle_direct.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp]
    lib.oracle_direct_rows.restype = None
    lib.oracle_direct_rows.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, i64p, i64p, ctypes.c_int64, dp]
    lib.oracle_feature_dim.restype = ctypes.c_int64
    lib.oracle_feature_dim.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_feature_form.restype = ctypes.c_int64
    lib.oracle_feature_form.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, dp, dp]
    lib.oracle_state_rows.restype = ctypes.c_int
    lib.oracle_state_rows.argtypes = [dp, dp, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, i64p,
                                      ctypes.c_int64, dp]
    lib.oracle_softmax.restype = None
    lib.oracle_softmax.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, dp]
    lib.oracle_softmax_rows.restype = None
    lib.oracle_softmax_rows.argtypes = [dp, dp, dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        i64p, i64p, ctypes.c_int64, dp]
    lib.oracle_direct_grad.restype = None
    lib.oracle_direct_grad.argtypes = [dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp, dp]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------------------
# Tables and features
# --------------------------------------------------------------------------

def tables(d: int, p: int):
    """(M_p int32 [m_p, p], C_p int64 [m_p]) by brute force over all d^p tuples."""
    lib = _load()
    m = lib.oracle_tables(d, p, None, None)
    if m < 0:
        raise ValueError("d^p too large to enumerate (d=%d, p=%d)" % (d, p))
    M = np.zeros((m, max(p, 1)), dtype=np.int32)
    C = np.zeros(m, dtype=np.int64)
    lib.oracle_tables(d, p, M.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                      C.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return M[:, :p].copy(), C


def features(p: int, M: np.ndarray, x) -> np.ndarray:
    """phi_p(x)[r] = prod_{i in M_p[r]} x[i] (literal product), fp64."""
    lib = _load()
    M = np.ascontiguousarray(M, dtype=np.int32)
    m = M.shape[0]
    Mflat = M.reshape(-1) if p > 0 else np.zeros(1, dtype=np.int32)
    x = _f64(x)
    out = np.zeros(m, dtype=np.float64)
    lib.oracle_features(p, Mflat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                        m, _dp(x), _dp(out))
    return out


def alpha(p: int, d_K: int) -> float:
    return _load().oracle_alpha(p, d_K)


def feature_dim(d_K: int, P: int) -> int:
    """Feature count M = sum_p m_p, counted by brute-force enumeration."""
    return int(_load().oracle_feature_dim(d_K, P))


# --------------------------------------------------------------------------
# y and the state
# --------------------------------------------------------------------------

def direct(q, k, v, P: int, return_den: bool = False):
    """O(n^2) direct form, fp64.  q,k: [..., n, dK]; v: [..., n, dV]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, dK = q.shape[-2:]
    dV = v.shape[-1]
    heads = int(np.prod(lead)) if lead else 1
    y = np.zeros(lead + (n, dV), dtype=np.float64)
    den = np.zeros(lead + (n,), dtype=np.float64)
    _load().oracle_direct(_dp(q), _dp(k), _dp(v), heads, n, dK, dV, P, _dp(y), _dp(den))
    return (y, den) if return_den else y


def direct_grad(q, k, v, dy, P: int):
    """Gradients (dq, dk, dv) of L = sum dy . y for the direct form, fp64, O(n^2) per head
    (the chain rule through y = N / D, written out pair by pair in oracle.c).
    q, k: [..., n, dK]; v, dy: [..., n, dV]."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    lead = q.shape[:-2]
    n, dK = q.shape[-2:]
    dV = v.shape[-1]
    heads = int(np.prod(lead)) if lead else 1
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    _load().oracle_direct_grad(_dp(q), _dp(k), _dp(v), _dp(dy), heads, n, dK, dV, P,
                               _dp(dq), _dp(dk), _dp(dv))
    return dq, dk, dv


def direct_rows(q, k, v, P: int, heads, rows):
    """Sampled rows of the direct form, fp64: out[r] = y[heads[r], rows[r]].
    q, k: [heads, n, dK]; v: [heads, n, dV] (leading dims flattened)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dK = q.shape[-2:]
    dV = v.shape[-1]
    q = q.reshape(-1, n, dK)
    k = k.reshape(-1, n, dK)
    v = v.reshape(-1, n, dV)
    heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if heads.shape != rows.shape or heads.ndim != 1:
        raise ValueError("heads and rows must be 1-D of one length")
    if heads.size and (heads.min() < 0 or heads.max() >= q.shape[0] or rows.min() < 0
                       or rows.max() >= n):
        raise ValueError("sampled head or row out of range")
    out = np.zeros((rows.shape[0], dV), dtype=np.float64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    _load().oracle_direct_rows(_dp(q), _dp(k), _dp(v), n, dK, dV, P,
                               heads.ctypes.data_as(i64p), rows.ctypes.data_as(i64p),
                               rows.shape[0], _dp(out))
    return out


def feature_form(q, k, v, P: int, want_y: bool = True):
    """Fixed-size-state form for one head: (y [n, dV] or None, S [dV+1, M])."""
    k, v = _f64(k), _f64(v)
    n, dK = k.shape
    dV = v.shape[1]
    M = feature_dim(dK, P)
    S = np.zeros((dV + 1, M), dtype=np.float64)
    lib = _load()
    if want_y:
        q = _f64(q)
        y = np.zeros((n, dV), dtype=np.float64)
        r = lib.oracle_feature_form(_dp(q), _dp(k), _dp(v), n, dK, dV, P, _dp(y), _dp(S))
    else:
        y = None
        r = lib.oracle_feature_form(None, _dp(k), _dp(v), n, dK, dV, P, None, _dp(S))
    if r < 0:
        raise RuntimeError("oracle_feature_form failed")
    return y, S


def state_rows(k, v, P: int, rows):
    """Rows f of the state of one head: out[r, j] = S[rows[r], j], j <= dV."""
    k, v = _f64(k), _f64(v)
    n, dK = k.shape
    dV = v.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((rows.shape[0], dV + 1), dtype=np.float64)
    r = _load().oracle_state_rows(_dp(k), _dp(v), n, dK, dV, P,
                                  rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  rows.shape[0], _dp(out))
    if r != 0:
        raise RuntimeError("oracle_state_rows failed")
    return out


def softmax(q, k, v):
    """Exact causal softmax attention, fp64 (for the truncation-error report)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, dK = q.shape[-2:]
    dV = v.shape[-1]
    heads = int(np.prod(lead)) if lead else 1
    y = np.zeros(lead + (n, dV), dtype=np.float64)
    _load().oracle_softmax(_dp(q), _dp(k), _dp(v), heads, n, dK, dV, _dp(y))
    return y


def softmax_rows(q, k, v, heads, rows):
    """Sampled rows of the exact causal softmax, fp64: out[r] = y[heads[r], rows[r]].
    q, k: [heads, n, dK]; v: [heads, n, dV] (leading dims flattened)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, dK = q.shape[-2:]
    dV = v.shape[-1]
    q = q.reshape(-1, n, dK)
    k = k.reshape(-1, n, dK)
    v = v.reshape(-1, n, dV)
    heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if heads.shape != rows.shape or heads.ndim != 1:
        raise ValueError("heads and rows must be 1-D of one length")
    if heads.size and (heads.min() < 0 or heads.max() >= q.shape[0] or rows.min() < 0
                       or rows.max() >= n):
        raise ValueError("sampled head or row out of range")
    out = np.zeros((rows.shape[0], dV), dtype=np.float64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    _load().oracle_softmax_rows(_dp(q), _dp(k), _dp(v), n, dK, dV, heads.ctypes.data_as(i64p),
                                rows.ctypes.data_as(i64p), rows.shape[0], _dp(out))
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# --------------------------------------------------------------------------
# Closed forms of [TA Size]
# --------------------------------------------------------------------------

def state_elems_term(d_K: int, d_V: int, p: int) -> int:
    """(d_V + 1) binom(d_K + p - 1, p): state of one Taylor term."""
    return (d_V + 1) * math.comb(d_K + p - 1, p)


def state_elems(d_K: int, d_V: int, P: int) -> int:
    """(d_V + 1) binom(d_K + P - 1, P - 1): state of all P terms."""
    return (d_V + 1) * math.comb(d_K + P - 1, P - 1)


def flops_term(d_K: int, d_V: int, p: int) -> int:
    """(4 d_V + 2p + 4) binom(d_K + p - 1, p): forward FLOPs/token of one term."""
    return (4 * d_V + 2 * p + 4) * math.comb(d_K + p - 1, p)


def flops_per_token(d_K: int, d_V: int, P: int) -> float:
    """(4 d_V + 2 (P d_K + 1)/(d_K + 1) + 2) binom(d_K + P - 1, P - 1)."""
    return (4 * d_V + 2 * (P * d_K + 1) / (d_K + 1) + 2) * math.comb(d_K + P - 1, P - 1)


# --------------------------------------------------------------------------
# Comparison metric
# --------------------------------------------------------------------------

def row_rel_err(y_test, y_ref) -> np.ndarray:
    """Per row: max_j |y_test - y_ref| / max_j |y_ref| (rows along the last axis)."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.max(np.abs(y_test - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    return num / np.where(den > 0, den, 1.0)
