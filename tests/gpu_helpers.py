"""Helpers for the GPU parity tests: upload seeded inputs, call the C ABI through
the binding, compare with the oracle by the per-row normalised metric."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from constant_cost_self_amd import inputs, sata

TOL_BF16 = 2e-2     # bf16 inputs, fp32 state: max_T max_j|dy| / max_j|y_ref|
TOL_F32 = 1e-5      # fp32 path


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(a, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def upload(x, dtype: str):
    return tuple(dev_tensor(x[s], dtype) for s in ("q", "k", "v"))


def prefill(t, q, k, v, chunk, state=None, continue_state=False):
    import torch
    B, H, n, _ = q.shape
    d_V = v.shape[-1]
    y = torch.full((B, H, n, d_V), float("nan"), device="cuda:0", dtype=torch.float32)
    sata.sata_prefill(t, q, k, v, y, state, chunk=chunk, continue_state=continue_state)
    return y


def new_state(B, H, d_K, d_V, P):
    import torch
    Mp = sata.sata_state_stride(d_K, P)
    return torch.zeros((B, H, d_V + 1, Mp), device="cuda:0", dtype=torch.float32)


def max_row_err(y_gpu, y_ref) -> float:
    return float(np.max(oracle.row_rel_err(np.asarray(y_gpu, dtype=np.float64), y_ref)))


def state_col_err(S_gpu, S_ref) -> float:
    """max over columns j of max_f |dS[j,f]| / max_f |S_ref[j,f]|; S as [cols, M]."""
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    num = np.max(np.abs(S_gpu - S_ref), axis=1)
    den = np.max(np.abs(S_ref), axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def sample_feature_rows(M: int, count: int, seed: int) -> np.ndarray:
    """Rows of the state to check: the first few (p = 0 and degree-1 features), the
    last two, and `count` drawn at random."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, M - 2, M - 1]
    return np.unique(np.concatenate([fixed, rng.choice(M, size=count, replace=False)]))


def sampled_state_err(S_gpu, S_ref_rows, rows) -> float:
    """The state bound on sampled rows: S_gpu is one head's [cols, M_pad] state,
    S_ref_rows[r, j] = S[rows[r], j] from the oracle.  max over columns j of
    max_r |dS| / max_r |S_ref| (row 0, the largest row, is always sampled)."""
    got = np.asarray(S_gpu, dtype=np.float64)[:, rows].T
    num = np.max(np.abs(got - S_ref_rows), axis=0)
    den = np.max(np.abs(S_ref_rows), axis=0)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


__all__ = ["inputs", "oracle", "sata", "TOL_BF16", "TOL_F32", "say", "dev_tensor", "upload",
           "prefill", "new_state", "max_row_err", "state_col_err", "sample_feature_rows",
           "sampled_state_err"]
