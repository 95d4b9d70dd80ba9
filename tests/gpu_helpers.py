"""Helpers for the GPU parity tests: upload seeded inputs, call the C ABI through
the binding, compare with the oracle by the per-row normalised metric (y) and by
the per-degree-block metric (states)."""
from __future__ import annotations

import math
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


def feature_degrees(d_K: int, P: int) -> np.ndarray:
    """Degree p of every feature f of the concatenated order p = 0 .. P-1 (block sizes
    binom(d_K + p - 1, p))."""
    return np.repeat(np.arange(P), [math.comb(d_K + p - 1, p) for p in range(P)])


def _block_err(got, ref, deg, P, joint_values=False) -> float:
    """got, ref: [rows, cols]; per degree block and column, max |got - ref| over the block's
    rows / max |ref| over them; the max over blocks and columns.  joint_values: the value
    columns (all but the last) of a degree block share one scale, the largest |ref| over
    them (the normaliser column keeps its own)."""
    worst = 0.0
    for p in range(P):
        sel = deg == p
        if not sel.any():
            continue
        num = np.max(np.abs(got[sel] - ref[sel]), axis=0)
        den = np.max(np.abs(ref[sel]), axis=0)
        if joint_values:
            den[:-1] = np.max(den[:-1])
        worst = max(worst, float(np.max(num / np.where(den > 0, den, 1.0))))
    return worst


def state_col_err(S_gpu, S_ref, d_K: int, P: int, joint_values: bool = False) -> float:
    """State bar, per Taylor term: for every degree block p (the rows of M_p) and column j,
    max_f |dS[j, f]| / max_f |S_ref[j, f]| over the block's features; the max over blocks
    and columns.  S as [cols, M or M_pad] (padding columns are ignored here; callers check
    that they are zero).  A block's own scale is the reference, so an error in the small
    high-degree rows cannot hide under the large p = 0 row."""
    deg = feature_degrees(d_K, P)
    M = deg.size
    got = np.asarray(S_gpu, dtype=np.float64)[:, :M].T
    ref = np.asarray(S_ref, dtype=np.float64)[:, :M].T
    return _block_err(got, ref, deg, P, joint_values)


def sample_feature_rows(d_K: int, P: int, count: int, seed: int) -> np.ndarray:
    """Rows of the state to check, stratified by degree: the first and last row of every
    degree block and about count / P rows drawn at random within each block."""
    rng = np.random.default_rng(seed)
    sizes = [math.comb(d_K + p - 1, p) for p in range(P)]
    offs = np.concatenate([[0], np.cumsum(sizes)])
    picks = []
    for p in range(P):
        lo, hi = int(offs[p]), int(offs[p + 1])
        picks += [lo, hi - 1]
        k = min(hi - lo, max(count // P, 1))
        picks += list(lo + rng.choice(hi - lo, size=k, replace=False))
    return np.unique(np.asarray(picks, dtype=np.int64))


def sampled_state_err(S_gpu, S_ref_rows, rows, d_K: int, P: int, joint_values: bool = False) -> float:
    """The state bar on sampled rows: S_gpu is one head's [cols, M_pad] state,
    S_ref_rows[r, j] = S[rows[r], j] from the oracle; per degree block of the sampled rows
    and column, max |dS| / max |S_ref| (see state_col_err)."""
    deg = feature_degrees(d_K, P)[np.asarray(rows)]
    got = np.asarray(S_gpu, dtype=np.float64)[:, rows].T
    return _block_err(got, np.asarray(S_ref_rows, dtype=np.float64), deg, P, joint_values)


def state16_layout(d_K: int, d_V: int, P: int):
    """The half-precision state layout of one head as include/sata.h documents it: block
    sizes m_p, block starts hoff[p] (multiples of 64), rows Mh, header bytes, head bytes."""
    m = [math.comb(d_K + p - 1, p) for p in range(P)]
    padded = [(x + 63) // 64 * 64 for x in m]
    hoff = [int(x) for x in np.concatenate([[0], np.cumsum(padded)[:-1]])]
    Mh = int(sum(padded))
    hdr = (8 * P * d_V + 255) // 256 * 256
    head = (hdr + 4 * Mh + 2 * d_V * Mh + 255) // 256 * 256
    return m, hoff, Mh, hdr, head


def state16_read(raw, d_K: int, d_V: int, P: int):
    """One head's half-precision state (its bytes) read on the host from the documented layout:
    returns (S [d_V + 1, M] fp64 in the fp32 state's row order, expo [P, d_V], bound [P, d_V],
    pads_zero) where pads_zero says every row past m_p of every block is 0."""
    m, hoff, Mh, hdr, head = state16_layout(d_K, d_V, P)
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8).reshape(-1)[:head])
    pd = P * d_V
    expo = raw[:4 * pd].view(np.int32).reshape(P, d_V)
    bound = raw[4 * pd:8 * pd].view(np.float32).reshape(P, d_V)
    Z = raw[hdr:hdr + 4 * Mh].view(np.float32)
    V = raw[hdr + 4 * Mh:hdr + 4 * Mh + 2 * d_V * Mh].view(np.float16).reshape(d_V, Mh)
    S = np.zeros((d_V + 1, sum(m)))
    pads_zero = True
    off = 0
    for p in range(P):
        r0, r1, rp = hoff[p], hoff[p] + m[p], hoff[p] + (m[p] + 63) // 64 * 64
        S[:d_V, off:off + m[p]] = V[:, r0:r1].astype(np.float64) * np.ldexp(1.0, expo[p].astype(np.int64))[:, None]
        S[d_V, off:off + m[p]] = Z[r0:r1]
        pads_zero = pads_zero and not V[:, r1:rp].any() and not Z[r1:rp].any()
        off += m[p]
    return S, expo.copy(), bound.copy(), pads_zero


def new_state16(B, H, d_K, d_V, P):
    import torch
    nb = sata.sata_state16_bytes(1, 1, d_K, d_V, P)
    return torch.zeros((B, H, nb), device="cuda:0", dtype=torch.uint8)


__all__ = ["inputs", "oracle", "sata", "TOL_BF16", "TOL_F32", "say", "dev_tensor", "upload",
           "prefill", "new_state", "max_row_err", "state_col_err", "sample_feature_rows",
           "sampled_state_err", "feature_degrees", "state16_layout", "state16_read", "new_state16"]
