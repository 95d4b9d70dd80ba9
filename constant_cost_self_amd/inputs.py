"""Seeded synthetic inputs for SATA causal self-attention.

This module holds NO arithmetic of the method: it only draws Gaussian arrays,
rounds them to bfloat16 when a workload says so, and names the workloads.  It is
the one piece of Python that both the oracle-based tests and the HIP path use.

Recipe (the same everywhere): ``numpy.random.default_rng(seed)`` (PCG64), arrays
drawn in the order q, k, v with ``standard_normal(shape, dtype=float32) * sigma``,
then rounded to bfloat16 (round to nearest, ties to even) for bf16 workloads.
The oracle always reads the stored values (the bf16 or fp32 bits upcast to fp64),
so parity does not depend on the generator.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def bf16_round(x: np.ndarray):
    """Round float32 to bfloat16, nearest-even.  Returns (uint16 bits, float32 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    vals = (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return r, vals


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload (shapes and distributions, no method data)."""
    name: str
    B: int
    H: int
    n: int
    d_K: int
    d_V: int
    P: int
    chunk: int
    dtype: str          # "f32" or "bf16"
    sigma_qk: float
    sigma_v: float
    seed: int = 0


# Workloads of the method's d=8/64/128, P=4 regimes.  Inputs are i.i.d. Gaussian
# with no structure; "decode" prefills 1024 tokens and then steps.
TINY = Workload("tiny", 1, 1, 256, 8, 8, 4, 16, "f32", 1.0, 1.0)
MID = Workload("mid", 1, 8, 4096, 64, 64, 4, 64, "bf16", 0.5, 1.0)
LONG = Workload("long", 4, 16, 65536, 64, 64, 4, 64, "bf16", 0.5, 1.0)
DECODE = Workload("decode", 16, 32, 1024, 64, 64, 4, 64, "bf16", 0.5, 1.0)
WIDE = Workload("wide", 1, 32, 16384, 128, 128, 4, 64, "bf16", 0.35, 1.0)
DECODE_STEPS = 256
WIDE_DECODE_STEPS = 128

WORKLOADS = {w.name: w for w in (TINY, MID, LONG, DECODE, WIDE)}


def draw(shape_qk, shape_v, dtype: str, sigma_qk: float, sigma_v: float, seed: int):
    """Draw q, k, v.  Returns dict with float32 values ('q','k','v') and, for
    bf16, the raw uint16 bits ('q_bits', 'k_bits', 'v_bits')."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape_qk, dtype=np.float32) * np.float32(sigma_qk)
    k = rng.standard_normal(shape_qk, dtype=np.float32) * np.float32(sigma_qk)
    v = rng.standard_normal(shape_v, dtype=np.float32) * np.float32(sigma_v)
    out = {}
    if dtype == "bf16":
        for name, a in (("q", q), ("k", k), ("v", v)):
            bits, vals = bf16_round(a)
            out[name] = vals
            out[name + "_bits"] = bits
    elif dtype == "f32":
        out.update(q=q, k=k, v=v)
    else:
        raise ValueError(dtype)
    return out


def prefill_inputs(w: Workload, n: int | None = None, B: int | None = None,
                   H: int | None = None, seed: int | None = None):
    """q, k: [B, H, n, d_K]; v: [B, H, n, d_V] for workload w (sizes overridable)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    n = w.n if n is None else n
    seed = w.seed if seed is None else seed
    return draw((B, H, n, w.d_K), (B, H, n, w.d_V), w.dtype, w.sigma_qk, w.sigma_v, seed)


def decode_inputs(w: Workload, steps: int, seed: int = 1, B: int | None = None,
                  H: int | None = None):
    """Per-step q, k: [steps, B, H, d_K]; v: [steps, B, H, d_V], one draw per tensor."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    return draw((steps, B, H, w.d_K), (steps, B, H, w.d_V), w.dtype,
                w.sigma_qk, w.sigma_v, seed)
