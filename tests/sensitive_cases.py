"""Inputs at which the highest Taylor term of each P moves y far beyond the parity bar.

With small q, k the top term alpha_{P-1} (q.k)^{P-1} is tiny, so a test at such scales
passes even when that term is wrong or missing.  The scales below make dropping it move y
by at least 10 x the 2e-2 bar on the rows each test checks, while the denominators stay
well away from zero (checked on the CPU by tests/test_sensitivity_cpu.py).  Only shapes,
seeds and scales live here; the inputs come from constant_cost_self_amd.inputs.draw.
"""
from constant_cost_self_amd import inputs

# q, k standard deviation per (d_K, P); v ~ N(0, 1)
SIGMA = {(64, 2): 0.75, (64, 3): 0.75, (64, 4): 0.75, (64, 5): 0.9,
         (128, 3): 0.8, (128, 4): 0.8, (128, 5): 0.9}

# (d, P, n, seed): one-level prefill, B = 1, H = 2, every row checked
ONE_LEVEL = [(64, 3, 700, 71), (64, 4, 700, 72), (64, 5, 700, 73),
             (128, 3, 300, 74), (128, 4, 300, 75), (128, 5, 300, 76)]
# (d, P, n, seed, nsub): forced two-level prefill, B = 1, H = 2, every row checked
TWO_LEVEL = [(64, 3, 1500, 81, 3), (64, 4, 1500, 82, 3), (64, 5, 1500, 83, 3),
             (128, 4, 700, 84, 3)]
# (d, P, n1, n2, seed): prefill(n1), then prefill(n2) continued from its state; rows n1..
CONTINUE = [(64, 4, 700, 500, 91), (128, 4, 300, 200, 92)]
# (d, P, n1, steps, seed, sigma): prefill(n1), then decode steps; the decode rows are
# checked (few rows, each an average over a short prefix: their own scales)
DECODE = [(64, 3, 200, 16, 207, 0.75), (64, 4, 400, 16, 211, 0.85), (64, 5, 200, 16, 208, 0.9),
          (128, 4, 150, 16, 209, 0.8)]
# the Mid shape (B=1, H=8, n=4096, d=64, P=4) at the sensitive scale, every row checked
MID_SHAPE = (1, 8, 4096, 64, 4, 111)
# the Long shape (B=4, H=16, n=65536, d=64, P=4), sampled rows past 4096 (averages over
# many tokens: a larger scale), plus head (0, 0) in full over its first 4096 rows
LONG_SHAPE = (4, 16, 65536, 64, 4, 112)
LONG_SIGMA = 0.85


def draw(d, P, B, H, n, seed, sigma=None):
    sigma = SIGMA[(d, P)] if sigma is None else sigma
    return inputs.draw((B, H, n, d), (B, H, n, d), "bf16", sigma, 1.0, seed)


def long_rows(n, seed, count=3):
    """Sampled (head, row) pairs of the Long-shape case: for every head, rows past 4096."""
    import numpy as np
    rng = np.random.default_rng(seed)
    B, H = LONG_SHAPE[0], LONG_SHAPE[1]
    pos = np.unique(np.concatenate([[4096, n - 1], rng.integers(4096, n, size=count)]))
    heads = np.repeat(np.arange(B * H), pos.size)
    return heads, np.tile(pos, B * H)
