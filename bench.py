"""Benchmark of the SATA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long|mid|wide]

One step = one chunked prefill (tables already built) of the workload with the
final state written.  value = prefill tokens/s (B*n/t) of --workload (long).  In the
same run: the prefill of the other two workloads (mid, wide; *_prefill), the batched
decode step (16 sequences x 32 heads, d=64, P=4, fp32 states prefilled with 1024
tokens) over 256 steps and the wide-head decode step (32 heads, d=128, states
prefilled with 16384 tokens) over 128 steps, both reported as state GB/s; and the
measured ceilings (ceilings: an in-place read-modify-write sweep over the decode
state's 6.4 GB, back-to-back fp16 MFMA), against which each roofline also gives
frac_of_measured_ceiling.

Rooflines come from HIP events recorded by libsata around each kernel launch on
its own stream: achieved = algorithmic work per launch / mean launch time.
  prefill scan: flops = B H n (4 d_V + 2 (P d_K + 1)/(d_K + 1) + 2) binom(d_K+P-1, P-1)
                (the forward FLOPs/token closed form of the method), peak = bf16 MFMA
                2.5 PFLOP/s.
  decode:       bytes = 8 (d_V + 1) M per head (fp32 state read + write), peak 8 TB/s.
  decode_f16:   the same decode steps on half-precision states (fp16 value columns, fp32
                normaliser): bytes = (4 d_V + 8) M per head, peak 8 TB/s; likewise
                wide_decode_f16.
  decode_pool:  the same step in its serving form: 16 of a pool of 24 prefilled sequences,
                at seeded scattered slots; bytes and peak as for decode (active heads only).
  two_level:    one head of 65536 tokens (too few slices to fill the CUs): the automatic
                two-level prefill against the one-level scan; flops as for prefill, over
                the scan time (both passes and the prefix sum).
  backward:     (sata_prefill_backward on the Mid shape, fp32 arithmetic, the state
                contractions on the matrix cores) flops = B H n [forward closed form +
                2 M (4 (d_V + 1) + d_V)]: the fp32 forward recompute plus the five state
                contractions of the gradient scans (S . u, S update, R . [v|1], phi(k) R,
                R update); peak = fp32 dense MFMA 157.3 TFLOP/s.
cpu_baseline: the fp64 oracle's fixed-size-state form, timed on the host's cores
on a bounded sample (one head, the first --cpu-tokens tokens); beside it the oracle's
Taylor-versus-exact-softmax error report (taylor_vs_softmax: per-row max and median for
P = 1..5 on one head of each of mid, long and wide; all rows of mid, --softmax-rows rows
spread over the others).
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops_per_token(d_K, d_V, P):
    return (4 * d_V + 2 * (P * d_K + 1) / (d_K + 1) + 2) * math.comb(d_K + P - 1, P - 1)


def traffic_from_profiles(kernel_key, chunks_per_launch=None):
    """Measured HBM bytes per launch from profiles/traffic.json, if the kernel's
    source has not changed since the counters were taken and (for a prefill kernel) the
    launches cover as many chunks as the measured ones; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec["source_sha256"]:
        return None
    if chunks_per_launch is not None and rec.get("chunks_per_launch") != chunks_per_launch:
        return None
    return rec["bytes_per_launch"]


def to_dev(a, dtype):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


WORKSPACE_CAP = 0          # bytes; 0 = the library's default (set from --workspace-gib)
PLANS = {}                 # per workload: how the prefill was cut (segments, workspace)


def bench_prefill(w, steps, warmup):
    import torch
    from constant_cost_self_amd import inputs, sata

    log("prefill %s: generating inputs B=%d H=%d n=%d d=%d" % (w.name, w.B, w.H, w.n, w.d_K))
    x = inputs.prefill_inputs(w)
    q, k, v = (to_dev(x[s], w.dtype) for s in ("q", "k", "v"))
    del x
    t = sata.sata_tables_build(w.d_K, w.P)
    t.set_workspace_limit(WORKSPACE_CAP)
    Mp = sata.sata_state_stride(w.d_K, w.P)
    y = torch.empty((w.B, w.H, w.n, w.d_V), device="cuda:0", dtype=torch.float32)
    state = torch.empty((w.B, w.H, w.d_V + 1, Mp), device="cuda:0", dtype=torch.float32)
    nbytes, nseg, nsub = t.prefill_workspace(w.B, w.H, w.n, w.d_V, chunk=w.chunk,
                                             dtype=sata.SATA_BF16 if w.dtype == "bf16" else sata.SATA_F32)
    log("  plan: %d segment(s), %d sub-segment(s), workspace %.2f GB" % (nseg, nsub, nbytes / 1e9))
    PLANS[w.name] = {"segments": nseg, "sub_segments": nsub, "workspace_gb": nbytes / 1e9}
    t.set_timing(True)
    for i in range(warmup):
        sata.sata_prefill(t, q, k, v, y, state, chunk=w.chunk)
        log("  warmup %d done" % i)
    torch.cuda.synchronize()
    t.read_timing()
    t0 = time.perf_counter()
    for i in range(steps):
        sata.sata_prefill(t, q, k, v, y, state, chunk=w.chunk)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tim = t.read_timing()
    log("  timed %d steps: %.3f s; kernels %s" % (steps, wall, tim))
    t.close()
    del q, k, v, y, state
    torch.cuda.empty_cache()
    return wall, tim


def chunks_per_launch(w):
    """Chunks one scan launch of this workload's prefill covers (the first segment's)."""
    plan = PLANS.get(w.name)
    if not plan or plan["sub_segments"] > 1:
        return None
    nchunks = (w.n + w.chunk - 1) // w.chunk
    return -(-nchunks // plan["segments"])


def prefill_record(w, steps, wall, tim, ceil_tflops):
    """The JSON object of one prefill leg: tokens/s and the scan kernel's roofline."""
    F = flops_per_token(w.d_K, w.d_V, w.P)
    scan_ms, scan_n = tim["scan"]
    alg_total = F * w.B * w.H * w.n * steps
    scan_tflops = alg_total / scan_n / (scan_ms / scan_n * 1e-3) / 1e12
    step_tflops = alg_total / wall / 1e12
    return {
        "workload": "%s prefill: B=%d H=%d n=%d d_K=%d d_V=%d P=%d chunk=%d %s inputs, fp32 state"
                    % (w.name, w.B, w.H, w.n, w.d_K, w.d_V, w.P, w.chunk, w.dtype),
        "value": w.B * w.n / (wall / steps), "unit": "tokens/s", "steps": steps,
        "ms_per_step": wall / steps * 1e3,
        "token_heads_per_s": w.B * w.H * w.n / (wall / steps),
        "roofline": {"bound": "mfma", "achieved": scan_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": scan_tflops / MFMA_BF16_PEAK_TFLOPS,
                     "frac_of_measured_ceiling": scan_tflops / ceil_tflops if ceil_tflops else None,
                     "traffic": traffic_from_profiles("prefill_scan_" + w.name, chunks_per_launch(w)),
                     "kernel": "prefill scan", "launches": scan_n, "ms_per_launch": scan_ms / scan_n,
                     "algorithmic_flops_per_launch": alg_total / scan_n},
        "step": {"tflops": step_tflops, "frac_mfma": step_tflops / MFMA_BF16_PEAK_TFLOPS,
                 "kernels_ms_per_step": {k: v[0] / steps for k, v in tim.items() if v[1]}},
        "plan": PLANS.get(w.name),
    }


def decode_record(w, steps, wall, tim, nbytes, ceil_gbs, label, state16=False):
    dk_ms, dk_n = tim["decode"]
    kern_gbs = nbytes / (dk_ms / dk_n * 1e-3) / 1e9
    form = "half-precision states (fp16 values, fp32 normaliser)" if state16 else "fp32 states"
    traffic_key = ("decode16_step" if state16 else "decode_step") + ("" if w.d_K == 64 else "_" + w.name)
    return {
        "workload": "%s: %d sequences x %d heads, d_K=%d d_V=%d, P=%d, %s (%.3f GB) "
                    "prefilled with %d tokens, %s q,k,v" % (label, w.B, w.H, w.d_K, w.d_V, w.P, form,
                                                          nbytes / 2e9, w.n, w.dtype),
        "value": nbytes * steps / wall / 1e9, "unit": "GB/s", "steps": steps,
        "ms_per_step": wall / steps * 1e3,
        "seq_tokens_per_s": w.B * steps / wall,
        "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kern_gbs / HBM_PEAK_GBS,
                     "frac_of_measured_ceiling": kern_gbs / ceil_gbs if ceil_gbs else None,
                     "traffic": traffic_from_profiles(traffic_key),
                     "kernel": "decode state read-modify-write",
                     "ms_per_launch": dk_ms / dk_n, "algorithmic_bytes_per_launch": nbytes},
        "reduce_ms_per_step": tim["decode_reduce"][0] / max(tim["decode_reduce"][1], 1),
    }


def measure_ceilings(rmw_bytes):
    """Measured ceilings on this device (probe library): the in-place read-modify-write of
    rmw_bytes in one linear sweep (GB/s of read + write traffic), and back-to-back fp16 MFMA
    (TFLOP/s) at the prefill scan's occupancy.  Timed with torch events on torch's stream,
    where the probes are launched."""
    import ctypes
    import torch
    from constant_cost_self_amd import build as hb

    lib = ctypes.CDLL(hb.PROBE_LIB)
    lib.probe_rmw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    lib.probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = torch.cuda.current_stream()
    n = int(rmw_bytes // 16 * 4)
    buf = torch.randn(n, device="cuda:0", dtype=torch.float32)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def rmw():
        assert lib.probe_rmw(buf.data_ptr(), n, 1.0000001, -1e-7, st.cuda_stream) == 0
    ms = timed(rmw, 10)
    rmw_gbs = 8.0 * n / (ms * 1e-3) / 1e9
    del buf
    blocks, iters = 4096, 2048
    out = torch.empty(blocks * 512, device="cuda:0", dtype=torch.float32)

    def mm():
        assert lib.probe_mfma(out.data_ptr(), blocks, iters, st.cuda_stream) == 0
    ms2 = timed(mm, 5)
    mfma_tflops = blocks * 8 * 4 * iters * 16384 / (ms2 * 1e-3) / 1e12
    del out
    torch.cuda.empty_cache()
    log("ceilings: read-modify-write %.0f GB/s over %.2f GB; fp16 MFMA %.0f TFLOP/s" %
        (rmw_gbs, 8.0 * n / 1e9, mfma_tflops))
    return {"hbm_rmw": {"value": rmw_gbs, "unit": "GB/s", "frac_of_peak": rmw_gbs / HBM_PEAK_GBS,
                        "bytes_per_launch": 8.0 * n, "ms_per_launch": ms,
                        "probe": "in-place x = a x + b over %.2f GB (the decode workload's state size), "
                                 "one 16-byte non-temporal load and store per thread" % (4.0 * n / 1e9)},
            "mfma_f16": {"value": mfma_tflops, "unit": "TFLOP/s",
                         "frac_of_peak": mfma_tflops / MFMA_BF16_PEAK_TFLOPS, "ms_per_launch": ms2,
                         "probe": "%d workgroups x 8 waves, 4 independent chains of "
                                  "v_mfma_f32_16x16x32_f16 x %d per wave" % (blocks, iters)}}


def bench_decode(w, steps, warmup, prefill_chunk=64, state16=False):
    """Decode steps over all B x H heads of workload w, states prefilled with its w.n tokens
    (fp32 states, or half-precision ones with state16)."""
    import torch
    from constant_cost_self_amd import inputs, sata

    log("decode %s%s: prefilling %d tokens for %dx%d heads" % (w.name, " (fp16 states)" if state16 else "",
                                                              w.n, w.B, w.H))
    x = inputs.prefill_inputs(w)
    q, k, v = (to_dev(x[s], w.dtype) for s in ("q", "k", "v"))
    t = sata.sata_tables_build(w.d_K, w.P)
    if state16:
        state = torch.zeros((w.B, w.H, sata.sata_state16_bytes(1, 1, w.d_K, w.d_V, w.P)),
                            device="cuda:0", dtype=torch.uint8)
        step = sata.sata_decode_step_f16
    else:
        Mp = sata.sata_state_stride(w.d_K, w.P)
        state = torch.zeros((w.B, w.H, w.d_V + 1, Mp), device="cuda:0", dtype=torch.float32)
        step = sata.sata_decode_step
    y = torch.empty((w.B, w.H, w.n, w.d_V), device="cuda:0", dtype=torch.float32)
    sata.sata_prefill(t, q, k, v, y, state, chunk=prefill_chunk, state16=state16)
    del q, k, v, y, x
    s = inputs.decode_inputs(w, warmup + steps, seed=1)
    qs, ks, vs = (to_dev(s[c], w.dtype) for c in ("q", "k", "v"))
    yd = torch.empty((w.B, w.H, w.d_V), device="cuda:0", dtype=torch.float32)
    torch.cuda.synchronize()
    t.set_timing(True)
    for i in range(warmup):
        step(t, state, qs[i], ks[i], vs[i], yd)
    torch.cuda.synchronize()
    t.read_timing()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        step(t, state, qs[i], ks[i], vs[i], yd)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tim = t.read_timing()
    log("  decode %d steps: %.3f s; kernels %s" % (steps, wall, tim))
    t.close()
    del state
    torch.cuda.empty_cache()
    M = math.comb(w.d_K + w.P - 1, w.P - 1)
    # read + write of every entry: 4-byte fp32 entries, or 2-byte value entries and the
    # 4-byte normaliser column of the half-precision state
    per_entry = (4.0 * w.d_V + 8.0) if state16 else 8.0 * (w.d_V + 1)
    bytes_per_step = per_entry * M * w.B * w.H
    return wall, tim, bytes_per_step


def bench_decode_pool(steps, warmup, pool_size=24, active=16, prefill_chunk=64):
    """Serving-style decode: a preallocated pool of pool_size sequence states (the decode
    workload's heads and sizes, each prefilled with its tokens), stepping a ragged batch of
    `active` sequences whose states sit at seeded, scattered slots of the pool."""
    import numpy as np
    import torch
    from constant_cost_self_amd import inputs, sata

    w = dataclasses.replace(inputs.DECODE, B=pool_size)
    log("decode pool: prefilling %d tokens for %dx%d heads" % (w.n, w.B, w.H))
    x = inputs.prefill_inputs(w)
    q, k, v = (to_dev(x[s], w.dtype) for s in ("q", "k", "v"))
    t = sata.sata_tables_build(w.d_K, w.P)
    Mp = sata.sata_state_stride(w.d_K, w.P)
    pool = torch.zeros((pool_size, w.H, w.d_V + 1, Mp), device="cuda:0", dtype=torch.float32)
    y = torch.empty((w.B, w.H, w.n, w.d_V), device="cuda:0", dtype=torch.float32)
    sata.sata_prefill(t, q, k, v, y, pool, chunk=prefill_chunk)
    del q, k, v, y, x
    slots_h = np.random.default_rng(5).permutation(pool_size)[:active].astype(np.int32)
    slots = torch.from_numpy(slots_h).to("cuda:0")
    s = inputs.decode_inputs(w, warmup + steps, seed=2, B=active)
    qs, ks, vs = (to_dev(s[c], w.dtype) for c in ("q", "k", "v"))
    yd = torch.empty((active, w.H, w.d_V), device="cuda:0", dtype=torch.float32)
    torch.cuda.synchronize()
    t.set_timing(True)
    for i in range(warmup):
        sata.sata_decode_step_pool(t, pool, slots, qs[i], ks[i], vs[i], yd)
    torch.cuda.synchronize()
    t.read_timing()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        sata.sata_decode_step_pool(t, pool, slots, qs[i], ks[i], vs[i], yd)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tim = t.read_timing()
    log("  decode pool %d steps: %.3f s; kernels %s" % (steps, wall, tim))
    t.close()
    M = math.comb(w.d_K + w.P - 1, w.P - 1)
    bytes_per_step = 8.0 * (w.d_V + 1) * M * active * w.H
    return wall, tim, bytes_per_step, w, slots_h


def backward_flops_per_token(d_K, d_V, P):
    M = math.comb(d_K + P - 1, P - 1)
    return flops_per_token(d_K, d_V, P) + 2.0 * M * (4 * (d_V + 1) + d_V)


def bench_two_level(steps, n=65536):
    """One head (B=H=1) of n tokens, d=64 P=4 bf16: the one-level scan against the automatic
    choice (the two-level form, since one head's slices fill under half of the CUs)."""
    import numpy as np
    import torch
    from constant_cost_self_amd import inputs, sata

    x = inputs.draw((1, 1, n, 64), (1, 1, n, 64), "bf16", 0.5, 1.0, 0)
    q, k, v = (to_dev(x[s], "bf16") for s in ("q", "k", "v"))
    y = torch.empty((1, 1, n, 64), device="cuda:0", dtype=torch.float32)
    t = sata.sata_tables_build(64, 4)
    t.set_timing(True)
    out = {}
    for split in (1, 0):
        t.set_prefill_split(split)
        sata.sata_prefill(t, q, k, v, y, None, chunk=64)
        torch.cuda.synchronize()
        t.read_timing()
        t0 = time.perf_counter()
        for i in range(steps):
            sata.sata_prefill(t, q, k, v, y, None, chunk=64)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        tim = t.read_timing()
        out[split] = (wall, tim["scan"][0] / steps)
    t.close()
    log("  two-level: one head n=%d: one-level %.3f ms, automatic %.3f ms" % (n, out[1][0] * 1e3, out[0][0] * 1e3))
    return out


def bench_backward(steps, warmup):
    import numpy as np
    import torch
    from constant_cost_self_amd import inputs, sata

    w = inputs.MID
    log("backward: %s shape B=%d H=%d n=%d d=%d" % (w.name, w.B, w.H, w.n, w.d_K))
    x = inputs.prefill_inputs(w)
    q, k, v = (to_dev(x[s], w.dtype) for s in ("q", "k", "v"))
    dy = to_dev(np.random.default_rng(7).standard_normal((w.B, w.H, w.n, w.d_V)).astype(np.float32), "f32")
    dq = torch.empty((w.B, w.H, w.n, w.d_K), device="cuda:0", dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty((w.B, w.H, w.n, w.d_V), device="cuda:0", dtype=torch.float32)
    t = sata.sata_tables_build(w.d_K, w.P)
    t.set_timing(True)
    for i in range(warmup):
        sata.sata_prefill_backward(t, q, k, v, dy, dq, dk, dv, chunk=w.chunk)
    torch.cuda.synchronize()
    t.read_timing()
    t0 = time.perf_counter()
    for i in range(steps):
        sata.sata_prefill_backward(t, q, k, v, dy, dq, dk, dv, chunk=w.chunk)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tim = t.read_timing()
    log("  backward %d steps: %.3f s; kernels %s" % (steps, wall, tim))
    t.close()
    return wall, tim, w


def taylor_vs_softmax(nrows):
    """The truncation error the pages describe as close to float16 resolution at P = 4: per-row
    max_j |y_taylor - y_softmax| / max_j |y_softmax| of the oracle's truncated-kernel attention
    against its exact causal softmax, for one head drawn by each workload's recipe (its own
    input scale and length): every row of a Mid head (n = 4096), nrows rows spread over a Long
    head (n = 65536) and over a Wide head (n = 16384).  P = 1 .. 5.  Reported, not gated: the
    pages give no metric."""
    import numpy as np
    import oracle
    from constant_cost_self_amd import inputs

    out = {}
    for w in (inputs.MID, inputs.LONG, inputs.WIDE):
        x = inputs.prefill_inputs(w, B=1, H=1)
        q, k, v = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0]
        if w.n <= 4096:
            rows = np.arange(w.n)
        else:
            rows = np.unique(np.linspace(0, w.n - 1, nrows).astype(np.int64))
        heads = np.zeros_like(rows)
        ys = oracle.softmax_rows(q[None], k[None], v[None], heads, rows)
        rec = {"d_K": w.d_K, "sigma_qk": w.sigma_qk, "n": w.n, "rows": int(rows.size)}
        for P in (1, 2, 3, 4, 5):
            e = oracle.row_rel_err(oracle.direct_rows(q[None], k[None], v[None], P, heads, rows), ys)
            rec["P=%d" % P] = {"max": float(np.max(e)), "median": float(np.median(e))}
        out[w.name] = rec
        log("  taylor vs softmax, %s: P=4 max %.2e median %.2e" % (w.name, rec["P=4"]["max"],
                                                                   rec["P=4"]["median"]))
    return out


def cpu_baseline(w, ntok, softmax_rows):
    """The oracle's fixed-size-state form on head (0, 0), first ntok tokens; and, beside it,
    the oracle's Taylor-versus-softmax error report."""
    import oracle
    from constant_cost_self_amd import inputs

    x = inputs.prefill_inputs(w, n=ntok, B=1, H=1)
    q, k, v = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0]
    oracle.feature_form(q[:4], k[:4], v[:4], w.P)         # load + warm the library
    t0 = time.perf_counter()
    oracle.feature_form(q, k, v, w.P)
    dt = time.perf_counter() - t0
    heads_per_token = w.H            # a token of the workload spans all H heads of a batch row
    rec = {"value": ntok / dt / heads_per_token, "unit": "tokens/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": "fp64 oracle, fixed-size-state form (state update + readout per token), "
                     "head (0,0) of the %s workload, first %d tokens, %.1f s; scaled to tokens "
                     "of all %d heads" % (w.name, ntok, dt, w.H),
           "seconds": dt}
    if softmax_rows:
        rec["taylor_vs_softmax"] = taylor_vs_softmax(softmax_rows)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long", choices=["long", "mid", "wide"])
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the prefill legs of the workloads other than --workload")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--workspace-gib", type=float, default=0.0,
                    help="workspace cap of the prefill legs (0: the library's default, 32 GiB; "
                         "64 runs the Long prefill as one segment of 1024 chunks instead of two "
                         "of 512, which measured the same within the boxes' spread)")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--softmax-rows", type=int, default=512)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-two-level", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "decode16", "backward"], default=None,
                    help="time one part only (for profiler runs)")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB, 3 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the path is single-GPU (heads shard across GPUs "
              "with no communication, so N GPUs run N independent copies); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from constant_cost_self_amd import inputs, sata

    global WORKSPACE_CAP
    WORKSPACE_CAP = int(args.workspace_gib * (1 << 30))
    sata.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_only:
        n = args.copy_only * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4}))
        return
    w = inputs.WORKLOADS[args.workload]
    if args.only == "backward":
        bwall, btim, bw = bench_backward(args.backward_steps, 1)
        print(json.dumps({"backward_ms": btim["backward"][0] / btim["backward"][1],
                          "backward_step_ms": bwall / args.backward_steps * 1e3}))
        return
    if args.only in ("decode", "decode16"):
        dw = inputs.DECODE if w.d_K == 64 else inputs.WIDE
        dwall, dtim, dbytes = bench_decode(dw, args.decode_steps, args.decode_warmup,
                                           state16=args.only == "decode16")
        dk_ms, dk_n = dtim["decode"]
        print(json.dumps({"decode_kernel_gbs": dbytes / (dk_ms / dk_n * 1e-3) / 1e9,
                          "decode_step_ms": dwall / args.decode_steps * 1e3}))
        return

    ceil = None
    if not args.no_ceilings and args.only is None:
        M = math.comb(inputs.DECODE.d_K + inputs.DECODE.P - 1, inputs.DECODE.P - 1)
        ceil = measure_ceilings(4.0 * (inputs.DECODE.d_V + 1) * M * inputs.DECODE.B * inputs.DECODE.H)
    ceil_tflops = ceil["mfma_f16"]["value"] if ceil else None
    ceil_gbs = ceil["hbm_rmw"]["value"] if ceil else None

    wall, tim = bench_prefill(w, args.steps, args.warmup)
    rec = prefill_record(w, args.steps, wall, tim, ceil_tflops)
    out = {
        "metric": "prefill tokens/s (d=64,P=4) + decode state GB/s; % of MFMA/HBM peak",
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded i.i.d. Gaussian q,k,v; no dataset, no weights)",
        "config": {"workload": rec["workload"],
                   "B": w.B, "H": w.H, "n": w.n, "d_K": w.d_K, "d_V": w.d_V, "P": w.P,
                   "chunk": w.chunk},
        "roofline": rec["roofline"],
        "prefill_step": dict(rec["step"], token_heads_per_s=rec["token_heads_per_s"], plan=rec["plan"]),
    }
    if ceil:
        out["ceilings"] = ceil

    if not args.no_other_prefill and args.only is None:
        for ow in (inputs.MID, inputs.LONG, inputs.WIDE):
            if ow.name == w.name:
                continue
            steps = 20 if ow is inputs.MID else args.steps
            owall, otim = bench_prefill(ow, steps, args.warmup)
            out[ow.name + "_prefill"] = prefill_record(ow, steps, owall, otim, ceil_tflops)

    if not args.no_decode and args.only is None:
        dwall, dtim, dbytes = bench_decode(inputs.DECODE, args.decode_steps, args.decode_warmup)
        out["decode"] = decode_record(inputs.DECODE, args.decode_steps, dwall, dtim, dbytes, ceil_gbs,
                                      "decode step")
        wsteps = inputs.WIDE_DECODE_STEPS
        wwall, wtim, wbytes = bench_decode(inputs.WIDE, wsteps, args.decode_warmup)
        out["wide_decode"] = decode_record(inputs.WIDE, wsteps, wwall, wtim, wbytes, ceil_gbs,
                                           "wide-head decode step")
        hwall, htim, hbytes = bench_decode(inputs.DECODE, args.decode_steps, args.decode_warmup, state16=True)
        out["decode_f16"] = decode_record(inputs.DECODE, args.decode_steps, hwall, htim, hbytes, ceil_gbs,
                                          "decode step", state16=True)
        out["decode_f16"]["speedup_vs_fp32_state"] = dwall / hwall
        hwall, htim, hbytes = bench_decode(inputs.WIDE, wsteps, args.decode_warmup, state16=True)
        out["wide_decode_f16"] = decode_record(inputs.WIDE, wsteps, hwall, htim, hbytes, ceil_gbs,
                                               "wide-head decode step", state16=True)
        out["wide_decode_f16"]["speedup_vs_fp32_state"] = wwall / hwall

    if not args.no_decode and args.only is None:
        pwall, ptim, pbytes, pw, pslots = bench_decode_pool(args.decode_steps, args.decode_warmup)
        pk_ms, pk_n = ptim["decode"]
        pk_gbs = pbytes / (pk_ms / pk_n * 1e-3) / 1e9
        out["decode_pool"] = {
            "workload": "serving-style decode step: %d of %d pooled sequences (slots %s) x %d heads, "
                        "d_K=d_V=%d, P=%d, fp32 states prefilled with %d tokens, %s q,k,v" %
                        (len(pslots), pw.B, ",".join(str(int(v)) for v in pslots), pw.H, pw.d_K,
                         pw.P, pw.n, pw.dtype),
            "value": pbytes * args.decode_steps / pwall / 1e9, "unit": "GB/s",
            "steps": args.decode_steps, "ms_per_step": pwall / args.decode_steps * 1e3,
            "roofline": {"bound": "hbm", "achieved": pk_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": pk_gbs / HBM_PEAK_GBS,
                         "frac_of_measured_ceiling": pk_gbs / ceil_gbs if ceil_gbs else None,
                         "traffic": None,
                         "kernel": "decode state read-modify-write (pool form)",
                         "ms_per_launch": pk_ms / pk_n, "algorithmic_bytes_per_launch": pbytes},
        }

    if not args.no_two_level and args.only is None:
        n2 = 65536
        tl = bench_two_level(5, n2)
        fl = flops_per_token(64, 64, 4) * n2
        out["two_level"] = {
            "workload": "prefill of one head (B=H=1) n=%d d_K=d_V=64 P=4 chunk=64, bf16: the automatic "
                        "two-level form (sub-segments scanned in parallel) against one level" % n2,
            "value": n2 / tl[0][0], "unit": "tokens/s", "ms_per_step": tl[0][0] * 1e3,
            "one_level_ms_per_step": tl[1][0] * 1e3, "speedup": tl[1][0] / tl[0][0],
            "roofline": {"bound": "mfma", "achieved": fl / (tl[0][1] * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": fl / (tl[0][1] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": None, "kernel": "prefill scan (both passes and the prefix sum)",
                         "ms_per_launch": tl[0][1], "algorithmic_flops_per_launch": fl},
        }

    if not args.no_backward and args.only is None:
        bwall, btim, bw = bench_backward(args.backward_steps, 1)
        b_ms, b_n = btim["backward"]
        bflops = backward_flops_per_token(bw.d_K, bw.d_V, bw.P) * bw.B * bw.H * bw.n
        b_tflops = bflops / (b_ms / b_n * 1e-3) / 1e12
        out["backward"] = {
            "workload": "prefill backward (dq, dk, dv for dL/dy = dy): B=%d H=%d n=%d d_K=d_V=%d "
                        "P=%d chunk=%d, %s q,k,v, fp32 dy; fp32 arithmetic" %
                        (bw.B, bw.H, bw.n, bw.d_K, bw.P, bw.chunk, bw.dtype),
            "value": bw.B * bw.n / (bwall / args.backward_steps), "unit": "tokens/s",
            "steps": args.backward_steps, "ms_per_step": bwall / args.backward_steps * 1e3,
            "roofline": {"bound": "mfma", "achieved": b_tflops, "peak": MFMA_FP32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": b_tflops / MFMA_FP32_PEAK_TFLOPS,
                         "traffic": None, "kernel": "prefill backward (all kernels of one call)",
                         "ms_per_launch": b_ms / b_n, "algorithmic_flops_per_launch": bflops},
        }

    if not args.no_cpu and args.only is None:
        log("cpu baseline: oracle on %d tokens" % args.cpu_tokens)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens, args.softmax_rows)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
