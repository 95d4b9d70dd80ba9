"""constant_cost_self_amd: SATA causal self-attention on MI355X (gfx950).

The hot path (tables, chunked prefill scan, decode step) is hand-written HIP
behind the C ABI declared in include/sata.h; ``constant_cost_self_amd.sata``
is the thin ctypes binding over it.  The library is loaded on first use, and
every entry point raises if the built HIP library is missing: there is no CPU
fallback.
"""
