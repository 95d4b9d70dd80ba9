"""Thin ctypes binding of libsata (include/sata.h).

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI.  PyTorch supplies device memory and the stream.  The functions keep
the C names; tensors are passed as torch tensors (their data pointers) and the
stream defaults to torch's current stream.  If the built library is missing the
first call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libsata.so")

SATA_F32 = 0
SATA_BF16 = 1
SATA_PREFILL_CONTINUE = 1
SATA_STATE_F16 = 2
SATA_OK = 0
SATA_ERR_ARG = -1
SATA_ERR_UNSUPPORTED = -2
SATA_ERR_ALIGN = -3
SATA_ERR_HIP = -4
SATA_ERR_OOM = -5

EXPORTED = ("sata_tables_build", "sata_tables_build_host", "sata_tables_get", "sata_tables_free", "sata_feature_dim",
            "sata_state_stride", "sata_state_bytes", "sata_prefill", "sata_decode_step",
            "sata_decode_step_pool", "sata_prefill_backward",
            "sata_last_error", "sata_set_workspace_limit", "sata_set_prefill_split", "sata_set_timing",
            "sata_read_timing", "sata_prefill_workspace", "sata_decode_workspace",
            "sata_reserve_workspace", "sata_decode_step_noalloc", "sata_state16_stride",
            "sata_state16_bytes", "sata_state_pack_f16", "sata_state_unpack_f16",
            "sata_decode_step_f16", "sata_decode_step_pool_f16")
KERNELS = ("scan", "finalize", "decode", "decode_reduce", "backward", "prep", "convert")

_lib = None


class SataError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("sata error %d: %s" % (code, msg))
        self.code = code


def load():
    """Load libsata.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsata.so is not built (%s); run __graft_entry__.build() or "
                           "python -m constant_cost_self_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.sata_tables_build.restype = i32
    lib.sata_tables_build.argtypes = [i32, i32, ctypes.POINTER(vp)]
    lib.sata_tables_build_host.restype = i32
    lib.sata_tables_build_host.argtypes = [i32, i32, ctypes.POINTER(vp)]
    lib.sata_tables_get.restype = i32
    lib.sata_tables_get.argtypes = [vp, i32, ctypes.POINTER(ctypes.POINTER(ctypes.c_int32)),
                                    ctypes.POINTER(ctypes.POINTER(ctypes.c_int32)),
                                    ctypes.POINTER(i64)]
    lib.sata_tables_free.restype = None
    lib.sata_tables_free.argtypes = [vp]
    lib.sata_feature_dim.restype = i64
    lib.sata_feature_dim.argtypes = [i32, i32]
    lib.sata_state_stride.restype = i64
    lib.sata_state_stride.argtypes = [i32, i32]
    lib.sata_state_bytes.restype = i64
    lib.sata_state_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sata_prefill.restype = i32
    lib.sata_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                 i32, i32, vp]
    lib.sata_decode_step.restype = i32
    lib.sata_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.sata_decode_step_noalloc.restype = i32
    lib.sata_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.sata_decode_step_pool.restype = i32
    lib.sata_decode_step_pool.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.sata_prefill_backward.restype = i32
    lib.sata_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                          i32, i32, i32, i32, vp]
    lib.sata_last_error.restype = ctypes.c_char_p
    lib.sata_last_error.argtypes = []
    lib.sata_set_workspace_limit.restype = i32
    lib.sata_set_workspace_limit.argtypes = [vp, i64]
    lib.sata_set_prefill_split.restype = i32
    lib.sata_set_prefill_split.argtypes = [vp, i32]
    lib.sata_set_timing.restype = i32
    lib.sata_set_timing.argtypes = [vp, i32]
    lib.sata_prefill_workspace.restype = i32
    lib.sata_prefill_workspace.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                           ctypes.POINTER(i64), ctypes.POINTER(i32),
                                           ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.sata_decode_workspace.restype = i32
    lib.sata_decode_workspace.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i64)]
    lib.sata_reserve_workspace.restype = i32
    lib.sata_reserve_workspace.argtypes = [vp, i64, vp]
    lib.sata_state16_stride.restype = i64
    lib.sata_state16_stride.argtypes = [i32, i32]
    lib.sata_state16_bytes.restype = i64
    lib.sata_state16_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sata_state_pack_f16.restype = i32
    lib.sata_state_pack_f16.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.sata_state_unpack_f16.restype = i32
    lib.sata_state_unpack_f16.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.sata_decode_step_f16.restype = i32
    lib.sata_decode_step_f16.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.sata_decode_step_pool_f16.restype = i32
    lib.sata_decode_step_pool_f16.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, vp, i32, i32, i32,
                                              i32, i32, vp]
    lib.sata_read_timing.restype = i32
    lib.sata_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    _lib = lib
    return lib


def last_error() -> str:
    return load().sata_last_error().decode()


def _check(rc: int):
    if rc != SATA_OK:
        raise SataError(rc, last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(*tensors):
    for t in tensors:
        if t is not None and not isinstance(t, int) and not t.is_contiguous():
            raise ValueError("tensors passed to libsata must be contiguous")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SATA_F32
    if t.dtype == torch.bfloat16:
        return SATA_BF16
    raise TypeError("inputs must be float32 or bfloat16, got %s" % t.dtype)


# --------------------------------------------------------------------------
# Size helpers
# --------------------------------------------------------------------------

def sata_feature_dim(d_K: int, P: int) -> int:
    return int(load().sata_feature_dim(d_K, P))


def sata_state_stride(d_K: int, P: int) -> int:
    return int(load().sata_state_stride(d_K, P))


def sata_state_bytes(B: int, H: int, d_K: int, d_V: int, P: int) -> int:
    return int(load().sata_state_bytes(B, H, d_K, d_V, P))


def sata_state16_stride(d_K: int, P: int) -> int:
    """Rows Mh of the half-precision state (degree blocks starting on multiples of 64)."""
    return int(load().sata_state16_stride(d_K, P))


def sata_state16_bytes(B: int, H: int, d_K: int, d_V: int, P: int) -> int:
    return int(load().sata_state16_bytes(B, H, d_K, d_V, P))


# --------------------------------------------------------------------------
# Tables
# --------------------------------------------------------------------------

class Tables:
    """Owner of a sata_tables handle (freed on close() or garbage collection)."""

    def __init__(self, handle: int, d_K: int, P: int):
        self.handle = handle
        self.d_K = d_K
        self.P = P

    def get(self, p: int):
        """Host copies of (M_p [m_p, p] int32, C_p [m_p] int32) as numpy arrays."""
        import numpy as np
        M = ctypes.POINTER(ctypes.c_int32)()
        C = ctypes.POINTER(ctypes.c_int32)()
        m = ctypes.c_int64()
        _check(load().sata_tables_get(self.handle, p, ctypes.byref(M), ctypes.byref(C),
                                      ctypes.byref(m)))
        mp = m.value
        Mnp = (np.ctypeslib.as_array(M, shape=(mp * p,)).reshape(mp, p).copy()
               if p > 0 else np.zeros((mp, 0), dtype=np.int32))
        Cnp = np.ctypeslib.as_array(C, shape=(mp,)).copy()
        return Mnp, Cnp

    def set_workspace_limit(self, nbytes: int):
        _check(load().sata_set_workspace_limit(self.handle, nbytes))

    def set_prefill_split(self, nsub: int):
        """Sub-segments of the two-level prefill: 0 automatic, 1 never, k >= 2 forced."""
        _check(load().sata_set_prefill_split(self.handle, nsub))

    def prefill_workspace(self, B: int, H: int, n: int, d_V: int, *, chunk: int = 64,
                          dtype: int = SATA_BF16, continue_state: bool = False,
                          with_state: bool = True, segment_chunks: bool = False,
                          state16: bool = False):
        """(workspace bytes, one-level segments, two-level sub-segments) of a prefill;
        with segment_chunks=True also the segments' length in chunks (a 4-tuple)."""
        nb = ctypes.c_int64()
        seg = ctypes.c_int()
        segc = ctypes.c_int()
        sub = ctypes.c_int()
        flags = (SATA_PREFILL_CONTINUE if continue_state else 0) | (SATA_STATE_F16 if state16 else 0)
        _check(load().sata_prefill_workspace(self.handle, B, H, n, self.d_K, d_V, self.P, chunk,
                                             dtype, flags, 1 if with_state else 0, ctypes.byref(nb),
                                             ctypes.byref(seg), ctypes.byref(segc), ctypes.byref(sub)))
        if segment_chunks:
            return nb.value, seg.value, sub.value, segc.value
        return nb.value, seg.value, sub.value

    def decode_workspace(self, B: int, H: int, d_V: int) -> int:
        nb = ctypes.c_int64()
        _check(load().sata_decode_workspace(self.handle, B, H, d_V, ctypes.byref(nb)))
        return nb.value

    def reserve_workspace(self, nbytes: int, stream=None):
        _check(load().sata_reserve_workspace(self.handle, nbytes, _stream(stream)))

    def set_timing(self, enable: bool):
        _check(load().sata_set_timing(self.handle, 1 if enable else 0))

    def read_timing(self):
        """{kernel: (summed ms, launches)} since the previous read (waits for them)."""
        n = len(KERNELS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(load().sata_read_timing(self.handle, ms, cnt))
        return {KERNELS[i]: (ms[i], cnt[i]) for i in range(n)}

    def close(self):
        if self.handle:
            load().sata_tables_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sata_tables_build(d_K: int, P: int) -> Tables:
    h = ctypes.c_void_p()
    _check(load().sata_tables_build(d_K, P, ctypes.byref(h)))
    return Tables(h.value, d_K, P)


def sata_tables_build_host(d_K: int, P: int) -> Tables:
    """Host-only handle (no GPU needed): table inspection and argument checks."""
    h = ctypes.c_void_p()
    _check(load().sata_tables_build_host(d_K, P, ctypes.byref(h)))
    return Tables(h.value, d_K, P)


# --------------------------------------------------------------------------
# Hot path
# --------------------------------------------------------------------------

def sata_prefill(t: Tables, q, k, v, y, state=None, *, chunk: int = 64,
                 continue_state: bool = False, state16: bool = False, stream=None):
    """Chunked causal prefill.  q, k: [B, H, n, d_K]; v: [B, H, n, d_V] (fp32 or
    bf16, contiguous, on the GPU); y: fp32 [B, H, n, d_V]; state: optional fp32
    [B, H, d_V + 1, M_pad], or with state16=True a half-precision state (uint8
    [B, H, sata_state16_bytes(1, 1, ...)])."""
    _need(q, k, v, y, state)
    B, H, n, d_K = q.shape
    d_V = v.shape[-1]
    flags = (SATA_PREFILL_CONTINUE if continue_state else 0) | (SATA_STATE_F16 if state16 else 0)
    _check(load().sata_prefill(t.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(state),
                               B, H, n, d_K, d_V, t.P, chunk, _dtype_code(q), flags,
                               _stream(stream)))


def sata_prefill_backward(t: Tables, q, k, v, dy, dq, dk, dv, *, chunk: int = 64, stream=None):
    """Gradients of the causal prefill for dL/dy = dy.  q, k, v as for sata_prefill;
    dy: fp32 [B, H, n, d_V]; dq, dk: fp32 [B, H, n, d_K] and dv: fp32 [B, H, n, d_V],
    written."""
    _need(q, k, v, dy, dq, dk, dv)
    B, H, n, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_prefill_backward(t.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(dy), _ptr(dq),
                                        _ptr(dk), _ptr(dv), B, H, n, d_K, d_V, t.P, chunk,
                                        _dtype_code(q), _stream(stream)))


def sata_decode_step(t: Tables, state, q, k, v, y, *, stream=None):
    """One decode step.  q, k: [B, H, d_K]; v: [B, H, d_V]; y: fp32 [B, H, d_V];
    state: fp32 [B, H, d_V + 1, M_pad], updated in place."""
    _need(state, q, k, v, y)
    B, H, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_decode_step(t.handle, _ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(y),
                                   B, H, d_K, d_V, t.P, _dtype_code(q), _stream(stream)))


def sata_decode_step_noalloc(t: Tables, state, q, k, v, y, *, stream=None):
    """sata_decode_step without any allocation (partials in the library's fixed 16 MiB
    device scratch; calls overlapping on one GPU race)."""
    _need(state, q, k, v, y)
    B, H, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_decode_step_noalloc(t.handle, _ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(y),
                                           B, H, d_K, d_V, t.P, _dtype_code(q), _stream(stream)))


def sata_decode_step_pool(t: Tables, pool, slots, q, k, v, y, *, stream=None):
    """Decode step over a state pool.  pool: fp32 [pool_size, H, d_V + 1, M_pad];
    slots: int32 [count] on the device; q, k: [count, H, d_K]; v: [count, H, d_V];
    y: fp32 [count, H, d_V]."""
    _need(pool, slots, q, k, v, y)
    count, H, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_decode_step_pool(t.handle, _ptr(pool), pool.shape[0], _ptr(slots), count,
                                        _ptr(q), _ptr(k), _ptr(v), _ptr(y), H, d_K, d_V, t.P,
                                        _dtype_code(q), _stream(stream)))


def sata_decode_step_f16(t: Tables, state16, q, k, v, y, *, stream=None):
    """One decode step on half-precision states (uint8 [B, H, sata_state16_bytes(1, 1, ...)])."""
    _need(state16, q, k, v, y)
    B, H, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_decode_step_f16(t.handle, _ptr(state16), _ptr(q), _ptr(k), _ptr(v), _ptr(y),
                                       B, H, d_K, d_V, t.P, _dtype_code(q), _stream(stream)))


def sata_decode_step_pool_f16(t: Tables, pool16, slots, q, k, v, y, *, stream=None):
    """Decode step over a pool of half-precision states (uint8 [pool_size, H, head bytes])."""
    _need(pool16, slots, q, k, v, y)
    count, H, d_K = q.shape
    d_V = v.shape[-1]
    _check(load().sata_decode_step_pool_f16(t.handle, _ptr(pool16), pool16.shape[0], _ptr(slots),
                                            count, _ptr(q), _ptr(k), _ptr(v), _ptr(y), H, d_K, d_V,
                                            t.P, _dtype_code(q), _stream(stream)))


def sata_state_pack_f16(t: Tables, state, state16, d_V: int, *, stream=None):
    """fp32 states [..., d_V + 1, M_pad] -> half-precision states (same leading shape)."""
    _need(state, state16)
    count = state.numel() // ((d_V + 1) * sata_state_stride(t.d_K, t.P))
    _check(load().sata_state_pack_f16(t.handle, _ptr(state), _ptr(state16), count, d_V, _stream(stream)))


def sata_state_unpack_f16(t: Tables, state16, state, d_V: int, *, stream=None):
    """Half-precision states -> fp32 states [..., d_V + 1, M_pad] (exact)."""
    _need(state16, state)
    count = state.numel() // ((d_V + 1) * sata_state_stride(t.d_K, t.P))
    _check(load().sata_state_unpack_f16(t.handle, _ptr(state16), _ptr(state), count, d_V, _stream(stream)))


def sata_last_error() -> str:
    return last_error()
