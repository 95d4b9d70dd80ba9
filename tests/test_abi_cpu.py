"""CPU checks of the C ABI: the library loads, exports what include/sata.h
declares, builds tables bit-exact to the oracle's brute force, and rejects bad
arguments before touching any device memory.  No compute call runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from constant_cost_self_amd import sata

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sata.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sata_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = sata.load()
    names = _declared()
    assert "sata_prefill" in names and "sata_decode_step" in names
    for name in names:
        assert hasattr(lib, name), name
        assert name in sata.EXPORTED, name


@pytest.mark.parametrize("d,P", [(1, 1), (2, 4), (8, 4), (64, 4), (128, 4), (16, 5), (7, 3)])
def test_size_helpers_match_closed_forms(d, P):
    M = sata.sata_feature_dim(d, P)
    assert M == oracle.feature_dim(d, P)
    Mp = sata.sata_state_stride(d, P)
    assert Mp % 64 == 0 and M <= Mp < M + 64
    assert sata.sata_state_bytes(2, 3, d, 5, P) == 4 * 2 * 3 * 6 * Mp


def test_size_helpers_reject_unsupported():
    assert sata.sata_feature_dim(0, 4) == -1
    assert sata.sata_feature_dim(129, 4) == -1
    assert sata.sata_feature_dim(8, 6) == -1
    assert sata.sata_state_bytes(0, 1, 8, 8, 4) == -1


@pytest.mark.parametrize("d", [1, 2, 3, 4, 8, 16, 64, 128])
def test_tables_bit_exact_to_oracle(d):
    P = 4
    t = sata.sata_tables_build_host(d, P)
    try:
        for p in range(P):
            M, C = t.get(p)
            Mo, Co = oracle.tables(d, p)
            assert M.dtype == np.int32 and C.dtype == np.int32
            assert M.shape == Mo.shape
            assert np.array_equal(M, Mo), (d, p)
            assert np.array_equal(C.astype(np.int64), Co), (d, p)
    finally:
        t.close()


def test_tables_p4_bit_exact():
    t = sata.sata_tables_build_host(8, 5)
    M, C = t.get(4)
    Mo, Co = oracle.tables(8, 4)
    assert np.array_equal(M, Mo) and np.array_equal(C.astype(np.int64), Co)
    t.close()


def test_tables_get_rejects_bad_p():
    t = sata.sata_tables_build_host(8, 4)
    with pytest.raises(sata.SataError) as e:
        t.get(4)
    assert e.value.code == sata.SATA_ERR_ARG
    t.close()


def test_tables_build_rejects_unsupported():
    with pytest.raises(sata.SataError) as e:
        sata.sata_tables_build_host(8, 6)
    assert e.value.code == sata.SATA_ERR_UNSUPPORTED
    with pytest.raises(sata.SataError):
        sata.sata_tables_build_host(0, 4)


# ---- argument checking (host-only handle; fake, aligned, never dereferenced) ----

A = 0x10000          # an aligned fake device address: the checks must not touch it


def _prefill(t, **kw):
    args = dict(q=A, k=A, v=A, y=A, state=0, B=1, H=2, n=100, d_K=8, d_V=8, P=4, chunk=16,
                dtype=sata.SATA_F32, flags=0)
    args.update(kw)
    lib = sata.load()
    return lib.sata_prefill(t.handle if t else None, args["q"], args["k"], args["v"],
                            args["y"], args["state"] or None, args["B"], args["H"], args["n"],
                            args["d_K"], args["d_V"], args["P"], args["chunk"], args["dtype"],
                            args["flags"], None)


def _decode(t, **kw):
    args = dict(state=A, q=A, k=A, v=A, y=A, B=1, H=2, d_K=8, d_V=8, P=4, dtype=sata.SATA_F32)
    args.update(kw)
    lib = sata.load()
    return lib.sata_decode_step(t.handle if t else None, args["state"] or None, args["q"] or None,
                                args["k"], args["v"], args["y"], args["B"], args["H"],
                                args["d_K"], args["d_V"], args["P"], args["dtype"], None)


@pytest.fixture()
def host_tables():
    t = sata.sata_tables_build_host(8, 4)
    yield t
    t.close()


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),                       # valid args, but host-only handle
    (dict(q=0), sata.SATA_ERR_ARG),
    (dict(n=0), sata.SATA_ERR_ARG),
    (dict(B=0), sata.SATA_ERR_ARG),
    (dict(d_K=16), sata.SATA_ERR_ARG),                 # handle mismatch
    (dict(P=3), sata.SATA_ERR_ARG),
    (dict(d_V=129), sata.SATA_ERR_UNSUPPORTED),
    (dict(chunk=48), sata.SATA_ERR_UNSUPPORTED),
    (dict(dtype=7), sata.SATA_ERR_ARG),
    (dict(flags=1), sata.SATA_ERR_ARG),                # CONTINUE without a state
    (dict(flags=4, state=A), sata.SATA_ERR_ARG),
    (dict(y=A + 4), sata.SATA_ERR_ALIGN),
    (dict(state=A + 8), sata.SATA_ERR_ALIGN),
])
def test_prefill_argument_errors(host_tables, kw, code):
    assert _prefill(host_tables, **kw) == code
    assert sata.last_error() != ""


def test_prefill_null_handle():
    assert _prefill(None) == sata.SATA_ERR_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),
    (dict(state=0), sata.SATA_ERR_ARG),
    (dict(H=0), sata.SATA_ERR_ARG),
    (dict(P=5), sata.SATA_ERR_ARG),
    (dict(d_V=0), sata.SATA_ERR_UNSUPPORTED),
    (dict(k=A + 2), sata.SATA_ERR_ALIGN),
])
def test_decode_argument_errors(host_tables, kw, code):
    assert _decode(host_tables, **kw) == code


def test_error_message_is_thread_local_and_cleared(host_tables):
    assert _prefill(host_tables, chunk=48) == sata.SATA_ERR_UNSUPPORTED
    assert "chunk" in sata.last_error()
    assert sata.load().sata_feature_dim(8, 4) == 165
    t = sata.sata_tables_build_host(8, 4)        # a successful call clears the message
    assert sata.last_error() == ""
    t.close()


def test_workspace_limit_argument(host_tables):
    host_tables.set_workspace_limit(1 << 20)
    host_tables.set_workspace_limit(0)
    with pytest.raises(sata.SataError):
        host_tables.set_workspace_limit(-1)


def test_prefill_split_argument(host_tables):
    for k in (0, 1, 2, 7, 4096):
        host_tables.set_prefill_split(k)
    for k in (-1, 4097):
        with pytest.raises(sata.SataError):
            host_tables.set_prefill_split(k)
    assert sata.load().sata_set_prefill_split(None, 2) == sata.SATA_ERR_ARG


def _decode_pool(t, **kw):
    args = dict(pool=A, pool_size=3, slots=A, count=2, q=A, k=A, v=A, y=A, H=2, d_K=8, d_V=8, P=4,
                dtype=sata.SATA_F32)
    args.update(kw)
    lib = sata.load()
    return lib.sata_decode_step_pool(t.handle if t else None, args["pool"] or None, args["pool_size"],
                                     args["slots"] or None, args["count"], args["q"], args["k"],
                                     args["v"], args["y"], args["H"], args["d_K"], args["d_V"],
                                     args["P"], args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),                       # valid args, but host-only handle
    (dict(pool=0), sata.SATA_ERR_ARG),
    (dict(slots=0), sata.SATA_ERR_ARG),
    (dict(count=0), sata.SATA_ERR_ARG),
    (dict(pool_size=0), sata.SATA_ERR_ARG),
    (dict(H=0), sata.SATA_ERR_ARG),
    (dict(d_K=16), sata.SATA_ERR_ARG),                 # handle mismatch
    (dict(d_V=0), sata.SATA_ERR_UNSUPPORTED),
    (dict(slots=A + 2), sata.SATA_ERR_ALIGN),
    (dict(y=A + 4), sata.SATA_ERR_ALIGN),
    (dict(count=40000, H=2), sata.SATA_ERR_UNSUPPORTED),
])
def test_decode_pool_argument_errors(host_tables, kw, code):
    assert _decode_pool(host_tables, **kw) == code
    assert sata.last_error() != ""


def test_decode_pool_null_handle():
    assert _decode_pool(None) == sata.SATA_ERR_ARG


def _backward(t, **kw):
    args = dict(q=A, k=A, v=A, dy=A, dq=A, dk=A, dv=A, B=1, H=2, n=100, d_K=8, d_V=8, P=4,
                chunk=16, dtype=sata.SATA_F32)
    args.update(kw)
    lib = sata.load()
    return lib.sata_prefill_backward(t.handle if t else None, args["q"] or None, args["k"], args["v"],
                                     args["dy"] or None, args["dq"], args["dk"], args["dv"] or None,
                                     args["B"], args["H"], args["n"], args["d_K"], args["d_V"],
                                     args["P"], args["chunk"], args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),                       # valid args, but host-only handle
    (dict(q=0), sata.SATA_ERR_ARG),
    (dict(dy=0), sata.SATA_ERR_ARG),
    (dict(dv=0), sata.SATA_ERR_ARG),
    (dict(n=0), sata.SATA_ERR_ARG),
    (dict(H=0), sata.SATA_ERR_ARG),
    (dict(d_K=16), sata.SATA_ERR_ARG),                 # handle mismatch
    (dict(d_V=129), sata.SATA_ERR_UNSUPPORTED),
    (dict(chunk=48), sata.SATA_ERR_UNSUPPORTED),
    (dict(dtype=7), sata.SATA_ERR_ARG),
    (dict(dk=A + 4), sata.SATA_ERR_ALIGN),
])
def test_backward_argument_errors(host_tables, kw, code):
    assert _backward(host_tables, **kw) == code
    assert sata.last_error() != ""


def test_backward_rejects_chunk_too_large_for_lds():
    t = sata.sata_tables_build_host(128, 4)
    try:
        assert _backward(t, d_K=128, d_V=128, chunk=128) == sata.SATA_ERR_UNSUPPORTED
        assert "too large" in sata.last_error()
    finally:
        t.close()


def test_backward_null_handle():
    assert _backward(None) == sata.SATA_ERR_ARG
