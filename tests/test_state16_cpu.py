"""CPU checks of the half-precision state's C ABI: its sizes against the layout that
include/sata.h documents, the workspace queries, and argument errors of the calls that use
it (host-only handle; fake aligned addresses that the checks must not touch)."""
import math

import pytest

from constant_cost_self_amd import sata

A = 0x10000


def _layout_bytes(d_K, d_V, P):
    rows = sum((math.comb(d_K + p - 1, p) + 63) // 64 * 64 for p in range(P))
    hdr = (8 * P * d_V + 255) // 256 * 256
    return rows, (hdr + 4 * rows + 2 * d_V * rows + 255) // 256 * 256


@pytest.mark.parametrize("d_K,d_V,P", [(1, 1, 1), (7, 20, 5), (8, 8, 4), (64, 64, 4), (128, 128, 4),
                                       (64, 64, 5), (128, 128, 5), (16, 3, 2)])
def test_state16_sizes(d_K, d_V, P):
    rows, head = _layout_bytes(d_K, d_V, P)
    assert sata.sata_state16_stride(d_K, P) == rows
    assert sata.sata_state16_bytes(3, 2, d_K, d_V, P) == 6 * head
    assert head % 256 == 0


def test_state16_halves_the_decode_bytes():
    # [TA] "Hidden-state size and compute analysis": about 6.2 MB per head in Float16 at
    # d = 64, P = 4 (47905 x 65 x 2 bytes); this layout holds the normaliser column in fp32
    b16 = sata.sata_state16_bytes(1, 1, 64, 64, 4)
    assert 6.2e6 < b16 < 6.4e6
    for d in (64, 128):
        r = sata.sata_state16_bytes(1, 1, d, d, 4) / sata.sata_state_bytes(1, 1, d, d, 4)
        assert 0.50 < r < 0.51


def test_state16_sizes_reject_unsupported():
    assert sata.sata_state16_stride(0, 4) == -1
    assert sata.sata_state16_stride(8, 6) == -1
    assert sata.sata_state16_bytes(0, 1, 8, 8, 4) == -1
    assert sata.sata_state16_bytes(1, 1, 8, 129, 4) == -1


@pytest.fixture()
def host_tables():
    t = sata.sata_tables_build_host(8, 4)
    yield t
    t.close()


def test_prefill_flag_needs_a_state(host_tables):
    lib = sata.load()
    rc = lib.sata_prefill(host_tables.handle, A, A, A, A, None, 1, 2, 100, 8, 8, 4, 16,
                          sata.SATA_F32, sata.SATA_STATE_F16, None)
    assert rc == sata.SATA_ERR_ARG and "state" in sata.last_error()
    rc = lib.sata_prefill(host_tables.handle, A, A, A, A, A, 1, 2, 100, 8, 8, 4, 16,
                          sata.SATA_F32, sata.SATA_STATE_F16 | sata.SATA_PREFILL_CONTINUE, None)
    assert rc == sata.SATA_ERR_ARG and "host-only" in sata.last_error()


def test_prefill_workspace_holds_the_fp32_copy():
    t = sata.sata_tables_build_host(64, 4)
    try:
        for B, H, n in ((1, 8, 4096), (4, 16, 65536), (16, 32, 1024)):
            w32 = t.prefill_workspace(B, H, n, 64)[0]
            w16 = t.prefill_workspace(B, H, n, 64, state16=True)[0]
            s32 = sata.sata_state_bytes(B, H, 64, 64, 4)
            assert w32 + s32 <= w16 <= w32 + s32 + 512, (B, H, n)
        with pytest.raises(sata.SataError):
            t.prefill_workspace(1, 8, 4096, 64, with_state=False, state16=True)
    finally:
        t.close()


def test_decode_workspace_covers_both_forms():
    for d, P in ((64, 4), (128, 4), (7, 5)):
        t = sata.sata_tables_build_host(d, P)
        try:
            rows = sata.sata_state16_stride(d, P)
            # readout partials of d + 1 columns and block maxima of P x d blocks, per wave of
            # 512 rows (two waves per 1024-row block)
            need16 = 16 * 32 * (d + 1 + P * d) * ((rows + 1023) // 1024) * 2 * 4
            need32 = 16 * 32 * (d + 1) * ((sata.sata_state_stride(d, P) + 1023) // 1024) * 2 * 4
            assert t.decode_workspace(16, 32, d) == max(need16, need32)
        finally:
            t.close()


def _decode16(t, **kw):
    args = dict(state=A, q=A, k=A, v=A, y=A, B=1, H=2, d_K=8, d_V=8, P=4, dtype=sata.SATA_F32)
    args.update(kw)
    return sata.load().sata_decode_step_f16(t.handle if t else None, args["state"] or None,
                                            args["q"] or None, args["k"], args["v"], args["y"],
                                            args["B"], args["H"], args["d_K"], args["d_V"], args["P"],
                                            args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),                       # valid args, but host-only handle
    (dict(state=0), sata.SATA_ERR_ARG),
    (dict(q=0), sata.SATA_ERR_ARG),
    (dict(B=0), sata.SATA_ERR_ARG),
    (dict(P=5), sata.SATA_ERR_ARG),
    (dict(d_V=0), sata.SATA_ERR_UNSUPPORTED),
    (dict(state=A + 8), sata.SATA_ERR_ALIGN),
    (dict(dtype=3), sata.SATA_ERR_ARG),
])
def test_decode16_argument_errors(host_tables, kw, code):
    assert _decode16(host_tables, **kw) == code
    assert sata.last_error() != ""


def test_decode16_null_handle():
    assert _decode16(None) == sata.SATA_ERR_ARG


def _pool16(t, **kw):
    args = dict(pool=A, pool_size=3, slots=A, count=2, q=A, k=A, v=A, y=A, H=2, d_K=8, d_V=8, P=4,
                dtype=sata.SATA_F32)
    args.update(kw)
    return sata.load().sata_decode_step_pool_f16(
        t.handle if t else None, args["pool"] or None, args["pool_size"], args["slots"] or None,
        args["count"], args["q"], args["k"], args["v"], args["y"], args["H"], args["d_K"],
        args["d_V"], args["P"], args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), sata.SATA_ERR_ARG),
    (dict(pool=0), sata.SATA_ERR_ARG),
    (dict(slots=0), sata.SATA_ERR_ARG),
    (dict(count=0), sata.SATA_ERR_ARG),
    (dict(pool_size=0), sata.SATA_ERR_ARG),
    (dict(slots=A + 2), sata.SATA_ERR_ALIGN),
    (dict(d_K=16), sata.SATA_ERR_ARG),
])
def test_pool16_argument_errors(host_tables, kw, code):
    assert _pool16(host_tables, **kw) == code


@pytest.mark.parametrize("fn", ["sata_state_pack_f16", "sata_state_unpack_f16"])
@pytest.mark.parametrize("args,code", [
    ((A, A, 4, 8), sata.SATA_ERR_ARG),                 # valid, but host-only handle
    ((0, A, 4, 8), sata.SATA_ERR_ARG),
    ((A, 0, 4, 8), sata.SATA_ERR_ARG),
    ((A, A, 0, 8), sata.SATA_ERR_ARG),
    ((A, A, 70000, 8), sata.SATA_ERR_ARG),
    ((A, A, 4, 129), sata.SATA_ERR_UNSUPPORTED),
    ((A + 4, A, 4, 8), sata.SATA_ERR_ALIGN),
])
def test_conversion_argument_errors(host_tables, fn, args, code):
    a, b, count, d_V = args
    rc = getattr(sata.load(), fn)(host_tables.handle, a or None, b or None, count, d_V, None)
    assert rc == code
    assert getattr(sata.load(), fn)(None, A, A, 4, 8, None) == sata.SATA_ERR_ARG
