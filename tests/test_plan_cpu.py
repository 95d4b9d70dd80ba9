"""CPU checks of the prefill's sequence plan through sata_prefill_workspace (host-only
handles, no device work): every workspace cap gives segments of whole readout windows that
cover the sequence, the cap holds whenever one window fits it, and no size divides by zero
(a segment length rounded down to zero used to crash the caller with SIGFPE)."""
import pytest

from constant_cost_self_amd import sata

# (d_K, d_V, chunk, dtype, chunks per readout window)
PATHS = [(64, 64, 64, sata.SATA_BF16, 4),     # matrix-core scan, d = 64
         (128, 128, 64, sata.SATA_BF16, 2),   # matrix-core scan, d = 128
         (8, 8, 16, sata.SATA_F32, 1)]        # fp32 scan


@pytest.fixture(scope="module")
def handles():
    hs = {d: sata.sata_tables_build_host(d, 4) for d in (8, 64, 128)}
    yield hs
    for t in hs.values():
        t.close()


def _plan(t, B, H, n, dV, chunk, dtype, with_state=True):
    return t.prefill_workspace(B, H, n, dV, chunk=chunk, dtype=dtype, with_state=with_state,
                               segment_chunks=True)


@pytest.mark.parametrize("dK,dV,chunk,dtype,win", PATHS)
def test_segments_cover_whole_windows_under_every_cap(handles, dK, dV, chunk, dtype, win):
    t = handles[dK]
    t.set_prefill_split(1)                       # the one-level form only
    B, H = 1, 2
    t.set_workspace_limit(1 << 62)
    one_window = _plan(t, B, H, win * chunk, dV, chunk, dtype)[0]
    per_chunk = (_plan(t, B, H, 2 * win * chunk, dV, chunk, dtype)[0] - one_window) // win
    assert per_chunk > 0 and one_window > 0
    try:
        for nch in range(1, 65):
            n = nch * chunk - (chunk // 3 if nch > 1 else 0)      # ragged last chunk
            for cap_chunks in range(1, nch + 2):
                for extra in (0, per_chunk // 2):
                    cap = one_window + (cap_chunks - 1) * per_chunk + extra
                    t.set_workspace_limit(cap)
                    nbytes, nseg, nsub, seg = _plan(t, B, H, n, dV, chunk, dtype)
                    assert nsub == 1
                    assert nseg >= 1 and seg >= 1
                    assert (nseg - 1) * seg < nch <= nseg * seg, (nch, cap_chunks, seg, nseg)
                    if nseg > 1:
                        assert seg % win == 0, (nch, cap_chunks, seg)
                    assert nbytes <= cap, (nch, cap_chunks, seg, nbytes, cap)
            # a cap below one window: single windows, above the cap
            t.set_workspace_limit(one_window // 2)
            nbytes, nseg, nsub, seg = _plan(t, B, H, nch * chunk, dV, chunk, dtype)
            assert seg == min(win, nch) or nseg == 1
    finally:
        t.set_workspace_limit(0)
        t.set_prefill_split(0)


def test_advisor_shapes_do_not_crash(handles):
    """The two shapes that reached a zero segment length: B=H=1, n=560 with a 4 MiB cap,
    and B=128, H=64, n=560 under the default cap."""
    t = handles[64]
    t.set_workspace_limit(4 << 20)
    nbytes, nseg, nsub, seg = _plan(t, 1, 1, 560, 64, 64, sata.SATA_BF16)
    assert nseg >= 1 and nbytes > 0 and seg >= 4
    t.set_workspace_limit(0)
    nbytes, nseg, nsub, seg = _plan(t, 128, 64, 560, 64, 64, sata.SATA_BF16)
    # 9 chunks of 8192 heads: one readout window (4 chunks) fits the 32 GiB cap, two do not,
    # so the segments are single windows
    assert nseg == 3 and seg == 4 and nbytes <= 32 << 30


def test_carrier_counted_without_caller_state(handles):
    """Without a caller state, several segments carry the state in the workspace."""
    t = handles[64]
    t.set_prefill_split(1)
    t.set_workspace_limit(1 << 62)
    full = t.prefill_workspace(1, 1, 64 * 64, 64)[0]
    t.set_workspace_limit(full // 3)
    with_state = _plan(t, 1, 1, 64 * 64, 64, 64, sata.SATA_BF16, with_state=True)
    without = _plan(t, 1, 1, 64 * 64, 64, 64, sata.SATA_BF16, with_state=False)
    assert with_state[1] > 1 and without[1] > 1
    assert without[3] <= with_state[3]
    t.set_workspace_limit(0)
    t.set_prefill_split(0)


def test_two_level_plan(handles):
    """One head of 65536 tokens leaves the CUs idle: the automatic plan takes sub-segments
    of at least 4 readout windows; a forced split is honoured; split 1 never uses it."""
    t = handles[64]
    nbytes, nseg, nsub = t.prefill_workspace(1, 1, 65536, 64)
    assert nseg == 1 and nsub >= 2
    t.set_prefill_split(5)
    assert t.prefill_workspace(1, 1, 65536, 64)[2] == 5
    t.set_prefill_split(1)
    assert t.prefill_workspace(1, 1, 65536, 64)[2] == 1
    t.set_prefill_split(0)
    assert t.prefill_workspace(4, 16, 65536, 64)[2] == 1     # enough heads: one level


def test_workspace_query_checks_arguments(handles):
    t = handles[64]
    with pytest.raises(sata.SataError):
        t.prefill_workspace(0, 1, 100, 64)
    with pytest.raises(sata.SataError):
        t.prefill_workspace(1, 1, 100, 64, chunk=48)
    with pytest.raises(sata.SataError):
        t.prefill_workspace(1, 1, 100, 64, continue_state=True, with_state=False)


def test_decode_workspace(handles):
    t = handles[64]
    nb = t.decode_workspace(16, 32, 64)
    assert nb > 0 and nb % 4 == 0
    assert t.decode_workspace(32, 32, 64) == 2 * nb


@pytest.mark.parametrize("d,P", [(64, 2), (64, 3), (64, 4), (64, 5), (128, 2), (128, 3), (128, 4)])
def test_matrix_core_rows_build_for_every_supported_shape(d, P):
    """The row tables of the matrix-core scan (every monomial of the basis in exactly one
    8-slot row, checked when they are built) exist for every bf16 shape it serves: its plan
    cuts a long sequence under a small cap into whole readout windows (4 chunks at d = 64,
    2 at d = 128), where the fp32 scan would cut single chunks."""
    t = sata.sata_tables_build_host(d, P)
    try:
        t.set_prefill_split(1)
        one = _plan(t, 1, 1, 64, d, 64, sata.SATA_BF16)[0]
        t.set_workspace_limit(3 * one)
        nbytes, nseg, nsub, seg = _plan(t, 1, 1, 64 * 40, d, 64, sata.SATA_BF16)
        assert nseg > 1 and seg % (4 if d == 64 else 2) == 0 and seg > 1
    finally:
        t.close()
