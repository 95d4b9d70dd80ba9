"""GPU checks of the pool form of the decode step (sata_decode_step_pool): sequences of
different lengths, each prefilled into its own slot of a preallocated pool, decoded
together; y of every step against the oracle's direct form over each whole sequence;
slots outside the batch and a guard slot past the pool left bit-identical; an entry
with an out-of-range slot reads out NaN and touches nothing; the pool step equal bit
for bit to the dense step on the same states.  d = 64, P = 4, bf16 inputs with the
Mid workload's distributions."""
import numpy as np
import pytest

from gpu_helpers import TOL_BF16, inputs, max_row_err, oracle, sata, say, upload

pytestmark = pytest.mark.gpu

D, P, H = 64, 4, 2
LENS = (100, 257, 64)          # ragged prefill lengths (the last chunk of two is partial)
SLOTS = (4, 0, 2)              # their pool slots
POOL = 5                       # slots 1 and 3 stay unused
STEPS = 3
SENTINEL = 7.0


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _setup(torch):
    w = inputs.MID
    t = sata.sata_tables_build(D, P)
    Mp = sata.sata_state_stride(D, P)
    # one guard slot past the pool: the calls are given POOL slots
    pool = torch.full((POOL + 1, H, D + 1, Mp), SENTINEL, device="cuda:0", dtype=torch.float32)
    seqs = []
    for i, (n, s) in enumerate(zip(LENS, SLOTS)):
        x = inputs.prefill_inputs(w, n=n, B=1, H=H, seed=10 + i)
        q, k, v = upload(x, w.dtype)
        pool[s].zero_()
        y = torch.empty((1, H, n, D), device="cuda:0", dtype=torch.float32)
        sata.sata_prefill(t, q, k, v, y, pool[s:s + 1], chunk=64)
        seqs.append(x)
    torch.cuda.synchronize()
    return w, t, pool, seqs


def test_pool_decode_ragged_batch(torch_cuda):
    torch = torch_cuda
    w, t, pool, seqs = _setup(torch)
    st = inputs.decode_inputs(w, STEPS, seed=20, B=len(LENS), H=H)
    qs, ks, vs = upload(st, w.dtype)
    slots = torch.tensor(SLOTS, dtype=torch.int32, device="cuda:0")
    ys = torch.empty((STEPS, len(LENS), H, D), device="cuda:0", dtype=torch.float32)
    untouched = [pool[s].clone() for s in (1, 3, POOL)]
    for i in range(STEPS):
        sata.sata_decode_step_pool(t, pool[:POOL], slots, qs[i], ks[i], vs[i], ys[i])
    torch.cuda.synchronize()
    yh = ys.cpu().numpy()
    for e, (x, n) in enumerate(zip(seqs, LENS)):
        for h in range(H):
            cat = {c: np.concatenate([x[c][0, h], st[c][:, e, h]], axis=0) for c in ("q", "k", "v")}
            rows = np.arange(n, n + STEPS)
            ref = oracle.direct_rows(cat["q"][None], cat["k"][None], cat["v"][None], P,
                                     np.zeros_like(rows), rows)
            err = max_row_err(yh[:, e, h], ref)
            say("  entry %d (slot %d, %d tokens) head %d: y err %.3e" % (e, SLOTS[e], n, h, err))
            assert err <= TOL_BF16
    for s, before in zip((1, 3, POOL), untouched):
        assert torch.equal(pool[s], before), "slot %d changed" % s
    # the sequence counts of the used slots: Z[p = 0] is the number of tokens seen
    for s, n in zip(SLOTS, LENS):
        z0 = pool[s, :, D, 0].cpu().numpy()
        assert np.all(z0 == n + STEPS), (s, z0)
    t.close()


def test_pool_decode_out_of_range_slot(torch_cuda):
    torch = torch_cuda
    w, t, pool, _ = _setup(torch)
    st = inputs.decode_inputs(w, 1, seed=21, B=3, H=H)
    qs, ks, vs = upload(st, w.dtype)
    slots = torch.tensor([SLOTS[0], POOL, -1], dtype=torch.int32, device="cuda:0")
    before = pool.clone()
    y = torch.zeros((3, H, D), device="cuda:0", dtype=torch.float32)
    sata.sata_decode_step_pool(t, pool[:POOL], slots, qs[0], ks[0], vs[0], y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(np.isfinite(yh[0]))
    assert np.all(np.isnan(yh[1])) and np.all(np.isnan(yh[2]))
    for s in range(POOL + 1):
        if s != SLOTS[0]:
            assert torch.equal(pool[s], before[s]), "slot %d changed" % s
    assert not torch.equal(pool[SLOTS[0]], before[SLOTS[0]])
    t.close()


def test_pool_step_equals_dense_step(torch_cuda):
    torch = torch_cuda
    w, t, pool, _ = _setup(torch)
    st = inputs.decode_inputs(w, 1, seed=22, B=len(LENS), H=H)
    qs, ks, vs = upload(st, w.dtype)
    order = [SLOTS[2], SLOTS[0], SLOTS[1]]                 # any order of distinct slots
    slots = torch.tensor(order, dtype=torch.int32, device="cuda:0")
    dense = pool[order].clone()
    y_pool = torch.empty((len(order), H, D), device="cuda:0", dtype=torch.float32)
    y_dense = torch.empty_like(y_pool)
    sata.sata_decode_step_pool(t, pool[:POOL], slots, qs[0], ks[0], vs[0], y_pool)
    sata.sata_decode_step(t, dense, qs[0], ks[0], vs[0], y_dense)
    torch.cuda.synchronize()
    assert torch.equal(y_pool, y_dense)
    assert torch.equal(pool[order], dense)
    t.close()
