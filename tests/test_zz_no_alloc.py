"""The allocation-free decode step (sata_decode_step_noalloc) against sata_decode_step.

Both run the same kernels; only where the partial readouts live differs (the library's
fixed device scratch, or the handle's workspace), so y and the state must be bit-identical.
Two calls in a row on the same library scratch, the second with a smaller batch, then the
largest batch the scratch holds at d = 64; the oracle bar (2e-2 per row, bf16 inputs) is
checked as well.  Runs alone in a fresh process and after the other tests."""
import numpy as np
import pytest

from gpu_helpers import TOL_BF16, inputs, max_row_err, new_state, oracle, prefill, sata, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _step_pair(torch, t, B, H, d, P, n1, seed):
    """Prefill n1 tokens into two copies of the state, then one step with each entry point."""
    x = inputs.draw((B, H, n1 + 1, d), (B, H, n1 + 1, d), "bf16", 0.75, 1.0, seed)
    q, k, v = upload(x, "bf16")
    S = new_state(B, H, d, d, P)
    prefill(t, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), 64, S)
    S2 = S.clone()
    qd, kd, vd = (a[:, :, n1].contiguous() for a in (q, k, v))
    y_ref = torch.full((B, H, d), float("nan"), device="cuda:0")
    y_na = torch.full((B, H, d), float("nan"), device="cuda:0")
    sata.sata_decode_step(t, S, qd, kd, vd, y_ref)
    sata.sata_decode_step_noalloc(t, S2, qd, kd, vd, y_na)
    torch.cuda.synchronize()
    return x, S, S2, y_ref, y_na


def test_noalloc_decode_equals_decode_two_calls(torch_cuda):
    torch = torch_cuda
    d, P = 64, 4
    t = sata.sata_tables_build(d, P)
    for (B, H, n1, seed) in ((4, 8, 300, 1), (2, 3, 130, 2)):     # second call: smaller batch
        say("noalloc decode B=%d H=%d after prefill(%d)" % (B, H, n1))
        x, S, S2, y_ref, y_na = _step_pair(torch, t, B, H, d, P, n1, seed)
        assert torch.equal(y_ref, y_na), "y differs from sata_decode_step"
        assert torch.equal(S, S2), "state differs from sata_decode_step"
        ref = oracle.direct(x["q"], x["k"], x["v"], P)[:, :, n1]
        err = max_row_err(y_na.cpu().numpy(), ref)
        say("  y err %.3e, identical to sata_decode_step" % err)
        assert err <= TOL_BF16
    t.close()


def test_noalloc_decode_largest_batch_and_rejection(torch_cuda):
    """512 heads of d = 64 (the decode workload's batch) fit the scratch; 1024 do not."""
    torch = torch_cuda
    d, P = 64, 4
    t = sata.sata_tables_build(d, P)
    B, H = 16, 32
    say("noalloc decode at the scratch's largest d=64 batch (%d heads)" % (B * H))
    Mp = sata.sata_state_stride(d, P)
    rng = np.random.default_rng(3)
    S = torch.from_numpy(rng.standard_normal((B, H, d + 1, Mp)).astype(np.float32) * 0.01).cuda()
    S[:, :, d, :] = 1.0
    S[..., sata.sata_feature_dim(d, P):] = 0.0
    S2 = S.clone()
    x = inputs.draw((B, H, d), (B, H, d), "bf16", 0.5, 1.0, 4)
    q, k, v = upload(x, "bf16")
    y1 = torch.empty((B, H, d), device="cuda:0")
    y2 = torch.empty((B, H, d), device="cuda:0")
    sata.sata_decode_step(t, S, q, k, v, y1)
    sata.sata_decode_step_noalloc(t, S2, q, k, v, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S, S2)
    big = torch.empty((2 * B, H, d), device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(sata.SataError) as e:
        sata.sata_decode_step_noalloc(t, torch.empty((1,), device="cuda:0"), big, big, big,
                                      torch.empty((2 * B, H, d), device="cuda:0"))
    assert e.value.code == sata.SATA_ERR_UNSUPPORTED
    t.close()
