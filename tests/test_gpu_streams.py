"""One tables handle used from two streams at once: the prefills and decode steps enqueued
on two streams overlap on the device, and each must give what it gives alone (each stream
has its own workspace).  Compared bit for bit with the same calls run one after another,
and the prefill against the oracle."""
import numpy as np
import pytest

from gpu_helpers import TOL_BF16, inputs, max_row_err, new_state, oracle, sata, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def test_one_handle_two_streams(torch_cuda):
    torch = torch_cuda
    d, P, n = 64, 4, 1500
    say("one handle, two streams: 2 x (prefill of 2 x 4 heads, n=%d, then 3 decode steps)" % n)
    xs = [inputs.draw((2, 4, n + 3, d), (2, 4, n + 3, d), "bf16", 0.5, 1.0, 401 + i) for i in range(2)]
    ups = [upload(x, "bf16") for x in xs]
    t = sata.sata_tables_build(d, P)

    def run(i, stream):
        q, k, v = ups[i]
        with torch.cuda.stream(stream):
            # allocated and zero-filled on the stream that uses them
            y = torch.empty((2, 4, n, d), device="cuda:0", dtype=torch.float32)
            S = new_state(2, 4, d, d, P)
            yd = torch.empty((3, 2, 4, d), device="cuda:0", dtype=torch.float32)
            sata.sata_prefill(t, q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                              y, S, stream=stream)
            for s in range(3):
                sata.sata_decode_step(t, S, q[:, :, n + s].contiguous(), k[:, :, n + s].contiguous(),
                                      v[:, :, n + s].contiguous(), yd[s], stream=stream)
        return y, S, yd

    # one after another on the default stream
    ref = [run(i, torch.cuda.current_stream()) for i in range(2)]
    torch.cuda.synchronize()
    # both at once, on two streams
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    got = [run(i, streams[i]) for i in range(2)]
    torch.cuda.synchronize()
    for i in range(2):
        for a, b, name in zip(got[i], ref[i], ("y", "state", "decode y")):
            assert torch.equal(a, b), "stream %d: %s differs from the serial run" % (i, name)
        err = max_row_err(got[i][0].cpu().numpy(), oracle.direct(xs[i]["q"][:, :, :n], xs[i]["k"][:, :, :n],
                                                                 xs[i]["v"][:, :, :n], P))
        say("  stream %d: prefill y err %.3e" % (i, err))
        assert err <= TOL_BF16
    t.close()
