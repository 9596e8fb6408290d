"""Calls on a side stream: the binding allocates outputs and workspaces on the stream the kernels
run on, so a temporary freed on return is not handed to other work on the current stream while
the kernels still use it.  The results on a side stream, with the current stream allocating and
writing meanwhile, must equal those of the same calls on the current stream."""
import numpy as np
import pytest

import synth
from tests.gpu_common import say, torch_dev

pytestmark = pytest.mark.gpu


def test_side_stream_results_match():
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    say("side stream")
    W = torch.from_numpy(synth.weight_normal(1024, 2048, 0.02, seed=91, outlier_frac=0.001, outlier_k=10.0)).cuda()
    x = torch.from_numpy(synth.activations(64, 2048, seed=92)).cuda()
    q0 = hq.hqq_quantize(W, nbits=4, group_size=64, axis=1, iters=20)
    y0 = hq.hqq_gemm_w4a16(q0.packed, q0.delta, q0.zero, 1024, 2048, 64, x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(4):
        q = hq.hqq_quantize(W, nbits=4, group_size=64, axis=1, iters=20, stream=side)
        y = hq.hqq_gemm_w4a16(q0.packed, q0.delta, q0.zero, 1024, 2048, 64, x, stream=side)
        outs.append((q, y))
        # the current stream allocates and overwrites memory while the side stream runs
        junk = [torch.full((1 << 20,), float(rep), device="cuda") for _ in range(8)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for q, y in outs:
        assert torch.equal(q.packed, q0.packed) and torch.equal(q.delta, q0.delta) and torch.equal(q.zero, q0.zero)
        assert int(q.stop_iter.item()) == int(q0.stop_iter.item())
        assert torch.equal(y, y0)
    assert np.isfinite(y0.float().cpu().numpy()).all()
