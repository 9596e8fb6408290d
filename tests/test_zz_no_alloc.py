"""hqq_quantize_noalloc (the library's own scratch array, no allocation) against hqq_quantize (the
caller's workspace) through the C ABI: two calls in a row, the second on a smaller tensor, so the
second runs on scratch the first has filled; every output bit for bit (the same kernels)."""
import numpy as np
import pytest

import synth
from tests.gpu_common import say, torch_dev

pytestmark = pytest.mark.gpu

CASES = [  # (rows, cols, nbits, g, axis, seed) of the first call, then of the smaller second call
    ((4096, 4096, 4, 64, 1, 501), (1024, 2048, 4, 64, 1, 502)),
    ((2048, 4096, 2, 16, 1, 503), (512, 1024, 2, 16, 1, 504)),      # stops early: the fix-up pass runs
    ((2048, 2048, 3, 64, 1, 505), (256, 640, 3, 64, 1, 506)),
    ((4096, 2048, 4, 128, 0, 507), (1024, 512, 4, 128, 0, 508)),
]


def _outs(torch, rows, cols, nbits, g, iters):
    import weight_only_quantization_amd as hq
    G = rows * cols // g
    return (torch.empty(hq.hqq_packed_bytes(rows, cols, nbits), dtype=torch.uint8, device="cuda"),
            torch.empty(G, dtype=torch.float16, device="cuda"), torch.empty(G, dtype=torch.float16, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"), torch.empty(iters, dtype=torch.float64, device="cuda"))


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry(first, second):
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    for rows, cols, nbits, g, axis, seed in (first, second):
        say("noalloc", rows, cols, nbits, g, axis)
        Wn = synth.weight_normal(rows, cols, 0.02, seed, 0.001, 10.0) if nbits == 4 else \
            synth.weight_laplace(rows, cols, 0.015, seed)
        W = torch.from_numpy(Wn).cuda()
        out = _outs(torch, rows, cols, nbits, g, 20)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        hq.hqq_quantize_noalloc(W, out, nbits=nbits, group_size=g, axis=axis, iters=20)
        assert torch.cuda.memory_allocated() == before  # nothing allocated through torch either
        ref = hq.hqq_quantize(W, nbits=nbits, group_size=g, axis=axis, iters=20)
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref.packed[:out[0].numel()])
        assert torch.equal(out[1], ref.delta) and torch.equal(out[2], ref.zero)
        assert int(out[3].item()) == int(ref.stop_iter.item())
        assert np.array_equal(out[4].cpu().numpy(), ref.mae_trace.cpu().numpy(), equal_nan=True)
        say("  stop", int(out[3].item()))
