"""GPU parity of the scale search (hqq_quantize_v2) with the oracle's reading of the second
solver: codes, steps, zeros and the chosen multiplier per group, bit for bit where both sides
evaluate the same expressions (everywhere the shrink stays zero)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import CODE_AGREEMENT, Z_TOL, say, torch_dev
from tests.test_gpu_small import edge_tensor

pytestmark = pytest.mark.gpu

GRID3 = [0.9, 1.0, 1.08]
GRID5 = [0.85, 0.925, 1.0, 1.05, 1.1]
GRID16 = list(np.linspace(0.8, 1.2, 16))


def gpu_v2(W16, grid, nbits, g, iters=20, meta="f64", axis=1, **kw):
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    Wd = torch.from_numpy(np.ascontiguousarray(W16)).cuda()
    md = {"f16": torch.float16, "f32": torch.float32, "f64": torch.float64}[meta]
    q, choice = hq.hqq_quantize_v2(Wd, grid, nbits=nbits, group_size=g, iters=iters, meta_dtype=md, axis=axis, **kw)
    torch.cuda.synchronize()
    out = {"packed": q.packed.cpu().numpy(), "delta": q.delta.cpu().numpy(), "zero": q.zero.cpu().numpy(),
           "choice": choice.cpu().numpy()}
    del Wd, q, choice
    return out


def check(W16, grid, nbits, g, iters=20, exact=True, meta="f64", axis=1, **kw):
    o = oracle.get()
    ref = o.quantize_v2(W16.astype(np.float64), grid, nbits=nbits, group_size=g, iters=iters, axis=axis, **kw)
    gq = gpu_v2(W16, grid, nbits, g, iters, meta=meta, axis=axis, **kw)
    N = W16.size
    G = N // g
    codes = o.unpack(gq["packed"], N, nbits)
    assert np.array_equal(o.pack(codes, nbits), gq["packed"][:o.packed_bytes(N, nbits)])
    if meta == "f16":
        assert np.array_equal(gq["delta"].view(np.uint16), ref["delta16"])
        assert np.array_equal(gq["zero"].view(np.uint16), ref["zero16"])
    elif meta == "f32":
        assert np.array_equal(gq["delta"], ref["delta"].astype(np.float32))
        assert np.array_equal(gq["zero"], ref["z"].astype(np.float32))
    if exact:
        assert np.array_equal(gq["choice"][:G], ref["choice"]), "choices differ"
        assert np.array_equal(codes, ref["codes"].reshape(-1)), "codes differ"
        if meta == "f64":
            assert np.array_equal(gq["delta"][:G], ref["delta"]) and np.array_equal(gq["zero"][:G], ref["z"])
    else:
        # an active shrink evaluates pow() on both sides, which may differ in the last bit
        assert np.mean(gq["choice"][:G] == ref["choice"]) >= 0.999
        assert np.mean(codes == ref["codes"].reshape(-1)) >= CODE_AGREEMENT
        same = gq["choice"][:G] == ref["choice"]
        z = np.asarray(gq["zero"][:G], dtype=np.float64)[same]
        err = np.abs(z - ref["z"][same]) / np.maximum(np.abs(ref["z"][same]), 1.0)
        assert err.max() <= Z_TOL
    return ref, gq


# several tiles of groups and a ragged last one (rows chosen so the group count is odd)
CASES = [(4, 64, 37, 128), (2, 16, 29, 192), (4, 32, 33, 256), (4, 128, 21, 512), (2, 256, 11, 512),
         (2, 64, 45, 320), (4, 16, 17, 64), (3, 64, 37, 128), (3, 32, 19, 160), (3, 16, 23, 48)]


@pytest.mark.parametrize("nbits,g,rows,cols", CASES)
@pytest.mark.parametrize("grid", [[1.0], GRID3, GRID5, GRID16], ids=["c1", "c3", "c5", "c16"])
def test_scale_search_parity(nbits, g, rows, cols, grid):
    say("scale search", nbits, g, rows, cols, len(grid))
    W = synth.weight_normal(rows, cols, 0.02, seed=rows + cols + g, outlier_frac=0.002, outlier_k=10.0)
    ref, _ = check(W, grid, nbits, g)
    if len(grid) > 1:
        assert len(set(ref["choice"].tolist())) > 1  # the inputs make the grid matter


# axis 0: (rows / g) * cols groups, a multiple of 8, with a ragged last tile of columns
CASES_AX0 = [(4, 64, 128, 40), (2, 16, 48, 56), (3, 32, 96, 24), (4, 128, 256, 24), (4, 256, 256, 40)]


@pytest.mark.parametrize("nbits,g,rows,cols", CASES_AX0)
@pytest.mark.parametrize("grid", [[1.0], GRID5], ids=["c1", "c5"])
def test_scale_search_axis0_parity(nbits, g, rows, cols, grid):
    say("scale search axis 0", nbits, g, rows, cols, len(grid))
    W = synth.weight_normal(rows, cols, 0.02, seed=rows * cols + g, outlier_frac=0.002, outlier_k=10.0)
    check(W, grid, nbits, g, axis=0)


@pytest.mark.parametrize("meta", ["f16", "f32"])
def test_scale_search_stored_metadata(meta):
    say("scale search metadata", meta)
    W = synth.weight_normal(24, 256, 0.02, seed=41)
    check(W, GRID5, 4, 64, meta=meta)


@pytest.mark.parametrize("iters", [0, 1, 2, 20])
@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_scale_search_edge_cases(nbits, iters):
    """Constant and zero groups, a tiny range, the 2e4 limit (multipliers above 1 push more
    groups against it), sigma-1 rows where the shrink is active, outliers, exact ties."""
    say("scale search edge", nbits, iters)
    W = edge_tensor()
    shrink_rows = (nbits == 2 or iters > 1)
    check(W, GRID5 + [2.0, 40.0], nbits, 64, iters=iters, exact=not shrink_rows)
    # the rows without sigma-1 values are exact at every setting
    Wq = np.concatenate([W[:2], W[6:]], axis=0)
    check(Wq, GRID5 + [2.0, 40.0], nbits, 64, iters=iters)


def test_scale_search_other_parameters():
    say("scale search p / beta / kappa / tiny")
    W = synth.weight_normal(40, 128, 0.02, seed=12, outlier_frac=0.01, outlier_k=8.0)
    for p, b0, k, tiny in [(1.0, 10.0, 1.01, 1e-4), (0.5, 3.0, 1.2, 1e-3), (0.9, 50.0, 0.95, 0.0)]:
        o = oracle.get()
        ref = o.quantize_v2(W.astype(np.float64), GRID3, nbits=4, group_size=32, iters=12, p=p, beta0=b0, kappa=k,
                            tiny=tiny)
        gq = gpu_v2(W, GRID3, 4, 32, 12, p=p, beta0=b0, kappa=k, tiny_range=tiny)
        codes = o.unpack(gq["packed"], W.size, 4)
        assert np.array_equal(gq["choice"][:ref["choice"].size], ref["choice"])
        assert np.array_equal(codes, ref["codes"].reshape(-1))
        assert np.array_equal(gq["zero"][:ref["z"].size], ref["z"])


def test_scale_search_full_layer_sampled():
    """A 4096 x 4096 layer (the Llama-7B projection shape) with five multipliers, in the launch
    the bench times; rows sampled across the tensor are compared with the oracle run on those
    rows alone (axis-1 groups never cross rows, so each row's groups are independent)."""
    say("scale search 4096x4096 sampled")
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    W = synth.weight_normal(4096, 4096, 0.02, seed=1, outlier_frac=0.001, outlier_k=10.0)
    Wd = torch.from_numpy(W).cuda()
    q, choice = hq.hqq_quantize_v2(Wd, GRID5, nbits=4, group_size=64, meta_dtype=torch.float64)
    torch.cuda.synchronize()
    packed, z, ch = q.packed.cpu().numpy(), q.zero.cpu().numpy(), choice.cpu().numpy()
    o = oracle.get()
    rows = [0, 1, 777, 2048, 3001, 4095]
    gpr = 4096 // 64
    for r in rows:
        ref = o.quantize_v2(W[r:r + 1].astype(np.float64), GRID5, nbits=4, group_size=64)
        got = o.unpack(packed[r * 2048:(r + 1) * 2048], 4096, 4)
        assert np.array_equal(got, ref["codes"].reshape(-1)), r
        assert np.array_equal(z[r * gpr:(r + 1) * gpr], ref["z"]), r
        assert np.array_equal(ch[r * gpr:(r + 1) * gpr], ref["choice"]), r
    # every multiplier is chosen somewhere, and only indices of the grid appear
    assert ch.max() < len(GRID5) and len(np.unique(ch)) == len(GRID5)
