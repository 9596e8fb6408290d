"""GPU parity at small sizes: the HIP path through the C ABI against the fp64 oracle, element by
element, for every format, both axes, several tiles with a ragged tail, and the edge cases."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import (GEMV_TOL, assert_zero_close, compare_quant, gpu_quantize, say, torch_dev)

pytestmark = pytest.mark.gpu


def weights(rows, cols, seed, sigma=0.02, frac=0.001, k=10.0):
    return synth.weight_normal(rows, cols, sigma, seed, frac, k)


# shapes: several solve blocks and a partial last block (axis=1: 32 groups per block at g=64;
# axis=0: 64 groups per block at g <= 32, 32 at g=64, 16 at g >= 128).  Axis-0 tile counts of 25,
# 13 and 13 (g = 128, 64 and the 3-bit 128) take both branches of the XCD tile order (eight
# contiguous ranges, then the remainder in place); the other axis-0 shapes (4 to 6 tiles) keep
# every tile in place.
CASES = [
    # nbits, g, axis, rows, cols
    (4, 64, 1, 37, 192),
    (4, 16, 1, 29, 96),
    (4, 32, 1, 33, 160),
    (4, 128, 1, 17, 384),
    (4, 256, 1, 9, 512),
    (3, 64, 1, 37, 192),
    (3, 16, 1, 23, 80),
    (2, 16, 1, 37, 192),
    (2, 64, 1, 21, 128),
    (4, 128, 0, 256, 200),
    (4, 64, 0, 192, 136),
    (4, 16, 0, 48, 120),
    (2, 16, 0, 64, 72),
    (3, 128, 0, 256, 104),
    (3, 32, 0, 96, 88),
    (2, 256, 0, 256, 64),
]


@pytest.mark.parametrize("nbits,g,axis,rows,cols", CASES)
def test_quantize_parity(nbits, g, axis, rows, cols):
    say("quantize parity", nbits, g, axis, rows, cols)
    W = weights(rows, cols, seed=1000 + rows + cols + nbits)
    ref = oracle.get().quantize(W.astype(np.float64), nbits=nbits, group_size=g, axis=axis, iters=20)
    gq = gpu_quantize(W, nbits, g, axis, 20, meta="f64")
    compare_quant(W, ref, gq, nbits, g, axis)


@pytest.mark.parametrize("meta", ["f16", "f32"])
def test_stored_metadata_rounding(meta):
    """fp16 / fp32 metadata are the nearest-even roundings of the solver's fp64 values."""
    say("metadata rounding", meta)
    W = weights(64, 256, seed=77)
    g64 = gpu_quantize(W, 4, 64, 1, 20, meta="f64")
    gm = gpu_quantize(W, 4, 64, 1, 20, meta=meta)
    if meta == "f16":
        o = oracle.get()
        assert np.array_equal(gm["zero"].view(np.uint16), o.to_half_bits(g64["zero"]))
        assert np.array_equal(gm["delta"].view(np.uint16), o.to_half_bits(g64["delta"]))
    else:
        assert np.array_equal(gm["zero"], g64["zero"].astype(np.float32))
        assert np.array_equal(gm["delta"], g64["delta"].astype(np.float32))
    assert np.array_equal(gm["packed"], g64["packed"])


def edge_tensor():
    """Groups of 64 (axis=1) with: constants, zeros, a tiny range (s = 1), a range that hits
    the 2e4 limit, sigma-1 values (shrink active at 2 bits), single outliers, exact ties."""
    r = np.random.default_rng(5)
    rows, cols = 16, 128
    W = r.normal(0, 0.02, (rows, cols))
    W[0, :64] = 0.375
    W[0, 64:] = 0.0
    W[1, :64] = 0.01 + r.uniform(0, 5e-5, 64)
    W[1, 64:] = 0.5 + r.uniform(0, 3e-4, 64)
    W[2:6] = r.normal(0, 1.0, (4, cols))
    W[6, 5] = 0.9
    W[7, 70] = -1.3
    W[8, :64] = np.arange(64) / 4.0
    return W.astype(np.float16)


@pytest.mark.parametrize("nbits", [2, 3, 4])
@pytest.mark.parametrize("iters", [0, 1, 2, 20])
def test_edge_cases(nbits, iters):
    say("edge cases", nbits, iters)
    W = edge_tensor()
    ref = oracle.get().quantize(W.astype(np.float64), nbits=nbits, group_size=64, axis=1, iters=iters)
    gq = gpu_quantize(W, nbits, 64, 1, iters, meta="f64")
    # rows 2-5 hold sigma-1 values: the shrink is active there, and pow() may differ in its last
    # bit between the two sides, so zeros are held to the tolerance rather than bit for bit
    compare_quant(W, ref, gq, nbits, 64, 1, exact=(iters <= 1), exact_codes=(nbits != 2))


def test_shrink_active_parity():
    """sigma = 1 weights at 2 bits: residuals above the shrink threshold in every round."""
    say("shrink active")
    W = synth.weight_normal(48, 256, 1.0, seed=9)
    ref = oracle.get().quantize(W.astype(np.float64), nbits=2, group_size=64, axis=1, iters=20)
    gq = gpu_quantize(W, 2, 64, 1, 20, meta="f64")
    compare_quant(W, ref, gq, 2, 64, 1, exact_codes=False, exact=False)


def test_other_solver_parameters():
    say("other p / beta / kappa")
    W = synth.weight_normal(40, 128, 0.5, seed=10)
    for p, b0, k in [(1.0, 10.0, 1.01), (0.5, 3.0, 1.2), (0.9, 50.0, 0.95)]:
        ref = oracle.get().quantize(W.astype(np.float64), nbits=3, group_size=32, axis=1, iters=12, p=p, beta0=b0,
                                    kappa=k)
        gq = gpu_quantize(W, 3, 32, 1, 12, p=p, beta0=b0, kappa=k, meta="f64")
        compare_quant(W, ref, gq, 3, 32, 1, exact_codes=False, exact=False)


def test_repeat_calls_deterministic():
    say("determinism")
    W = weights(64, 512, seed=12)
    a = gpu_quantize(W, 4, 64, 1, 20, meta="f64")
    b = gpu_quantize(W, 4, 64, 1, 20, meta="f64")
    for k in ("packed", "delta", "zero"):
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(a["mae"], b["mae"], equal_nan=True) and a["stop"] == b["stop"]


# ---------------------------------------------------------------------------- dequantisation

# every fused form: 4-/2-bit axis 1, 4-bit axis 0, 2-bit axis 0 with (rows/g) cols a multiple of 16
# (and the general kernel when it is not), 3-bit axis 1 with two or three groups per 40 codes and
# a ragged end, and the general 3-bit axis-0 kernel
DQ_CASES = [(4, 64, 1, 37, 192), (4, 128, 0, 256, 200), (3, 64, 1, 37, 192), (3, 16, 0, 48, 120),
            (2, 16, 1, 37, 192), (2, 32, 0, 96, 88), (4, 16, 1, 13, 48), (2, 32, 0, 64, 96),
            (4, 16, 0, 32, 40), (3, 16, 1, 13, 48), (3, 32, 1, 7, 96), (3, 256, 1, 5, 256), (2, 64, 1, 9, 320)]


@pytest.mark.parametrize("nbits,g,axis,rows,cols", DQ_CASES)
@pytest.mark.parametrize("meta", ["f16", "f32"])
def test_dequant_bit_exact(nbits, g, axis, rows, cols, meta):
    """GPU dequantisation of the oracle's packed codes and stored metadata equals the oracle's
    nearest-even fp16 of the exact (q - z) * delta."""
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    say("dequant", nbits, g, axis, rows, cols, meta)
    o = oracle.get()
    W = weights(rows, cols, seed=2000 + rows)
    ref = o.quantize(W.astype(np.float64), nbits=nbits, group_size=g, axis=axis, iters=20)
    packed = o.pack(ref["codes"], nbits)
    if meta == "f16":
        d = ref["delta16"].view(np.float16)
        z = ref["zero16"].view(np.float16)
    else:
        d = ref["delta"].astype(np.float32)
        z = ref["z"].astype(np.float32)
    _, w16 = o.dequant(packed, d, z, rows, cols, nbits, g, axis)
    out = hq.hqq_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(z).cuda(),
                            rows, cols, nbits, g, axis)
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, w16), int((got != w16).sum())


def test_dequant_synthetic_extremes():
    """Random codes with metadata across fp16's range (subnormal steps, large and negative
    zeros): still the nearest-even fp16 of the exact product."""
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    say("dequant extremes")
    o = oracle.get()
    r = np.random.default_rng(3)
    rows, cols, g = 64, 256, 64
    G = rows * cols // g
    codes = r.integers(0, 16, (rows, cols)).astype(np.uint8)
    d = np.concatenate([r.uniform(5e-5, 6e-5, G // 4), r.uniform(1e-3, 0.1, G // 4), r.uniform(1, 30, G // 4),
                        r.uniform(1e-7, 5e-6, G - 3 * (G // 4))]).astype(np.float16)
    z = np.concatenate([r.uniform(-100, 100, G // 2), r.uniform(0, 15, G - G // 2)]).astype(np.float16)
    packed = o.pack(codes, 4)
    _, w16 = o.dequant(packed, d, z, rows, cols, 4, g, 1)
    out = hq.hqq_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(d).cuda(), torch.from_numpy(z).cuda(),
                            rows, cols, 4, g, 1)
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, w16), int((got != w16).sum())


# ---------------------------------------------------------------------------- fused product

def gemv_inputs(N, K, g, seed):
    o = oracle.get()
    W = weights(N, K, seed=seed, frac=0.0)
    ref = o.quantize(W.astype(np.float64), nbits=4, group_size=g, axis=1, iters=20)
    return o.pack(ref["codes"], 4), ref["delta16"].view(np.float16), ref["zero16"].view(np.float16)


def check_gemv(packed, d16, z16, N, K, g, x, out_f32, rows_sel=None):
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    o = oracle.get()
    y = hq.hqq_gemv_w4a16(torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(),
                          torch.from_numpy(z16).cuda(), N, K, g, torch.from_numpy(x).cuda(),
                          out_dtype=torch.float32 if out_f32 else torch.float16)
    yg = y.float().cpu().numpy().astype(np.float64)
    yr = o.gemv(packed, d16, z16, N, K, g, x.astype(np.float64), rows_sel=rows_sel)
    if rows_sel is not None:
        yg = yg[:, rows_sel]
    scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
    err = np.abs(yg - yr) / scale
    assert err.max() <= GEMV_TOL, "max rel err %.3g" % err.max()
    return float(err.max())


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 7, 8, 9, 16, 33, 130])
def test_gemv_parity(g, batch):
    say("gemv", g, batch)
    N, K = 96, 1152  # 9 chunks of 128 codes: uneven over the 8 waves of a block
    packed, d16, z16 = gemv_inputs(N, K, g, seed=3000 + g)
    x = synth.activations(batch, K, seed=11)
    check_gemv(packed, d16, z16, N, K, g, x, out_f32=True)
    check_gemv(packed, d16, z16, N, K, g, x, out_f32=False)


@pytest.mark.parametrize("K", [2048, 4224, 8192, 16384])
@pytest.mark.parametrize("batch", [1, 2, 8])
def test_gemv_parity_long_rows(K, batch):
    """Long rows: several chunks per lane in the row-streaming kernel, ragged last chunk set."""
    say("gemv long rows", K, batch)
    N = 48
    packed, d16, z16 = gemv_inputs(N, K, 64, seed=4000 + K)
    x = synth.activations(batch, K, seed=13)
    check_gemv(packed, d16, z16, N, K, 64, x, out_f32=True)


@pytest.mark.parametrize("N,K,batch", [(12320, 256, 1), (8224, 256, 1), (8208, 384, 1), (4112, 512, 1),
                                       (4096, 256, 2), (8192, 128, 2), (1040, 640, 1)])
def test_gemv_parity_rows_per_wave(N, K, batch):
    """The row-streaming GEMV's wave shapes: 8 consecutive rows per wave (N a multiple of 32 with
    at least 256 blocks whose last round of 256 holds more than 96: N = 12320, 385 blocks), 4
    (N / 16 >= 256, and N = 8224, whose 8-row grid would leave 1 block in its last round), 2
    otherwise; every row of every wave checked."""
    say("gemv rows per wave", N, K, batch)
    packed, d16, z16 = gemv_inputs(N, K, 64, seed=4200 + N + K)
    x = synth.activations(batch, K, seed=23)
    check_gemv(packed, d16, z16, N, K, 64, x, out_f32=True)


def random_w4(N, K, g, seed):
    """Stored 4-bit operands drawn directly (codes U{0..15}, steps U(1e-3, 5e-2), zeros U(0, 15),
    fp16), packed by the oracle: sizes past what the oracle quantizer finishes in seconds."""
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, N * K).astype(np.uint8)
    d16 = r.uniform(1e-3, 5e-2, N * K // g).astype(np.float16)
    z16 = r.uniform(0, 15, N * K // g).astype(np.float16)
    return oracle.get().pack(codes, 4), d16, z16


def sampled_rows(N, seed, n=384):
    """The first and last 32 rows, and n random ones."""
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N), r.choice(N, n, replace=False)]))


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("N,K,batch", [(8192, 2176, 6), (8192, 2304, 3), (4112, 4224, 5), (16384, 1152, 8),
                                       (11008, 4096, 4), (4096, 10240, 5), (32, 20480, 1), (32, 18432, 2)])
def test_gemv_parity_mfma_blocks(g, N, K, batch):
    """The batched MFMA GEMV that keeps codes exact (batch 3-8 past 2^24 weights): two 16-row
    strips per block (N = 8192, 16384), one strip (N = 4112, and N = 11008, where a two-strip grid
    would leave its last round of 256 blocks at 88), 8-wave blocks with two to five 1024-code
    segments and a partial last one, 16-wave blocks in the run-time segment loop (K = 10240); and
    batch 1-2 rows longer than the streaming kernel takes."""
    say("gemv mfma", g, N, K, batch)
    if N * K > (1 << 24):
        packed, d16, z16 = random_w4(N, K, g, seed=4100 + N + K)
        sel = sampled_rows(N, seed=N + K)
    else:
        packed, d16, z16 = gemv_inputs(N, K, g, seed=4100 + N + K)
        sel = None
    x = synth.activations(batch, K, seed=19)
    check_gemv(packed, d16, z16, N, K, g, x, out_f32=True, rows_sel=sel)
    check_gemv(packed, d16, z16, N, K, g, x, out_f32=False, rows_sel=sel)


@pytest.mark.parametrize("N,K,batch", [(4096, 4096, 8), (4112, 4096, 8), (2048, 8192, 3), (8192, 8192, 16),
                                       (8192, 8192, 9), (8320, 8192, 9), (11008, 4096, 12), (4096, 11008, 16)])
def test_gemv_w4a16_size_paths(N, K, batch):
    """hqq_gemv_w4a16 on both sides of its size thresholds: batch 3-8 up to 2^24 weights and batch
    9-16 up to 2^26 dequantise in registers into the MFMA; 4112 x 4096 at batch 8 keeps the exact-code
    GEMV, 8320 x 8192 at batch 9 the split GEMM; the 7B projections at batch 12 and 16."""
    say("gemv_w4a16 size paths", N, K, batch)
    packed, d16, z16 = random_w4(N, K, 64, seed=4300 + N + K + batch)
    x = synth.activations(batch, K, seed=29)
    sel = sampled_rows(N, seed=K + batch, n=256)
    check_gemv(packed, d16, z16, N, K, 64, x, out_f32=True, rows_sel=sel)
    check_gemv(packed, d16, z16, N, K, 64, x, out_f32=False, rows_sel=sel)


def test_gemv_onehot_columns():
    """A one-hot activation row returns one column of W_hat (to fp32 rounding)."""
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    say("gemv one-hot")
    o = oracle.get()
    N, K, g = 64, 512, 64
    packed, d16, z16 = gemv_inputs(N, K, g, seed=55)
    w64, _ = o.dequant(packed, d16, z16, N, K, 4, g, 1)
    for batch in (1, 8, 24):
        ks = np.arange(batch) * 37 % K
        x = np.zeros((batch, K), np.float16)
        x[np.arange(batch), ks] = 1.0
        y = hq.hqq_gemv_w4a16(torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(),
                              torch.from_numpy(z16).cuda(), N, K, g, torch.from_numpy(x).cuda(),
                              out_dtype=torch.float32).cpu().numpy()
        ref = w64[:, ks].T
        assert np.allclose(y, ref, rtol=2e-3, atol=2e-3 * np.abs(ref).max())


# ---------------------------------------------------------------------------- split-K GEMM

def check_gemm(packed, d16, z16, N, K, g, x, out_f32, rows_sel=None, workspace=None):
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    o = oracle.get()
    y = hq.hqq_gemm_w4a16(torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(),
                          torch.from_numpy(z16).cuda(), N, K, g, torch.from_numpy(x).cuda(),
                          out_dtype=torch.float32 if out_f32 else torch.float16, workspace=workspace)
    yg = y.float().cpu().numpy().astype(np.float64)
    yr = o.gemv(packed, d16, z16, N, K, g, x.astype(np.float64), rows_sel=rows_sel)
    if rows_sel is not None:
        yg = yg[:, rows_sel]
    scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
    err = np.abs(yg - yr) / scale
    assert err.max() <= GEMV_TOL, "max rel err %.3g" % err.max()
    return float(err.max())


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("N,K,batch", [(128, 512, 9), (256, 1024, 100), (384, 2048, 256), (128, 4096, 300),
                                       (1024, 512, 37), (128, 1536, 513)])
def test_gemm_split_parity(g, N, K, batch):
    """Split-K GEMM: one or several K splits (the split count depends on the tile count), a
    ragged batch inside one 256-row block and over two and three blocks."""
    say("gemm split", g, N, K, batch)
    packed, d16, z16 = gemv_inputs(N, K, g, seed=5000 + N + K)
    x = synth.activations(batch, K, seed=17)
    check_gemm(packed, d16, z16, N, K, g, x, out_f32=True)
    check_gemm(packed, d16, z16, N, K, g, x, out_f32=False)


def test_gemm_split_errors():
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    pk = torch.zeros(128 * 512 // 2, dtype=torch.uint8, device="cuda")
    md = torch.zeros(128 * 512 // 64, dtype=torch.float16, device="cuda")
    x = torch.zeros((16, 512), dtype=torch.float16, device="cuda")
    need = hq.hqq_gemm_workspace_bytes(128, 512, 16)
    assert need > 0 and hq.hqq_gemm_workspace_bytes(120, 512, 16) == 0 and hq.hqq_gemm_workspace_bytes(128, 384, 16) == 0
    with pytest.raises(hq.HQQError):  # workspace too small
        hq.hqq_gemm_w4a16(pk, md, md, 128, 512, 64, x, workspace=torch.empty(need - 256, dtype=torch.uint8,
                                                                                  device="cuda"))
    with pytest.raises(hq.HQQError):  # N not a multiple of 128
        hq.hqq_gemm_w4a16(pk, md, md, 64, 512, 64, x)


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("N,K,batch", [(384, 1280, 17), (128, 512, 64), (256, 2048, 300)])
def test_gemv_w4a16_split_path(g, N, K, batch):
    """Above batch 16, with N a multiple of 128 and K of 256, hqq_gemv_w4a16 runs the split GEMM on
    the workspace the library keeps for the stream: the oracle's values, and bit for bit the
    result of hqq_gemm_w4a16 with a caller's workspace."""
    import weight_only_quantization_amd as hq
    say("gemv_w4a16 split path", g, N, K, batch)
    torch = torch_dev()
    packed, d16, z16 = gemv_inputs(N, K, g, seed=5200 + N + K)
    x = synth.activations(batch, K, seed=19)
    check_gemv(packed, d16, z16, N, K, g, x, out_f32=True)
    args = (torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(), torch.from_numpy(z16).cuda(), N, K, g,
            torch.from_numpy(x).cuda())
    for dt in (torch.float32, torch.float16):
        a = hq.hqq_gemv_w4a16(*args, out_dtype=dt)
        b = hq.hqq_gemm_w4a16(*args, out_dtype=dt)
        assert torch.equal(a, b)


def test_gemv_w4a16_workspace_streams():
    """The library's workspaces: calls of different batches interleaved on two streams (one buffer
    each), a batch that outgrows a stream's buffer, then a release and a call that allocates
    again; every result equals the same call's result on the default stream."""
    import weight_only_quantization_amd as hq
    say("gemv_w4a16 workspaces on two streams")
    torch = torch_dev()
    N, K, g = 256, 1024, 64
    packed, d16, z16 = gemv_inputs(N, K, g, seed=5300)
    w = (torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(), torch.from_numpy(z16).cuda())
    xs = {b: torch.from_numpy(synth.activations(b, K, seed=23 + b)).cuda() for b in (16, 200, 700)}
    ref = {b: hq.hqq_gemv_w4a16(*w, N, K, g, xs[b], out_dtype=torch.float32) for b in xs}
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for b, st in ((16, s1), (200, s2), (200, s1), (16, s2), (700, s1 if rep else s2)):
            with torch.cuda.stream(st):
                outs.append((b, hq.hqq_gemv_w4a16(*w, N, K, g, xs[b], out_dtype=torch.float32, stream=st)))
    torch.cuda.synchronize()
    for b, y in outs:
        assert torch.equal(y, ref[b]), b
    hq.hqq_release_workspaces()
    y = hq.hqq_gemv_w4a16(*w, N, K, g, xs[200], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, ref[200])


# ---------------------------------------------------------------------------- input gradient

@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("N,K,batch", [(512, 256, 9), (1024, 384, 100), (512, 1024, 256), (2048, 128, 300),
                                       (1536, 512, 37)])
def test_gemm_dx_parity(g, N, K, batch):
    """dX = dY @ W_hat through the transposed split GEMM against the oracle's input gradient:
    one to sixteen splits of N, ragged batches over one and two 256-row blocks."""
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    say("gemm dx", g, N, K, batch)
    o = oracle.get()
    packed, d16, z16 = gemv_inputs(N, K, g, seed=6000 + N + K)
    dy = synth.activations(batch, N, seed=19)
    ref = o.gemv_t(packed, d16, z16, N, K, 4, g, 1, dy.astype(np.float64))
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    for out_dtype in (torch.float32, torch.float16):
        dx = hq.hqq_gemm_w4a16_dx(torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(),
                                  torch.from_numpy(z16).cuda(), N, K, g, torch.from_numpy(dy).cuda(),
                                  out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(dx - ref) / scale))
        assert err <= GEMV_TOL, "max rel err %.3g" % err


def test_gemm_dx_adjoint():
    """<dY, x W_hat^T> = <dY W_hat, x> between the GPU forward product and the GPU input gradient
    (both fp32 outputs), to fp32 accumulation error."""
    import weight_only_quantization_amd as hq
    torch = torch_dev()
    N, K, g = 1024, 512, 64
    packed, d16, z16 = gemv_inputs(N, K, g, seed=77)
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, d16, z16))
    x = torch.from_numpy(synth.activations(16, K, seed=21)).cuda()
    dy = torch.from_numpy(synth.activations(16, N, seed=22)).cuda()
    y = hq.hqq_gemm_w4a16(pk, dl, zr, N, K, g, x, out_dtype=torch.float32).double()
    dx = hq.hqq_gemm_w4a16_dx(pk, dl, zr, N, K, g, dy, out_dtype=torch.float32).double()
    lhs = (dy.double() * y).sum(dim=1)
    rhs = (dx * x.double()).sum(dim=1)
    assert torch.allclose(lhs, rhs, rtol=1e-4, atol=1e-3 * float(lhs.abs().max()))
