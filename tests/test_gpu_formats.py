"""GPU parity of the fused product for the other stored formats (hqq_gemv): 4-bit with
axis-0 groups, 3-bit (ten codes per 32-bit word, rows starting inside words) and 2-bit with
axis-1 groups of 16 (batch 1-2 on the dot-product units, 3-16 on the matrix units), against the
oracle's fp64 product of the same stored codes and fp16 metadata.

Inputs are seeded synthetic codes and metadata (steps U(1e-3, 5e-2), zeros U(0, 2^b - 1),
activations N(0, 1), all fp16), packed by the oracle; sizes span several lanes' chunks, a
ragged last chunk, every group size, and the full 28672 x 8192 axis-0 shape (sampled rows).
Tolerance: |y - y_ref| <= 2e-3 max(|y_ref|, rms(y_ref)).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_common import GEMV_TOL, say, torch_dev

pytestmark = pytest.mark.gpu


def _operands(seed, N, K, nbits, g, axis):
    r = np.random.default_rng(seed)
    o = oracle.get()
    G = N * K // g
    codes = r.integers(0, 2 ** nbits, N * K).astype(np.uint8)
    delta = r.uniform(1e-3, 5e-2, G).astype(np.float16)
    zero = r.uniform(0, 2 ** nbits - 1, G).astype(np.float16)
    packed = o.pack(codes, nbits)
    return packed, delta, zero


def _check(N, K, nbits, g, axis, batches, seed, rows_sel=None):
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    o = oracle.get()
    packed, delta, zero = _operands(seed, N, K, nbits, g, axis)
    X = np.random.default_rng(seed + 1).normal(0, 1, (max(batches), K)).astype(np.float16)
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    for B in batches:
        x = X[:B]
        yr = o.gemv_fmt(packed, delta.astype(np.float64), zero.astype(np.float64), N, K, nbits, g, axis,
                        x.astype(np.float64), rows_sel=rows_sel)
        scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
        for out_dtype in (torch.float32, torch.float16):
            y = hq.hqq_gemv(pk, dl, zr, N, K, nbits, g, axis, torch.from_numpy(x).cuda(),
                            out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
            yg = y if rows_sel is None else y[:, rows_sel]
            err = float(np.max(np.abs(yg - yr) / scale))
            say("  N=%d K=%d b%d g%d axis%d B=%d %s: max rel err %.3g" % (N, K, nbits, g, axis, B, out_dtype, err))
            assert err <= GEMV_TOL


AX0_CASES = [(16, 32, 256), (32, 64, 1056), (64, 128, 2048), (128, 256, 4096), (256, 512, 8192), (128, 384, 16384)]


@pytest.mark.parametrize("g,N,K", AX0_CASES, ids=lambda v: str(v))
def test_axis0_4bit(g, N, K):
    _check(N, K, 4, g, 0, (1, 2), seed=1000 + g + K)


# batch 3..8 (MFMA): one and two 16-row strips per block, one to five 2048-code segments and a
# ragged last segment (K = 1152, 10240)
AX0_MF_CASES = [(16, 64, 128), (32, 128, 1152), (64, 256, 2048), (128, 512, 4096), (256, 512, 8192),
                (128, 256, 10240)]


@pytest.mark.parametrize("g,N,K", AX0_MF_CASES, ids=lambda v: str(v))
def test_axis0_4bit_batched(g, N, K):
    _check(N, K, 4, g, 0, (3, 4, 5, 6, 7, 8), seed=1100 + g + K)


SHAPES_2B = [(16, 64), (48, 192), (64, 4160), (256, 4096), (32, 16384)]


@pytest.mark.parametrize("N,K", SHAPES_2B, ids=lambda v: str(v))
def test_2bit_g16(N, K):
    _check(N, K, 2, 16, 1, (1, 2), seed=2000 + N + K)


# 3-bit: every supported g; K with every residue of a row's start inside a word (K mod 10) and
# inside a 40-code superblock (K mod 40); one and two rows per wave (N mod 8); the smallest K;
# K at the largest span of one and of two superblocks per lane (2512, 2528)
CASES_3B = [(16, 12, 208), (32, 64, 800), (64, 40, 4096), (64, 20, 1216), (128, 48, 1152), (64, 16, 5056),
            (16, 100, 96), (256, 24, 8192), (64, 4, 640), (16, 4, 48), (16, 36, 2512), (32, 8, 2528)]


@pytest.mark.parametrize("g,N,K", CASES_3B, ids=lambda v: str(v))
def test_3bit(g, N, K):
    _check(N, K, 3, g, 1, (1, 2), seed=2500 + g + N + K)


def test_3bit_full_shape():
    """The 11008 x 4096 projection of the 3-bit layer set (g = 64)."""
    N, K = 11008, 4096
    sel = np.sort(np.random.default_rng(9).choice(N, 512, replace=False))
    _check(N, K, 3, 64, 1, (1, 2), seed=3003, rows_sel=sel)


# batch 3..16 (3/2-bit, the tile dequantised in registers into the MFMA): a block of 32 rows splits
# the K / 128 chunks among 8 waves (4 from 8192 rows on).  Cases: one chunk for 8 waves (seven
# empty runs), ragged strips (N = 40, 100, 8 rows), runs of unequal length (C = 5, 9, 86), every
# row-start slot of the 3-bit words (K mod 10 = 8, 6, 4, 2, 0 for K = 128 .. 640), every group
# size, and the longest rows the chunk counts take (3-bit 12288 codes, 2-bit 32768).
DQ_BATCHES = (3, 4, 5, 8, 9, 16)
CASES_DQ_3B = [(16, 16, 128), (32, 40, 256), (64, 100, 384), (128, 24, 512), (128, 48, 640), (64, 64, 1152),
               (16, 32, 4096), (256, 8, 8192), (64, 8, 12288)]


@pytest.mark.parametrize("g,N,K", CASES_DQ_3B, ids=lambda v: str(v))
def test_3bit_batched(g, N, K):
    _check(N, K, 3, g, 1, DQ_BATCHES, seed=2700 + g + N + K)


CASES_DQ_2B = [(16, 128), (40, 640), (100, 1152), (64, 4096), (48, 16384), (8, 32768)]


@pytest.mark.parametrize("N,K", CASES_DQ_2B, ids=lambda v: str(v))
def test_2bit_batched(N, K):
    _check(N, K, 2, 16, 1, DQ_BATCHES, seed=2800 + N + K)


@pytest.mark.parametrize("nbits,g", [(3, 64), (2, 16)], ids=["3bit_g64", "2bit_g16"])
def test_batched_full_shapes(nbits, g):
    """The 11008 x 4096 projection (4 waves per block) at batch 3, 8 and 16 and the 4096 x 11008 one
    (8 waves, runs of 10 and 11 chunks) at batch 8, sampled rows."""
    sel = np.sort(np.random.default_rng(10).choice(11008, 512, replace=False))
    _check(11008, 4096, nbits, g, 1, (3, 8, 16), seed=3010 + nbits, rows_sel=sel)
    sel = np.sort(np.random.default_rng(11).choice(4096, 384, replace=False))
    _check(4096, 11008, nbits, g, 1, (8,), seed=3020 + nbits, rows_sel=sel)


def test_axis0_full_shape():
    """The 70B-MLP shape of the axis-0 quantizer workload: 28672 x 8192, g = 128, batch 1 and 8."""
    N, K = 28672, 8192
    sel = np.sort(np.random.default_rng(7).choice(N, 384, replace=False))
    _check(N, K, 4, 128, 0, (1, 8), seed=3001, rows_sel=sel)


def test_2bit_full_shape():
    """The 11008 x 4096 projection of the 2-bit layer set."""
    N, K = 11008, 4096
    sel = np.sort(np.random.default_rng(8).choice(N, 512, replace=False))
    _check(N, K, 2, 16, 1, (1, 2), seed=3002, rows_sel=sel)


def test_unsupported_formats_rejected():
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    pk = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    md = torch.zeros(1024, dtype=torch.float16, device="cuda")
    x = torch.zeros((1, 128), dtype=torch.float16, device="cuda")
    for nbits, g, axis in ((3, 32, 0), (2, 32, 1), (2, 16, 0)):
        with pytest.raises(hq.HQQError):
            hq.hqq_gemv(pk, md, md, 64, 128, nbits, g, axis, x)
    with pytest.raises(hq.HQQError):  # 3-bit rows shorter than 40 codes
        hq.hqq_gemv(pk, md, md, 64, 32, 3, 16, 1, x[:, :32].contiguous())
    with pytest.raises(hq.HQQError):  # batch 17 is not fused for 3-bit codes
        hq.hqq_gemv(pk, md, md, 64, 128, 3, 16, 1, torch.zeros((17, 128), dtype=torch.float16, device="cuda"))
    with pytest.raises(hq.HQQError):  # batch 3..16: K a multiple of 128
        hq.hqq_gemv(pk, md, md, 16, 192, 2, 16, 1, torch.zeros((3, 192), dtype=torch.float16, device="cuda"))
    pk3 = torch.zeros(hq.load().hqq_packed_bytes(1, 24704, 3), dtype=torch.uint8, device="cuda")
    md3 = torch.zeros(24704 // 16, dtype=torch.float16, device="cuda")
    with pytest.raises(hq.HQQError):  # batch 3..16, 3-bit: rows past 24576 codes
        hq.hqq_gemv(pk3, md3, md3, 1, 24704, 3, 16, 1, torch.zeros((3, 24704), dtype=torch.float16, device="cuda"))
    with pytest.raises(hq.HQQError):  # nor batch 9 for axis-0 codes
        hq.hqq_gemv(pk, md, md, 64, 128, 4, 16, 0, torch.zeros((9, 128), dtype=torch.float16, device="cuda"))
    with pytest.raises(hq.HQQError):  # axis 0, batch 3..8: K a multiple of 128
        hq.hqq_gemv(pk, md, md, 64, 96, 4, 16, 0, torch.zeros((4, 96), dtype=torch.float16, device="cuda"))


# ---------------------------------------------------------------- batched product (hqq_gemm)
# 3-bit rows start at word slot n K mod 10: K = 512, 1024, 1536, 2048, 4096 give every even
# residue; batches 3 .. 300 span one and two 256-row blocks; N from one to four 128-row tiles
GEMM_CASES = [(3, 64, 128, 512, 3), (3, 16, 256, 1024, 9), (3, 32, 384, 2048, 100), (3, 128, 128, 1536, 256),
              (3, 256, 512, 4096, 300), (2, 16, 128, 512, 5), (2, 32, 256, 1024, 64), (2, 16, 384, 4096, 257),
              (2, 128, 128, 2048, 17), (2, 256, 256, 1536, 40), (4, 64, 256, 1024, 33), (4, 128, 128, 512, 3),
              # K / 256 pairs of chunks not a power of two: splits of unequal length
              (3, 64, 128, 1280, 20), (2, 16, 256, 768, 70), (4, 64, 256, 768, 40), (4, 128, 128, 256, 9)]


def _check_gemm(nbits, g, N, K, batch, seed, rows_sel=None, axis=1):
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    o = oracle.get()
    packed, delta, zero = _operands(seed, N, K, nbits, g, axis)
    x = np.random.default_rng(seed + 1).normal(0, 1, (batch, K)).astype(np.float16)
    yr = o.gemv_fmt(packed, delta.astype(np.float64), zero.astype(np.float64), N, K, nbits, g, axis,
                    x.astype(np.float64), rows_sel=rows_sel)
    scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    for out_dtype in (torch.float32, torch.float16):
        y = hq.hqq_gemm(pk, dl, zr, N, K, nbits, g, axis, torch.from_numpy(x).cuda(),
                        out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
        yg = y if rows_sel is None else y[:, rows_sel]
        err = float(np.max(np.abs(yg - yr) / scale))
        say("  gemm N=%d K=%d b%d g%d axis%d batch=%d %s: max rel err %.3g" % (N, K, nbits, g, axis, batch, out_dtype,
                                                                             err))
        assert err <= GEMV_TOL


@pytest.mark.parametrize("nbits,g,N,K,batch", GEMM_CASES, ids=lambda v: str(v))
def test_gemm_formats(nbits, g, N, K, batch):
    _check_gemm(nbits, g, N, K, batch, seed=4000 + 7 * nbits + g + N + K + batch)


@pytest.mark.parametrize("nbits,g,N,K", [(3, 64, 11008, 4096), (2, 16, 11008, 4096), (3, 64, 4096, 11008),
                                          (2, 16, 4096, 11008)], ids=lambda v: str(v))
def test_gemm_formats_full_shape(nbits, g, N, K):
    """The 11008 x 4096 and 4096 x 11008 projections of the 3-bit and 2-bit layer sets at batch
    256 (sampled rows); the second contracts over 43 pairs of chunks in 8 unequal splits."""
    sel = np.sort(np.random.default_rng(10 + nbits).choice(N, 256, replace=False))
    _check_gemm(nbits, g, N, K, 256, seed=4500 + nbits + K, rows_sel=sel)


def test_gemm_formats_rejected():
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    pk = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    md = torch.zeros(1 << 14, dtype=torch.float16, device="cuda")
    x = torch.zeros((4, 512), dtype=torch.float16, device="cuda")
    for nbits, g, axis, N, K in ((3, 64, 0, 128, 512), (4, 32, 1, 128, 512), (2, 16, 1, 64, 512), (3, 16, 1, 128, 384),
                                 (4, 512, 0, 512, 256), (4, 8, 0, 128, 512), (4, 64, 0, 64, 512),
                                 (2, 512, 1, 128, 512), (5, 64, 1, 128, 512)):
        with pytest.raises(hq.HQQError):
            hq.hqq_gemm(pk, md, md, N, K, nbits, g, axis, x[:, :K].contiguous())


# ------------------------------------------------------------ input gradient (hqq_gemm_dx)
# dX [batch, K] = dY [batch, N] @ W_hat, W [N, K]: the contraction N in pairs of 128-row chunks
# (one to eight, also counts that do not split evenly), output columns K in 128-column tiles
# whose 32-code pieces start at every even slot of a 3-bit word
DX_CASES = [(3, 64, 512, 128, 3), (3, 16, 256, 384, 9), (3, 32, 768, 256, 100), (3, 128, 1024, 640, 256),
            (3, 256, 2048, 512, 300), (2, 16, 512, 128, 5), (2, 32, 768, 384, 64), (2, 128, 1280, 256, 257),
            (2, 256, 256, 512, 17), (4, 64, 768, 256, 33), (4, 128, 512, 384, 3)]


def _check_dx(nbits, g, N, K, batch, seed, cols_sel=None, axis=1):
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    o = oracle.get()
    packed, delta, zero = _operands(seed, N, K, nbits, g, axis)
    dy = np.random.default_rng(seed + 1).normal(0, 1, (batch, N)).astype(np.float16)
    ref = o.gemv_t(packed, delta, zero, N, K, nbits, g, axis, dy.astype(np.float64), cols_sel=cols_sel)
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    for out_dtype in (torch.float32, torch.float16):
        dx = hq.hqq_gemm_dx(pk, dl, zr, N, K, nbits, g, axis, torch.from_numpy(dy).cuda(),
                            out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
        dxg = dx if cols_sel is None else dx[:, cols_sel]
        err = float(np.max(np.abs(dxg - ref) / scale))
        say("  dx N=%d K=%d b%d g%d axis%d batch=%d %s: max rel err %.3g" % (N, K, nbits, g, axis, batch, out_dtype,
                                                                           err))
        assert err <= GEMV_TOL


@pytest.mark.parametrize("nbits,g,N,K,batch", DX_CASES, ids=lambda v: str(v))
def test_gemm_dx_formats(nbits, g, N, K, batch):
    _check_dx(nbits, g, N, K, batch, seed=7000 + 7 * nbits + g + N + K + batch)


@pytest.mark.parametrize("nbits,g,N,K", [(3, 64, 11008, 4096), (2, 16, 11008, 4096), (3, 64, 4096, 11008),
                                          (4, 64, 11008, 4096)], ids=lambda v: str(v))
def test_gemm_dx_formats_full_shape(nbits, g, N, K):
    """Input gradients of the layer sets' projections at batch 256 (sampled columns); the
    11008-row weights contract over 43 pairs of chunks in unequal splits."""
    sel = np.sort(np.random.default_rng(20 + nbits).choice(K, 256, replace=False))
    _check_dx(nbits, g, N, K, 256, seed=7500 + nbits + N, cols_sel=sel)


@pytest.mark.parametrize("nbits,g", [(3, 32), (2, 16)])
def test_gemm_dx_formats_adjoint(nbits, g):
    """<dY, x W_hat^T> = <dY W_hat, x> between hqq_gemm and hqq_gemm_dx (fp32 outputs)."""
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    N, K, B = 768, 512, 24
    packed, delta, zero = _operands(90 + nbits, N, K, nbits, g, 1)
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    r = np.random.default_rng(91)
    x = torch.from_numpy(r.normal(0, 1, (B, K)).astype(np.float16)).cuda()
    dy = torch.from_numpy(r.normal(0, 1, (B, N)).astype(np.float16)).cuda()
    y = hq.hqq_gemm(pk, dl, zr, N, K, nbits, g, 1, x, out_dtype=torch.float32).double()
    dx = hq.hqq_gemm_dx(pk, dl, zr, N, K, nbits, g, 1, dy, out_dtype=torch.float32).double()
    lhs = (dy.double() * y).sum(dim=1)
    rhs = (dx * x.double()).sum(dim=1)
    assert torch.allclose(lhs, rhs, rtol=1e-4, atol=1e-4 * float(lhs.abs().max()))


def test_gemm_dx_formats_rejected():
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    pk = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    md = torch.zeros(1 << 14, dtype=torch.float16, device="cuda")
    for nbits, g, axis, N, K in ((3, 64, 0, 512, 128), (4, 32, 1, 512, 128), (2, 16, 1, 384, 128),
                                 (3, 16, 1, 512, 64), (2, 512, 1, 512, 512), (4, 512, 0, 512, 128), (2, 16, 0, 512, 128)):
        with pytest.raises(hq.HQQError):
            hq.hqq_gemm_dx(pk, md, md, N, K, nbits, g, axis, torch.zeros((4, N), dtype=torch.float16, device="cuda"))


# ------------------------------------- 4-bit axis-0 codes through the split GEMM (any batch)
# every group size; one to four row tiles; the metadata row n mod (N / g) cycles inside a tile
# (N / g < 128) or spans several tiles; batches over one and two 256-row blocks
AX0_GEMM_CASES = [(16, 128, 256, 9), (32, 256, 768, 40), (64, 384, 1024, 100), (128, 512, 2048, 256),
                  (256, 256, 512, 300), (128, 1024, 256, 17)]
AX0_DX_CASES = [(16, 256, 128, 5), (32, 768, 384, 64), (64, 512, 256, 257), (128, 1024, 640, 33), (256, 512, 128, 3)]


@pytest.mark.parametrize("g,N,K,batch", AX0_GEMM_CASES, ids=lambda v: str(v))
def test_gemm_axis0(g, N, K, batch):
    _check_gemm(4, g, N, K, batch, seed=8000 + g + N + K + batch, axis=0)


@pytest.mark.parametrize("g,N,K,batch", AX0_DX_CASES, ids=lambda v: str(v))
def test_gemm_dx_axis0(g, N, K, batch):
    _check_dx(4, g, N, K, batch, seed=8500 + g + N + K + batch, axis=0)


def test_gemm_axis0_full_shape():
    """The 28672 x 8192 g128 axis-0 weight at batch 256: the product on sampled rows and the
    input gradient on sampled columns."""
    r = np.random.default_rng(30)
    _check_gemm(4, 128, 28672, 8192, 256, seed=8900, rows_sel=np.sort(r.choice(28672, 256, replace=False)), axis=0)
    _check_dx(4, 128, 28672, 8192, 256, seed=8901, cols_sel=np.sort(r.choice(8192, 256, replace=False)), axis=0)


def test_gemm_axis0_adjoint():
    """<dY, x W_hat^T> = <dY W_hat, x> between hqq_gemm and hqq_gemm_dx on axis-0 codes."""
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    N, K, B, g = 768, 512, 24, 32
    packed, delta, zero = _operands(95, N, K, 4, g, 0)
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    r = np.random.default_rng(96)
    x = torch.from_numpy(r.normal(0, 1, (B, K)).astype(np.float16)).cuda()
    dy = torch.from_numpy(r.normal(0, 1, (B, N)).astype(np.float16)).cuda()
    y = hq.hqq_gemm(pk, dl, zr, N, K, 4, g, 0, x, out_dtype=torch.float32).double()
    dx = hq.hqq_gemm_dx(pk, dl, zr, N, K, 4, g, 0, dy, out_dtype=torch.float32).double()
    lhs = (dy.double() * y).sum(dim=1)
    rhs = (dx * x.double()).sum(dim=1)
    assert torch.allclose(lhs, rhs, rtol=1e-4, atol=1e-4 * float(lhs.abs().max()))
