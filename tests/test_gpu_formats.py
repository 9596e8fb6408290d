"""GPU parity of the fused product for the other stored formats (hqq_gemv): 4-bit with
axis-0 groups, 3-bit (ten codes per 32-bit word, rows starting inside words) and 2-bit with
axis-1 groups of 16, against the oracle's fp64 product of the same stored codes and fp16
metadata.

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


def test_axis0_full_shape():
    """The 70B-MLP shape of the axis-0 quantizer workload: 28672 x 8192, g = 128."""
    N, K = 28672, 8192
    sel = np.sort(np.random.default_rng(7).choice(N, 384, replace=False))
    _check(N, K, 4, 128, 0, (1,), seed=3001, rows_sel=sel)


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
    with pytest.raises(hq.HQQError):  # batch 3 is not fused for these formats
        hq.hqq_gemv(pk, md, md, 64, 128, 4, 16, 0, torch.zeros((3, 128), dtype=torch.float16, device="cuda"))


# ---------------------------------------------------------------- batched product (hqq_gemm)
# 3-bit rows start at word slot n K mod 10: K = 512, 1024, 1536, 2048, 4096 give every even
# residue; batches 3 .. 300 span one and two 256-row blocks; N from one to four 128-row tiles
GEMM_CASES = [(3, 64, 128, 512, 3), (3, 16, 256, 1024, 9), (3, 32, 384, 2048, 100), (3, 128, 128, 1536, 256),
              (3, 256, 512, 4096, 300), (2, 16, 128, 512, 5), (2, 32, 256, 1024, 64), (2, 16, 384, 4096, 257),
              (2, 128, 128, 2048, 17), (2, 256, 256, 1536, 40), (4, 64, 256, 1024, 33), (4, 128, 128, 512, 3)]


def _check_gemm(nbits, g, N, K, batch, seed, rows_sel=None):
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    o = oracle.get()
    packed, delta, zero = _operands(seed, N, K, nbits, g, 1)
    x = np.random.default_rng(seed + 1).normal(0, 1, (batch, K)).astype(np.float16)
    yr = o.gemv_fmt(packed, delta.astype(np.float64), zero.astype(np.float64), N, K, nbits, g, 1,
                    x.astype(np.float64), rows_sel=rows_sel)
    scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
    pk, dl, zr = (torch.from_numpy(a).cuda() for a in (packed, delta, zero))
    for out_dtype in (torch.float32, torch.float16):
        y = hq.hqq_gemm(pk, dl, zr, N, K, nbits, g, 1, torch.from_numpy(x).cuda(),
                        out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
        yg = y if rows_sel is None else y[:, rows_sel]
        err = float(np.max(np.abs(yg - yr) / scale))
        say("  gemm N=%d K=%d b%d g%d batch=%d %s: max rel err %.3g" % (N, K, nbits, g, batch, out_dtype, err))
        assert err <= GEMV_TOL


@pytest.mark.parametrize("nbits,g,N,K,batch", GEMM_CASES, ids=lambda v: str(v))
def test_gemm_formats(nbits, g, N, K, batch):
    _check_gemm(nbits, g, N, K, batch, seed=4000 + 7 * nbits + g + N + K + batch)


@pytest.mark.parametrize("nbits,g", [(3, 64), (2, 16)])
def test_gemm_formats_full_shape(nbits, g):
    """The 11008 x 4096 projection of the 3-bit and 2-bit layer sets at batch 256 (sampled rows)."""
    sel = np.sort(np.random.default_rng(10 + nbits).choice(11008, 256, replace=False))
    _check_gemm(nbits, g, 11008, 4096, 256, seed=4500 + nbits, rows_sel=sel)


def test_gemm_formats_rejected():
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    pk = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    md = torch.zeros(1 << 14, dtype=torch.float16, device="cuda")
    x = torch.zeros((4, 512), dtype=torch.float16, device="cuda")
    for nbits, g, axis, N, K in ((3, 64, 0, 128, 512), (4, 32, 1, 128, 512), (2, 16, 1, 64, 512), (3, 16, 1, 128, 256),
                                 (2, 512, 1, 128, 512), (5, 64, 1, 128, 512)):
        with pytest.raises(hq.HQQError):
            hq.hqq_gemm(pk, md, md, N, K, nbits, g, axis, x[:, :K].contiguous())
