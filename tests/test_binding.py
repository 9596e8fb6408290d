"""The Python binding checks every tensor operand before its pointer reaches the C ABI: the
library reads raw memory of the type the stored format implies (fp16 steps and zeros for the
fused products), so a wrong dtype, a short buffer or a host tensor would otherwise be read
silently.  These run on the CPU: each check raises before any device work."""
import pytest
import torch

import weight_only_quantization_amd as hq

N, K, G = 128, 512, 64


def ops(meta=torch.float16, packed_bytes=N * K // 2, meta_n=N * K // G, x_dtype=torch.float16, x_shape=(4, K)):
    return (torch.zeros(packed_bytes, dtype=torch.uint8), torch.zeros(meta_n, dtype=meta),
            torch.zeros(meta_n, dtype=meta), torch.zeros(x_shape, dtype=x_dtype))


@pytest.mark.parametrize("fn", ["gemv_w4a16", "gemm_w4a16", "gemv", "gemm"])
def test_product_operand_checks(fn):
    hq.load()

    def call(pk, d, z, x, out=None):
        if fn == "gemv_w4a16":
            return hq.hqq_gemv_w4a16(pk, d, z, N, K, G, x, out=out)
        if fn == "gemm_w4a16":
            return hq.hqq_gemm_w4a16(pk, d, z, N, K, G, x, out=out)
        if fn == "gemv":
            return hq.hqq_gemv(pk, d, z, N, K, 4, G, 1, x, out=out)
        return hq.hqq_gemm(pk, d, z, N, K, 4, G, 1, x, out=out)

    with pytest.raises(ValueError, match="delta must be torch.float16"):  # fp32 metadata misread as fp16
        call(*ops(meta=torch.float32))
    with pytest.raises(ValueError, match="x must be torch.float16"):
        call(*ops(x_dtype=torch.float32))
    with pytest.raises(ValueError, match="packed holds"):
        call(*ops(packed_bytes=N * K // 2 - 1))
    with pytest.raises(ValueError, match="(delta|zero) holds"):
        call(*ops(meta_n=N * K // G - 1))
    with pytest.raises(ValueError, match="2-D"):
        call(*ops(x_shape=(K,)))
    with pytest.raises(ValueError, match="x must be"):
        call(*ops(x_shape=(4, K + 8)))
    pk, d, z, x = ops()
    with pytest.raises(ValueError, match="out must have shape"):
        call(pk, d, z, x, out=torch.zeros((4, N + 1), dtype=torch.float16))
    with pytest.raises(ValueError, match="CUDA"):  # every check passed: host memory is refused last
        call(pk, d, z, x)


@pytest.mark.parametrize("fn", ["gemm_w4a16_dx", "gemm_dx"])
def test_gradient_operand_checks(fn):
    hq.load()
    pk, d, z, _ = ops()

    def call(dy, pk=pk, d=d, z=z, out=None):
        if fn == "gemm_w4a16_dx":
            return hq.hqq_gemm_w4a16_dx(pk, d, z, N, K, G, dy, out=out)
        return hq.hqq_gemm_dx(pk, d, z, N, K, 4, G, 1, dy, out=out)

    with pytest.raises(ValueError, match="dy must be torch.float16"):
        call(torch.zeros((4, N), dtype=torch.float32))
    with pytest.raises(ValueError, match="dy must be"):  # [batch, N], not [batch, K]
        call(torch.zeros((4, K), dtype=torch.float16))
    with pytest.raises(ValueError, match="delta must be torch.float16"):
        call(torch.zeros((4, N), dtype=torch.float16), d=d.float())
    with pytest.raises(ValueError, match="packed holds"):
        call(torch.zeros((4, N), dtype=torch.float16), pk=pk[:-1])
    with pytest.raises(ValueError, match="out must have shape"):  # dX is [batch, K]
        call(torch.zeros((4, N), dtype=torch.float16), out=torch.zeros((4, N), dtype=torch.float16))
    with pytest.raises(ValueError, match="CUDA"):
        call(torch.zeros((4, N), dtype=torch.float16))


def test_quantize_and_dequantize_checks():
    hq.load()
    with pytest.raises(ValueError, match="W must be torch.float16"):
        hq.hqq_quantize(torch.zeros((64, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        hq.hqq_quantize(torch.zeros((64, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="W must be torch.float16"):
        hq.hqq_quantize_v2(torch.zeros((64, 64), dtype=torch.float32), [1.0])
    pk, d, z, _ = ops()
    with pytest.raises(ValueError, match="zero must be torch.float16"):  # delta and zero share one type
        hq.hqq_dequantize(pk, d, z.float(), N, K, 4, G, 1)
    with pytest.raises(ValueError, match="delta must be"):
        hq.hqq_dequantize(pk, d.double(), z.double(), N, K, 4, G, 1)
    with pytest.raises(ValueError, match="packed holds"):
        hq.hqq_dequantize(pk[:-1], d, z, N, K, 4, G, 1)
    with pytest.raises(ValueError, match="CUDA"):
        hq.hqq_dequantize(pk, d.float(), z.float(), N, K, 4, G, 1)
