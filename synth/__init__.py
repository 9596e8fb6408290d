"""Seeded synthetic inputs for the HQQ workloads (weights and activations).

Everything here draws numbers and rounds them to fp16; none of the quantizer's
arithmetic lives in this module.  The oracle and the GPU path both consume the
arrays it returns, so they see identical bits.

The drawing itself is in ``synth.c`` (counter-based SplitMix64 streams,
Box-Muller normals, inverse-CDF Laplace, Floyd's sampling for outlier
positions).  The values are rounded to fp16 once, with numpy's
round-to-nearest-even conversion.

Workloads (shapes and distributions):
  * ``single_1024``   one 1024x1024 weight, N(0, 0.02) with 0.1 % of the
    entries replaced by +/-10 sigma.
  * ``llama7b_layers`` q/k/v/o 4096x4096 and three 11008x4096 MLP weights,
    N(0, 0.02) with 0.1 % +/-10 sigma outliers.
  * ``llama7b_laplace`` the same seven shapes, Laplace(0, b=0.015).
  * ``mlp70b``        one 28672x8192 weight, N(0, 0.01) with 0.05 % of the
    entries at +/-12 sigma.
  * ``gemv8192``      one 8192x8192 weight, N(0, 0.02), and activations
    [256, 8192] drawn from N(0, 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

CHUNK = 1 << 24


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so with gcc (OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        p = ctypes.c_void_p
        lib.synth_normal.argtypes = [u64, u64, dbl, dbl, i64, i64, p]
        lib.synth_laplace.argtypes = [u64, u64, dbl, i64, i64, p]
        lib.synth_randint.argtypes = [u64, u64, u64, i64, p]
        lib.synth_outliers.argtypes = [u64, u64, i64, i64, p, p]
        lib.synth_outliers.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def normal_f64(seed: int, n: int, sigma: float = 1.0, mean: float = 0.0, stream: int = 0,
               start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal(seed, stream, mean, sigma, start, n, _ptr(out))
    return out


def laplace_f64(seed: int, n: int, b: float, stream: int = 0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_laplace(seed, stream, b, start, n, _ptr(out))
    return out


def randint(seed: int, n: int, bound: int, stream: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    _load().synth_randint(seed, stream, bound, n, _ptr(out))
    return out


def outlier_positions(seed: int, N: int, count: int, stream: int = 1):
    pos = np.empty(count, dtype=np.int64)
    sign = np.empty(count, dtype=np.int8)
    rc = _load().synth_outliers(seed, stream, N, count, _ptr(pos), _ptr(sign))
    if rc != 0:
        raise ValueError("outlier sampling failed (count > N or out of memory)")
    return pos, sign


def _fill_f16(n: int, draw_chunk) -> np.ndarray:
    """Fill an fp16 array chunk by chunk from fp64 draws (RNE rounding)."""
    out = np.empty(n, dtype=np.float16)
    for s in range(0, n, CHUNK):
        m = min(CHUNK, n - s)
        out[s:s + m] = draw_chunk(s, m).astype(np.float16)
    return out


def outlier_count(N: int, frac: float) -> int:
    return int(np.floor(frac * N + 0.5))


def weight_normal(rows: int, cols: int, sigma: float, seed: int, outlier_frac: float = 0.0,
                  outlier_k: float = 10.0) -> np.ndarray:
    """fp16 [rows, cols]: N(0, sigma), then round(frac*N) entries replaced by +/-k*sigma."""
    N = rows * cols
    w = _fill_f16(N, lambda s, m: normal_f64(seed, m, sigma=sigma, stream=0, start=s))
    cnt = outlier_count(N, outlier_frac)
    if cnt:
        pos, sign = outlier_positions(seed, N, cnt, stream=1)
        w[pos] = (sign.astype(np.float64) * (outlier_k * sigma)).astype(np.float16)
    return w.reshape(rows, cols)


def weight_laplace(rows: int, cols: int, b: float, seed: int) -> np.ndarray:
    N = rows * cols
    return _fill_f16(N, lambda s, m: laplace_f64(seed, m, b, stream=0, start=s)).reshape(rows, cols)


def activations(batch: int, K: int, seed: int) -> np.ndarray:
    return _fill_f16(batch * K, lambda s, m: normal_f64(seed, m, sigma=1.0, stream=0, start=s)).reshape(batch, K)


# --------------------------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Tensor:
    name: str
    rows: int
    cols: int
    seed: int
    kind: str            # "normal" | "laplace"
    sigma: float = 0.0   # normal sigma, or Laplace b
    outlier_frac: float = 0.0
    outlier_k: float = 0.0

    def make(self) -> np.ndarray:
        if self.kind == "normal":
            return weight_normal(self.rows, self.cols, self.sigma, self.seed, self.outlier_frac, self.outlier_k)
        if self.kind == "laplace":
            return weight_laplace(self.rows, self.cols, self.sigma, self.seed)
        raise ValueError(self.kind)


@dataclass(frozen=True)
class QuantParams:
    nbits: int
    group_size: int
    axis: int
    iters: int = 20
    p: float = 0.7
    beta0: float = 10.0
    kappa: float = 1.01


_LLAMA_SHAPES = [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
                 ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                 ("down_proj", 11008, 4096)]

WORKLOADS = {
    "single_1024": {
        "tensors": [Tensor("w", 1024, 1024, 1, "normal", 0.02, 0.001, 10.0)],
        "quant": [QuantParams(4, 64, 1)],
    },
    "llama7b_layers": {
        "tensors": [Tensor(n, r, c, 101 + i, "normal", 0.02, 0.001, 10.0)
                    for i, (n, r, c) in enumerate(_LLAMA_SHAPES)],
        "quant": [QuantParams(4, 64, 1)],
    },
    "llama7b_laplace": {
        "tensors": [Tensor(n, r, c, 201 + i, "laplace", 0.015) for i, (n, r, c) in enumerate(_LLAMA_SHAPES)],
        "quant": [QuantParams(3, 64, 1), QuantParams(2, 16, 1)],
    },
    "mlp70b": {
        "tensors": [Tensor("w", 28672, 8192, 301, "normal", 0.01, 0.0005, 12.0)],
        "quant": [QuantParams(4, 128, 0)],
    },
    "gemv8192": {
        "tensors": [Tensor("w", 8192, 8192, 401, "normal", 0.02)],
        "quant": [QuantParams(4, 64, 1)],
        "x_seed": 402,
        "batches": [1, 8, 256],
    },
}
