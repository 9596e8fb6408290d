"""Helpers shared by the GPU parity tests: running the HIP path through the C ABI on torch
device memory, and comparing with the oracle to the stated tolerances."""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

import oracle
import weight_only_quantization_amd as hq

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_workloads.json")

# Tolerances (zero and step: relative 1e-5 against max(|ref|, 1); integer codes: at least
# 99.99 % equal; GEMV: 2e-3 relative to max(|y_ref|, rms(y_ref)), fp32 accumulation).
Z_TOL = 1e-5
CODE_AGREEMENT = 0.9999
GEMV_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    hq.load()
    return torch


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def golden_records():
    with open(GOLDEN) as f:
        return json.load(f)["records"]


def golden_for(workload, tensor, nbits, g, axis):
    for r in golden_records():
        if (r["workload"], r["tensor"], r["nbits"], r["group_size"], r["axis"]) == (workload, tensor, nbits, g, axis):
            return r
    raise KeyError((workload, tensor, nbits, g, axis))


def gpu_quantize(W16: np.ndarray, nbits, g, axis, iters=20, p=0.7, beta0=10.0, kappa=1.01, meta="f64", **ex):
    """Quantize on the GPU; returns numpy copies of packed, delta, zero, stop index, MAE trace.
    `ex` (stop_rule, tiny_range, debug_flags) goes to hqq_quantize_ex."""
    torch = torch_dev()
    Wd = torch.from_numpy(np.ascontiguousarray(W16)).cuda()
    md = {"f16": torch.float16, "f32": torch.float32, "f64": torch.float64}[meta]
    q = hq.hqq_quantize(Wd, nbits=nbits, group_size=g, axis=axis, iters=iters, p=p, beta0=beta0, kappa=kappa,
                        meta_dtype=md, **ex)
    torch.cuda.synchronize()
    out = {"packed": q.packed.cpu().numpy(), "delta": q.delta.cpu().numpy(), "zero": q.zero.cpu().numpy(),
           "stop": int(q.stop_iter.cpu().numpy()[0]), "mae": q.mae_trace.cpu().numpy()}
    del Wd, q
    return out


def assert_zero_close(z_gpu, z_ref, what="zero"):
    z_gpu = np.asarray(z_gpu, dtype=np.float64)
    z_ref = np.asarray(z_ref, dtype=np.float64)
    err = np.abs(z_gpu - z_ref) / np.maximum(np.abs(z_ref), 1.0)
    assert err.max() <= Z_TOL, "%s: max rel err %.3g at %d" % (what, err.max(), int(err.argmax()))
    return float(err.max())


def compare_quant(W16, ref, gq, nbits, g, axis, exact_codes=True, exact=True):
    """Full comparison of a GPU quantisation with the whole-tensor oracle result.  With
    `exact`, the MAE trace, zeros and steps must also be bit-identical (both sides use the same
    summation order; only pow() in an active shrink may differ in its last bit)."""
    o = oracle.get()
    rows, cols = W16.shape
    N = rows * cols
    assert gq["stop"] == ref["kout"], (gq["stop"], ref["kout"])
    R = ref["rounds"]
    if R:
        rel = np.abs(gq["mae"][:R] - ref["mae"]) / np.maximum(np.abs(ref["mae"]), 1e-300)
        assert rel.max() <= 1e-12, rel
    iters = len(gq["mae"]) if R else 0
    if R < iters:
        assert np.isnan(gq["mae"][R:iters]).all(), gq["mae"]
    codes = o.unpack(gq["packed"], N, nbits)
    # packing layout: the GPU bytes are exactly the oracle's packing of the GPU codes
    assert np.array_equal(o.pack(codes, nbits), gq["packed"][:o.packed_bytes(N, nbits)])
    agree = float(np.mean(codes == ref["codes"].reshape(-1)))
    if exact_codes:
        assert agree == 1.0, agree
    assert agree >= CODE_AGREEMENT, agree
    assert np.array_equal(gq["delta"], ref["delta"]) or \
        np.max(np.abs(gq["delta"] - ref["delta"]) / ref["delta"]) <= Z_TOL
    assert_zero_close(gq["zero"], ref["z"])
    if exact:
        assert np.array_equal(gq["mae"][:R], ref["mae"]), "MAE trace not bit-identical"
        assert np.array_equal(gq["zero"], ref["z"]), "zeros not bit-identical"
        assert np.array_equal(gq["delta"], ref["delta"]), "steps not bit-identical"
    return agree
