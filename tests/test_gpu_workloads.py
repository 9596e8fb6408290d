"""GPU parity on the five full-size workloads (synthetic, seeded): every tensor is quantized on
the GPU in the configuration the benchmark times, and compared with the oracle:

  * stop index: bit-exact with the whole-tensor oracle's (stored by
    tests/golden/make_oracle_golden.py); the MAE of each evaluated round to 1e-12;
  * codes and packing: the oracle's per-group steps with that stop index recomputed for every
    group here (threads over disjoint blocks of groups; the result's digest must equal the
    stored whole-tensor digest), then code agreement >= 99.99 % and the packed bytes
    identical to the oracle's packing of the GPU codes;
  * zeros and steps: within 1e-5 relative (max(|ref|, 1)) for every group;
  * dequantisation: bit-exact on the oracle's own packed codes and fp16 metadata;
  * fused product (8192 x 8192 weight): batch 1 and 8 on every output, batch 256 on sampled
    output rows, within 2e-3 of max(|y_ref|, rms(y_ref)).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import (CODE_AGREEMENT, GEMV_TOL, assert_zero_close, golden_for, gpu_quantize, say, sha,
                              torch_dev)

pytestmark = pytest.mark.gpu

THREADS = int(os.environ.get("HQQ_TEST_THREADS", "16"))

JOBS = [(w, ti, qi) for w, spec in synth.WORKLOADS.items()
        for ti in range(len(spec["tensors"])) for qi in range(len(spec["quant"]))]


def job_id(j):
    w, ti, qi = j
    t = synth.WORKLOADS[w]["tensors"][ti]
    q = synth.WORKLOADS[w]["quant"][qi]
    return "%s-%s-b%d" % (w, t.name, q.nbits)


def oracle_full(W, q, kout):
    """Oracle per-group steps for every group with the given stop index: codes in flat order,
    fp64 step and zero, and the stored fp16 metadata (oracle rounding)."""
    o = oracle.get()
    r = oracle.quantize_groups_threaded(W, q.nbits, q.group_size, q.axis, kout, q.p, q.beta0, q.kappa,
                                        threads=THREADS)
    cg = r["codes"]
    codes = cg.reshape(-1) if q.axis == 1 else np.ascontiguousarray(cg.T).reshape(-1)
    return {"codes": codes, "delta": r["delta"], "z": r["z"], "delta16": o.to_half_bits(r["delta"]),
            "zero16": o.to_half_bits(r["z"])}


@pytest.mark.parametrize("job", JOBS, ids=job_id)
def test_workload_quantize(job):
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    wname, ti, qi = job
    t = synth.WORKLOADS[wname]["tensors"][ti]
    q = synth.WORKLOADS[wname]["quant"][qi]
    gold = golden_for(wname, t.name, q.nbits, q.group_size, q.axis)
    say("workload", job_id(job), t.rows, t.cols)
    W = t.make()
    assert sha(W.view(np.uint16)) == gold["sha_input_f16"], "input generator drifted"
    o = oracle.get()
    N = t.rows * t.cols

    gq = gpu_quantize(W, q.nbits, q.group_size, q.axis, q.iters, q.p, q.beta0, q.kappa, meta="f64")
    say("  gpu stop", gq["stop"], "oracle stop", gold["kout"])
    assert gq["stop"] == gold["kout"]
    ref_mae = np.array([float.fromhex(h) for h in gold["mae_hex"]])
    rel = np.abs(gq["mae"][:gold["rounds"]] - ref_mae) / ref_mae
    assert rel.max() <= 1e-12, rel.max()
    if gold["rounds"] < q.iters:
        assert np.isnan(gq["mae"][gold["rounds"]:q.iters]).all()

    ref = oracle_full(W, q, gold["kout"])
    assert sha(ref["codes"]) == gold["sha_codes"], "per-group oracle differs from the whole-tensor oracle"
    codes = o.unpack(gq["packed"], N, q.nbits)
    agree = float(np.mean(codes == ref["codes"]))
    say("  code agreement", agree)
    assert agree >= CODE_AGREEMENT
    assert np.array_equal(o.pack(codes, q.nbits), gq["packed"][:o.packed_bytes(N, q.nbits)])
    zerr = assert_zero_close(gq["zero"], ref["z"])
    derr = np.max(np.abs(gq["delta"] - ref["delta"]) / ref["delta"])
    assert derr <= 1e-5
    say("  max zero err %.3g, max step err %.3g" % (zerr, derr))

    # the stored format (fp16 metadata): same codes, metadata = nearest-even of the fp64 values
    g16 = gpu_quantize(W, q.nbits, q.group_size, q.axis, q.iters, q.p, q.beta0, q.kappa, meta="f16")
    assert np.array_equal(g16["packed"], gq["packed"])
    assert np.array_equal(g16["zero"].view(np.uint16), o.to_half_bits(gq["zero"]))
    assert np.array_equal(g16["delta"].view(np.uint16), o.to_half_bits(gq["delta"]))

    # dequantisation of the oracle's own stored format, bit-exact
    packed = o.pack(ref["codes"], q.nbits)
    d16, z16 = ref["delta16"].view(np.float16), ref["zero16"].view(np.float16)
    out = hq.hqq_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(d16).cuda(),
                            torch.from_numpy(z16).cuda(), t.rows, t.cols, q.nbits, q.group_size, q.axis)
    got = out.cpu().numpy().view(np.uint16).reshape(-1)
    del out
    _, w16 = o.dequant(packed, d16, z16, t.rows, t.cols, q.nbits, q.group_size, q.axis)
    mism = int(np.count_nonzero(got != w16.reshape(-1)))
    say("  dequant mismatches", mism)
    assert mism == 0


def test_workload_gemv():
    """8192 x 8192 weight quantized by the oracle; y = x W_hat^T at batch 1, 8 and 256."""
    torch = torch_dev()
    import weight_only_quantization_amd as hq
    spec = synth.WORKLOADS["gemv8192"]
    t, q = spec["tensors"][0], spec["quant"][0]
    gold = golden_for("gemv8192", t.name, q.nbits, q.group_size, q.axis)
    say("gemv workload")
    W = t.make()
    assert sha(W.view(np.uint16)) == gold["sha_input_f16"]
    ref = oracle_full(W, q, gold["kout"])
    assert sha(ref["codes"]) == gold["sha_codes"]
    assert sha(ref["delta16"]) == gold["sha_delta16"] and sha(ref["zero16"]) == gold["sha_zero16"]
    o = oracle.get()
    packed = o.pack(ref["codes"], 4)
    d16, z16 = ref["delta16"].view(np.float16), ref["zero16"].view(np.float16)
    N, K = t.rows, t.cols
    X = synth.activations(256, K, spec["x_seed"])
    pk_d, d_d, z_d = (torch.from_numpy(a).cuda() for a in (packed, d16, z16))
    rsel = np.sort(np.random.default_rng(0).choice(N, 256, replace=False))
    for B in spec["batches"]:
        say("  batch", B)
        x = X[:B]
        for out_dtype in (torch.float32, torch.float16):
            y = hq.hqq_gemv_w4a16(pk_d, d_d, z_d, N, K, q.group_size, torch.from_numpy(x).cuda(),
                                  out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
            sel = None if B <= 8 else rsel
            yr = o.gemv(packed, d16, z16, N, K, q.group_size, x.astype(np.float64), rows_sel=sel)
            yg = y if sel is None else y[:, sel]
            scale = np.maximum(np.abs(yr), np.sqrt(np.mean(yr ** 2)))
            err = float(np.max(np.abs(yg - yr) / scale))
            say("    %s max rel err %.3g" % (out_dtype, err))
            assert err <= GEMV_TOL
            if B > 8:  # the split-K GEMM entry point on the same operands
                y = hq.hqq_gemm_w4a16(pk_d, d_d, z_d, N, K, q.group_size, torch.from_numpy(x).cuda(),
                                      out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
                err = float(np.max(np.abs(y[:, sel] - yr) / scale))
                say("    split GEMM %s max rel err %.3g" % (out_dtype, err))
                assert err <= GEMV_TOL
                # input gradient dX = dY W_hat with dY = the same activations (N = K here)
                dx = hq.hqq_gemm_w4a16_dx(pk_d, d_d, z_d, N, K, q.group_size, torch.from_numpy(x).cuda(),
                                          out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
                dxr = o.gemv_t(packed, d16, z16, N, K, 4, q.group_size, 1, x.astype(np.float64), cols_sel=sel)
                sc = np.maximum(np.abs(dxr), np.sqrt(np.mean(dxr ** 2)))
                err = float(np.max(np.abs(dx[:, sel] - dxr) / sc))
                say("    input gradient %s max rel err %.3g" % (out_dtype, err))
                assert err <= GEMV_TOL
