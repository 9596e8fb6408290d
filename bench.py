"""Benchmark of the HQQ hot path on one MI355X.

One step = one pass of the whole path over the Llama-7B-shaped layer set (q/k/v/o 4096x4096 and
three 11008x4096 fp16 weights, N(0, 0.02) with 0.1 % +/-10 sigma outliers):
  * hqq_quantize of every layer (4-bit, group 64, axis 1, up to 20 rounds, p 0.7, beta 10 x1.01):
    min-max start, proximal rounds with the whole-tensor early stop, final codes, packing, fp16
    step and zero;
  * hqq_dequantize of every layer back to fp16 (the round trip);
  * the fused product on an 8192x8192 4-bit g64 weight: hqq_gemv_w4a16 at batch 1 and 8 (GEMV),
    hqq_gemm_w4a16 (split-K MFMA GEMM, workspace preallocated) at batch 256.
Beside the step (in "legs", not in `value`): the input gradient dX = dY W_hat on the 8192x8192
weight at batch 256 (hqq_gemm_w4a16_dx), the same layer shapes on Laplace weights at 3-bit
g64 and 2-bit g16, the 28672x8192 weight with axis-0 groups of 128, and the fused products over
the 3-bit, 2-bit and axis-0 formats (with the 3-/2-bit input gradients, hqq_gemm_dx).
The seven layers are independent tensors: their quantize calls are spread over two streams (joined
before the dequantisation).  Inputs are resident in HBM before the timed region; the
product and dequant operands rotate over enough copies (> 1 GB) that the 256 MB last-level cache
cannot hold them.

Prints one JSON line.  `value` is the step's throughput in quantized weights per second
(all legs inside the step time); the per-leg rates and the roofline of the dominant kernel
(the quantizer) are reported beside it, with the single-threaded fp64 oracle timed on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HQQ quantize Gweights/s + dequant-GEMV GB/s (4-bit g64), % of roofline"
PEAK_HBM = 8.0e12            # B/s
PEAK_FP16_MFMA = 2.5e15      # FLOP/s dense
# fp64 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13 lane-operations/s
# (one fp64 add/mul/min/max/round per lane per clock; 78.6 TFLOP/s counts an FMA as two)
PEAK_FP64_ALU = 256 * 4 * 16 * 2.4e9
# algorithmic operations per weight: c per evaluated round + a fixed part.  c = 6 is the
# minimum a round needs when the shrink is exactly zero (the case on these inputs):
# t = W*s + z, round, clip, t - q, accumulate |.|, accumulate q - W*s; fixed = min, max,
# W*s, final t, round, two clip compares, pack (8).
OPS_PER_ROUND = 6
OPS_FIXED = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_traffic.json")
# The layers are independent tensors: their hqq_quantize calls go to this many streams (default
# priority), so one layer's solve fills the GPU while another's stop decision and fix-up (small,
# latency-bound launches) run.  Measured on the 7-layer set (quantize phase / whole step,
# Gweights/s, two runs each): 1 stream 215-216 / 181-182, 2 streams 222-226 / 184-187,
# 3 streams 227 / 184-185, 4 streams 228-229 / 185-186.
QSTREAMS = 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


QUANT_SOURCES = ("hqq_quant.hip", "hqq_internal.h")  # the quantizer kernels and their arguments


def source_digest() -> str:
    """Digest of the quantizer's kernel sources: stored counter readings apply only to them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_quantization_amd", "csrc")
    for f in QUANT_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


GEMV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
GEMV_SOURCES = ("hqq_gemv.hip", "hqq_gemv_common.h", "hqq_internal.h")


def gemv_traffic():
    """HBM bytes per call of the batch-1 GEMV from the committed counter runs, if they were taken
    on the current kernel sources (else null)."""
    if not os.path.exists(GEMV_TRAFFIC_FILE):
        return None
    with open(GEMV_TRAFFIC_FILE) as f:
        tr = json.load(f)
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_quantization_amd", "csrc")
    for fn in GEMV_SOURCES:
        with open(os.path.join(csrc, fn), "rb") as fh:
            h.update(fn.encode() + fh.read())
    k = tr.get("kernels", {}).get("gemv_b1")
    if not k or k.get("source_sha") != h.hexdigest():
        return None
    return k.get("bytes_per_call")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer_tensor, q):
    """The fp64 oracle as it stands, single-threaded on the host (pinned to one core for the
    call), on one 4096x4096 layer."""
    import numpy as np

    import oracle
    o = oracle.get()
    W = layer_tensor.make().astype(np.float64)
    allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if allowed:
        os.sched_setaffinity(0, {min(allowed)})
    try:
        t0 = time.perf_counter()
        r = o.quantize(W, nbits=q.nbits, group_size=q.group_size, axis=q.axis, iters=q.iters, p=q.p, beta0=q.beta0,
                       kappa=q.kappa)
        dt = time.perf_counter() - t0
    finally:
        if allowed:
            os.sched_setaffinity(0, allowed)
    return {"value": W.size / dt / 1e9, "unit": "Gweights/s", "cores": 1, "kind": "oracle",
            "sample": "oracle quantize of one %dx%d layer (%s), 4-bit g64 axis=1, %d rounds evaluated, %.1f s"
                      % (layer_tensor.rows, layer_tensor.cols, layer_tensor.name, r["rounds"], dt),
            "cpu_model": _cpu_model(), "host_cores": os.cpu_count()}


def sleep_rate(stream):
    """Clock rate of torch's spin kernel in cycles per millisecond (measured)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record(stream)
    torch.cuda._sleep(2_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    return 2_000_000 / max(e0.elapsed_time(e1), 1e-3)


SCALE_GRID = (0.85, 0.925, 1.0, 1.05, 1.1)


def scale_search_leg(timed, dev, fan, assign):
    """The second solver (hqq_quantize_v2) on the Llama-7B layer set, 4-bit g64, 20 rounds, over
    five multipliers of the min-max scale: its rate and, next to the default solver's, the mean
    |W - W_hat| it reaches (both dequantised by the library, averaged on the device)."""
    import torch

    import synth
    import weight_only_quantization_amd as hq

    spec = synth.WORKLOADS["llama7b_layers"]
    qp = spec["quant"][0]
    tensors = spec["tensors"]
    Ws = [torch.from_numpy(t.make()).to(dev) for t in tensors]
    outs = [hq.hqq_quantize_v2(W, SCALE_GRID, nbits=qp.nbits, group_size=qp.group_size, iters=qp.iters, p=qp.p,
                               beta0=qp.beta0, kappa=qp.kappa) for W in Ws]

    where = assign([t.rows * t.cols for t in tensors])

    def vall(r):  # the layers spread over the streams, as in the step
        fan([lambda W=W, q=q, ch=ch: hq.hqq_quantize_v2(
            W, SCALE_GRID, nbits=qp.nbits, group_size=qp.group_size, iters=qp.iters, p=qp.p, beta0=qp.beta0,
            kappa=qp.kappa, out=(q.packed, q.delta, q.zero, ch)) for W, (q, ch) in zip(Ws, outs)], where)

    tv = timed(vall, 3)
    n = sum(t.rows * t.cols for t in tensors)

    def mae(pk, d, z, t, W):
        Wh = hq.hqq_dequantize(pk, d, z, t.rows, t.cols, qp.nbits, qp.group_size, 1)
        return float((Wh.double() - W.double()).abs().sum())

    e2 = sum(mae(q.packed, q.delta, q.zero, t, W) for (q, _), t, W in zip(outs, tensors, Ws)) / n
    e1 = 0.0
    for t, W in zip(tensors, Ws):
        q = hq.hqq_quantize(W, nbits=qp.nbits, group_size=qp.group_size, axis=1, iters=qp.iters, p=qp.p,
                            beta0=qp.beta0, kappa=qp.kappa)
        e1 += mae(q.packed, q.delta, q.zero, t, W)
    e1 /= n
    counts = torch.zeros(len(SCALE_GRID), dtype=torch.int64, device=dev)
    for _, ch in outs:
        counts += torch.bincount(ch.long(), minlength=len(SCALE_GRID))
    del Ws, outs
    return {"grid": list(SCALE_GRID), "quantize_s": tv, "quantize_gweights_per_s": n / tv / 1e9,
            "mae_fp16_dequant": e2, "mae_fp16_dequant_default_solver": e1,
            "chosen_per_multiplier": counts.cpu().tolist()}


def config_legs(a, timed, stream, dev, rotated, read_floor, fan, assign):
    """Legs outside the step, one per remaining configuration: the 7B-shaped layer set at 3-bit
    g64 and 2-bit g16 (Laplace weights), the 28672x8192 axis-0 g128 weight, and the fused
    products over the 3-bit, 2-bit and axis-0 formats (batch 1 and 2; batch 256 through hqq_gemm for
    the axis-1 formats; operands rotated over > 1 GB)."""
    import numpy as np
    import torch

    import synth
    import weight_only_quantization_amd as hq

    legs = {}

    def quant_leg(tensors, qp, reps):
        Ws = [torch.from_numpy(t.make()).to(dev) for t in tensors]
        wss = [torch.empty(hq.hqq_quantize_workspace_bytes(t.rows, t.cols, qp.nbits, qp.group_size, qp.axis,
                                                           qp.iters), dtype=torch.uint8, device=dev)
               for t in tensors]
        outs = [hq.hqq_quantize(W, nbits=qp.nbits, group_size=qp.group_size, axis=qp.axis, iters=qp.iters, p=qp.p,
                                beta0=qp.beta0, kappa=qp.kappa, workspace=ws) for W, ws in zip(Ws, wss)]

        where = assign([t.rows * t.cols for t in tensors])

        def qall(r):  # the layers spread over the streams, as in the step
            fan([lambda W=W, ws=ws, q=q: hq.hqq_quantize(
                W, nbits=qp.nbits, group_size=qp.group_size, axis=qp.axis, iters=qp.iters, p=qp.p, beta0=qp.beta0,
                kappa=qp.kappa, workspace=ws, out=(q.packed, q.delta, q.zero, q.stop_iter, q.mae_trace))
                for W, ws, q in zip(Ws, wss, outs)], where)

        tq = timed(qall, reps)
        del wss
        Wh = [torch.empty_like(W) for W in Ws]
        del Ws
        n = sum(t.rows * t.cols for t in tensors)
        wb = 3.2 if qp.nbits == 3 else qp.nbits
        byt = sum(t.rows * t.cols * (wb / 8 + 4 / qp.group_size) for t in tensors)
        dcopies = rotated([(q.packed, q.delta, q.zero) for q in outs], byt)

        def dqall(r):  # one stream: concurrent write streams measured slower (0.49 against 0.64 of peak)
            for t, (pk, d, z), o in zip(tensors, dcopies[r % len(dcopies)], Wh):
                hq.hqq_dequantize(pk, d, z, t.rows, t.cols, qp.nbits, qp.group_size, qp.axis, out=o)

        td = timed(dqall, 2 * len(dcopies))
        leg = {"quantize_s": tq, "quantize_gweights_per_s": n / tq / 1e9,
               "stop_index_per_layer": [int(q.stop_iter.item()) for q in outs],
               "dequant_s": td, "dequant_GB/s": (byt + 2 * n) / td / 1e9,
               "dequant_frac_hbm": (byt + 2 * n) / td / PEAK_HBM, "dequant_copies_rotated": len(dcopies)}
        del Wh, dcopies
        return leg, outs

    def gemv_leg(name, q, N, K, nbits, g, axis, byt_w):
        ncopy = max(4, int(np.ceil(1.1e9 / byt_w)))
        copies = [(q.packed.clone(), q.delta.clone(), q.zero.clone()) for _ in range(ncopy)]
        X = torch.from_numpy(synth.activations(16, K, 402)).to(dev)
        legs["%s_read_floor" % name] = read_floor(copies)
        for b in ((1, 2, 8) if axis == 0 else (1, 2, 8, 16)):
            Y = torch.empty((b, N), dtype=torch.float16, device=dev)

            def gv(r, b=b, Y=Y):
                pk, d, z = copies[r % ncopy]
                hq.hqq_gemv(pk, d, z, N, K, nbits, g, axis, X[:b], out=Y)
            tg = timed(gv, 2 * ncopy)
            byt = byt_w + 2 * b * K + 2 * b * N
            legs["%s_b%d" % (name, b)] = {"us": tg * 1e6, "GB/s": byt / tg / 1e9, "frac_hbm": byt / tg / PEAK_HBM,
                                          "bytes": byt, "shape": [N, K], "copies_rotated": ncopy,
                                          "frac_of_read_floor": legs["%s_read_floor" % name]["us"] / (tg * 1e6)}
        # the batched product over the same format at batch 256 (hqq_gemm)
        for B in (256,):
            X2 = torch.from_numpy(synth.activations(B, K, 403)).to(dev)
            Y = torch.empty((B, N), dtype=torch.float16, device=dev)
            ws = torch.empty(hq.hqq_gemm_workspace_bytes(N, K, B), dtype=torch.uint8, device=dev)

            def gm(r, X2=X2, Y=Y, ws=ws):
                pk, d, z = copies[r % ncopy]
                hq.hqq_gemm(pk, d, z, N, K, nbits, g, axis, X2, out=Y, workspace=ws)
            tg = timed(gm, 2 * ncopy)
            fl = 2.0 * B * N * K
            byt = byt_w + 2 * B * K + 2 * B * N
            legs["%s_b%d" % (name.replace("gemv", "gemm"), B)] = {
                "us": tg * 1e6, "TFLOP/s": fl / tg / 1e12, "frac_mfma_f16": fl / tg / PEAK_FP16_MFMA,
                "GB/s": byt / tg / 1e9, "frac_hbm": byt / tg / PEAK_HBM, "shape": [N, K], "copies_rotated": ncopy}
            del X2, ws
        # the input gradient dX = dY W_hat at batch 256 (hqq_gemm_dx)
        DY = torch.from_numpy(synth.activations(256, N, 404)).to(dev)
        DX = torch.empty((256, K), dtype=torch.float16, device=dev)
        ws = torch.empty(hq.hqq_gemm_dx_workspace_bytes(N, K, 256), dtype=torch.uint8, device=dev)

        def gdx(r):
            pk, d, z = copies[r % ncopy]
            hq.hqq_gemm_dx(pk, d, z, N, K, nbits, g, axis, DY, out=DX, workspace=ws)
        tg = timed(gdx, 2 * ncopy)
        fl = 2.0 * 256 * N * K
        legs["%s_b256" % name.replace("gemv", "dx")] = {
            "us": tg * 1e6, "TFLOP/s": fl / tg / 1e12, "frac_mfma_f16": fl / tg / PEAK_FP16_MFMA,
            "shape": [N, K], "copies_rotated": ncopy}
        del DY, DX, ws
        del copies

    log("config legs: 3-bit and 2-bit layer sets")
    lap = synth.WORKLOADS["llama7b_laplace"]
    for qp in lap["quant"]:
        leg, outs = quant_leg(lap["tensors"], qp, 3)
        legs["layers_laplace_%dbit_g%d" % (qp.nbits, qp.group_size)] = leg
        t = lap["tensors"][4]
        if qp.nbits == 2:
            gemv_leg("gemv_2bit_g16", outs[4], t.rows, t.cols, 2, 16, 1, t.rows * t.cols * (2 / 8 + 4 / 16))
        else:
            gemv_leg("gemv_3bit_g%d" % qp.group_size, outs[4], t.rows, t.cols, 3, qp.group_size, 1,
                     4 * ((t.rows * t.cols + 9) // 10) + 4 * t.rows * t.cols / qp.group_size)
        del outs
        torch.cuda.empty_cache()
    log("config legs: scale search over the 4-bit layer set")
    legs["layers_scale_search_4bit_g64"] = scale_search_leg(timed, dev, fan, assign)
    torch.cuda.empty_cache()
    log("config legs: 28672x8192 axis 0")
    m70 = synth.WORKLOADS["mlp70b"]
    qp = m70["quant"][0]
    leg, outs = quant_leg(m70["tensors"], qp, 3)
    legs["mlp70b_axis0_4bit_g128"] = leg
    t = m70["tensors"][0]
    gemv_leg("gemv_axis0_g128", outs[0], t.rows, t.cols, 4, 128, 0, t.rows * t.cols * (4 / 8 + 4 / 128))
    del outs
    torch.cuda.empty_cache()
    return legs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="skip the 3-/2-bit, axis-0 and other-format legs outside the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--qstreams", type=int, default=QSTREAMS,
                    help="streams the layers' hqq_quantize calls are spread over (independent tensors)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="each leg's kernels run a few times without timing loops (for rocprofv3 --pmc runs)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import weight_only_quantization_amd as hq

    assert torch.cuda.is_available(), "no GPU"
    hq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = synth.WORKLOADS["llama7b_layers"]
    qp = spec["quant"][0]
    gspec = synth.WORKLOADS["gemv8192"]
    gq = gspec["quant"][0]

    # ---------------------------------------------------------------- inputs resident in HBM
    log("generating inputs")
    layers = []
    for t in spec["tensors"]:
        W = torch.from_numpy(t.make()).to(dev)
        G = t.rows * t.cols // qp.group_size
        ws = torch.empty(hq.hqq_quantize_workspace_bytes(t.rows, t.cols, qp.nbits, qp.group_size, qp.axis, qp.iters),
                         dtype=torch.uint8, device=dev)
        out = (torch.empty(hq.hqq_packed_bytes(t.rows, t.cols, qp.nbits), dtype=torch.uint8, device=dev),
               torch.empty(G, dtype=torch.float16, device=dev), torch.empty(G, dtype=torch.float16, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev), torch.empty(qp.iters, dtype=torch.float64, device=dev))
        What = torch.empty((t.rows, t.cols), dtype=torch.float16, device=dev)
        layers.append((t, W, ws, out, What))
    n_weights = sum(t.rows * t.cols for t, *_ in layers)

    gt = gspec["tensors"][0]
    GN, GK = gt.rows, gt.cols
    Wg = torch.from_numpy(gt.make()).to(dev)
    q0 = hq.hqq_quantize(Wg, nbits=gq.nbits, group_size=gq.group_size, axis=gq.axis, iters=gq.iters)
    gemv_bytes_w = q0.packed.numel() + 4 * q0.delta.numel()
    ncopy = max(4, int(np.ceil(1.1e9 / gemv_bytes_w)))
    copies = [(q0.packed.clone(), q0.delta.clone(), q0.zero.clone()) for _ in range(ncopy)]
    del Wg
    X = torch.from_numpy(synth.activations(256, GK, gspec["x_seed"])).to(dev)
    Y = {b: torch.empty((b, GN), dtype=torch.float16, device=dev) for b in (1, 8, 256)}
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    gemm_ws = torch.empty(max(hq.hqq_gemm_workspace_bytes(GN, GK, 256), 16), dtype=torch.uint8, device=dev)

    def product(pk, d, z, b):
        """Batch <= 8: the streaming GEMV; larger: the split-K GEMM with its workspace."""
        if b <= 8:
            hq.hqq_gemv_w4a16(pk, d, z, GN, GK, gq.group_size, X[:b], out=Y[b])
        else:
            hq.hqq_gemm_w4a16(pk, d, z, GN, GK, gq.group_size, X[:b], out=Y[b], workspace=gemm_ws)

    # layers to streams: largest first, each to the stream with the least work so far
    nqs = max(1, a.qstreams)
    qstreams = [stream] if nqs == 1 else [torch.cuda.Stream(device=dev) for _ in range(nqs)]

    def assign(sizes):
        load, where = [0] * nqs, [0] * len(sizes)
        for li in sorted(range(len(sizes)), key=lambda k: -sizes[k]):
            where[li] = min(range(nqs), key=lambda k: load[k])
            load[where[li]] += sizes[li]
        return where

    qstream_of = assign([t.rows * t.cols for t, *_ in layers])

    def fan(fns, where):
        """Run fns[i] on stream qstreams[where[i]], forked from and joined back to the launch stream."""
        if nqs == 1:
            for f in fns:
                f()
            return
        fork = torch.cuda.Event()
        fork.record(stream)
        for qs in qstreams:
            qs.wait_event(fork)
        for f, w in zip(fns, where):
            with torch.cuda.stream(qstreams[w]):
                f()
        for qs in qstreams:
            j = torch.cuda.Event()
            j.record(qs)
            stream.wait_event(j)

    def quantize_all(ev=None):
        """The layers' hqq_quantize calls; ev = (start, end) events on the launch stream around them."""
        if ev is not None:
            ev[0].record(stream)
        fan([lambda W=W, ws=ws, out=out: hq.hqq_quantize(
            W, nbits=qp.nbits, group_size=qp.group_size, axis=qp.axis, iters=qp.iters, p=qp.p, beta0=qp.beta0,
            kappa=qp.kappa, workspace=ws, out=out) for t, W, ws, out, What in layers], qstream_of)
        if ev is not None:
            ev[1].record(stream)

    def dequantize_all():
        """The layers' hqq_dequantize calls on the launch stream (write-heavy kernels on several streams at
        once measured slower than one after another)."""
        for t, W, ws, out, What in layers:
            hq.hqq_dequantize(out[0], out[1], out[2], t.rows, t.cols, qp.nbits, qp.group_size, qp.axis, out=What)

    def step(i, ev=None):
        quantize_all(ev)
        dequantize_all()
        for j, b in enumerate((1, 8, 256)):
            pk, d, z = copies[(3 * i + j) % ncopy]
            product(pk, d, z, b)

    # ---------------------------------------------------------------- warmup + timed steps
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(a.steps):
        step(i, ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(end) / a.steps
    qtimes = np.array([s.elapsed_time(e) for s, e in ev])  # ms per step of the layers' hqq_quantize calls

    stops = [int(out[3].item()) for _, _, _, out, _ in layers]
    rounds = [min(s + 2, qp.iters) if s < qp.iters else qp.iters for s in stops]

    # ---------------------------------------------------------------- per-leg timing loops
    cycles_per_ms = sleep_rate(stream)

    def timed(fn, reps):
        """Mean GPU time of one call over `reps` back-to-back calls on the launch stream.  A spin
        kernel holds the stream while the host enqueues the calls (so that host launch overhead
        never leaves the GPU idle between them); one event pair brackets the calls.  In a counter
        pass the calls run a few times, untimed (rocprofv3 serialises and samples each dispatch)."""
        if a.counter_pass:
            for r in range(min(reps, 3)):
                fn(r)
            torch.cuda.synchronize()
            return float("nan")
        fn(0)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for r in range(reps):
            fn(r)
        host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        torch.cuda._sleep(int(cycles_per_ms * (2.0 * host_ms + 1.0)))
        t0_ev, t1_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0_ev.record(stream)
        for r in range(reps):
            fn(r)
        t1_ev.record(stream)
        torch.cuda.synchronize()
        return t0_ev.elapsed_time(t1_ev) * 1e-3 / reps  # s per call

    def rotated(bufs, nbytes):
        """Copies of `bufs` (a list of tensors or of tuples of tensors) totalling >= 1.1 GB of
        operands (`nbytes` per set), so that a timing loop over them reads HBM, not the 256 MB
        last-level cache."""
        n = max(4, int(np.ceil(1.1e9 / nbytes)))
        cl = lambda b: tuple(t.clone() for t in b) if isinstance(b, tuple) else b.clone()
        return [[cl(b) for b in bufs] for _ in range(n)]

    probe_sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def read_floor(copies):
        """The HBM floor of a kernel that must stream these operands once: the probe's streaming
        read of one copy's buffers in one launch, timed back to back over the rotated copies
        (best of 4 and 8 loads in flight per thread)."""
        nb = sum((t.numel() * t.element_size()) & ~15 for t in copies[0])  # whole 16-byte blocks
        best = None
        for u in (4, 8):
            tr = timed(lambda r, u=u: hq.probe_read(copies[r % len(copies)], probe_sink, unroll=u), 2 * len(copies))
            if best is None or tr < best[0]:
                best = (tr, u)
        return {"us": best[0] * 1e6, "GB/s": nb / best[0] / 1e9, "frac_hbm": nb / best[0] / PEAK_HBM, "bytes": nb,
                "loads_in_flight": best[1], "copies_rotated": len(copies)}

    legs = {}
    dq_bytes = sum(t.rows * t.cols * (qp.nbits / 8 + 2) + 4 * t.rows * t.cols / qp.group_size
                   for t, *_ in layers)
    dq_in = sum(t.rows * t.cols * qp.nbits / 8 + 4 * t.rows * t.cols / qp.group_size for t, *_ in layers)
    dq_copies = rotated([(out[0], out[1], out[2]) for _, _, _, out, _ in layers], dq_in)

    def dq_all(r):
        for (t, W, ws, out, What), (pk, d, z) in zip(layers, dq_copies[r % len(dq_copies)]):
            hq.hqq_dequantize(pk, d, z, t.rows, t.cols, qp.nbits, qp.group_size, qp.axis, out=What)

    t_dq = timed(dq_all, 2 * len(dq_copies))
    legs["dequant"] = {"s_per_layer_set": t_dq, "GB/s": dq_bytes / t_dq / 1e9,
                       "frac_hbm": dq_bytes / t_dq / PEAK_HBM, "bytes": dq_bytes, "copies_rotated": len(dq_copies)}
    del dq_copies
    legs["gemv_read_floor"] = read_floor(copies)
    for b in (1, 8, 256):
        def gv(r, b=b):
            pk, d, z = copies[r % ncopy]
            product(pk, d, z, b)
        tg = timed(gv, 2 * ncopy)
        byt = GN * GK / 2 + 4 * GN * GK / gq.group_size + 2 * b * GK + 2 * b * GN
        flops = 2.0 * b * GN * GK
        legs["gemv_b%d" % b] = {"us": tg * 1e6, "GB/s": byt / tg / 1e9, "frac_hbm": byt / tg / PEAK_HBM,
                                "TFLOP/s": flops / tg / 1e12, "frac_mfma_f16": flops / tg / PEAK_FP16_MFMA,
                                "bytes": byt, "frac_of_read_floor": legs["gemv_read_floor"]["us"] / (tg * 1e6)}

    # the input gradient dX = dY W_hat (training through the frozen weight) at batch 256
    dx_ws = torch.empty(max(hq.hqq_gemm_dx_workspace_bytes(GN, GK, 256), 16), dtype=torch.uint8, device=dev)
    DX = torch.empty((256, GK), dtype=torch.float16, device=dev)
    DY = torch.from_numpy(synth.activations(256, GN, gspec["x_seed"] + 1)).to(dev)

    def dxl(r):
        pk, d, z = copies[r % ncopy]
        hq.hqq_gemm_w4a16_dx(pk, d, z, GN, GK, gq.group_size, DY, out=DX, workspace=dx_ws)
    tg = timed(dxl, 2 * ncopy)
    flops = 2.0 * 256 * GN * GK
    legs["dx_b256"] = {"us": tg * 1e6, "TFLOP/s": flops / tg / 1e12, "frac_mfma_f16": flops / tg / PEAK_FP16_MFMA}

    # the layer set's 4096 x 4096 projection at batch 8 and 16: weights of up to 2^24 codes take the
    # register-dequant MFMA kernel at batch 3-16 (32 rotated copies, ~300 MB: past the 256 MB
    # last-level cache, and few enough calls for the spin kernel to cover their enqueue)
    t0l, _, _, out0, _ = layers[0]
    pq_bytes = out0[0].numel() + 4 * out0[1].numel()
    pcop = [(out0[0].clone(), out0[1].clone(), out0[2].clone()) for _ in range(max(4, int(np.ceil(0.3e9 / pq_bytes))))]
    XS = torch.from_numpy(synth.activations(16, t0l.cols, 405)).to(dev)
    legs["gemv_4096x4096_read_floor"] = read_floor(pcop)
    for b in (8, 16):
        Yp = torch.empty((b, t0l.rows), dtype=torch.float16, device=dev)

        def gp(r, b=b, Yp=Yp):
            pk, d, z = pcop[r % len(pcop)]
            hq.hqq_gemv_w4a16(pk, d, z, t0l.rows, t0l.cols, qp.group_size, XS[:b], out=Yp)
        tg = timed(gp, 2 * len(pcop))
        byt = pq_bytes + 2 * b * (t0l.rows + t0l.cols)
        legs["gemv_4096x4096_b%d" % b] = {"us": tg * 1e6, "GB/s": byt / tg / 1e9, "frac_hbm": byt / tg / PEAK_HBM,
                                          "bytes": byt, "copies_rotated": len(pcop),
                                          "frac_of_read_floor": legs["gemv_4096x4096_read_floor"]["us"] / (tg * 1e6)}
    del pcop, XS

    # a streaming device copy on the same box (the probe's 16-byte non-temporal loads and stores,
    # best of 4 and 8 loads in flight): the HBM rate a read + write kernel reaches in practice
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    tc = min(timed(lambda r, u=u: hq.probe_copy(csrc, cdst, unroll=u), 20) for u in (4, 8))
    copy_bps = 2.0 * csrc.numel() / tc
    legs["probe_copy_1GiB"] = {"us": tc * 1e6, "GB/s": copy_bps / 1e9, "frac_hbm": copy_bps / PEAK_HBM}
    del csrc, cdst

    if not a.no_extra_legs:
        legs.update(config_legs(a, timed, stream, dev, rotated, read_floor, fan, assign))
    for leg in legs.values():  # every HBM fraction also against the measured copy rate
        if "frac_hbm" in leg:
            leg["frac_copy"] = leg["frac_hbm"] * PEAK_HBM / copy_bps
        if "dequant_frac_hbm" in leg:
            leg["dequant_frac_copy"] = leg["dequant_frac_hbm"] * PEAK_HBM / copy_bps

    if a.copy_probe:  # one 1 GiB probe copy: the counter calibration of known size
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        hq.probe_copy(src, dst, unroll=4)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- roofline of the quantizer
    ops = sum((OPS_PER_ROUND * r + OPS_FIXED) * t.rows * t.cols for (t, *_), r in zip(layers, rounds))
    q_s_total = float(qtimes.mean()) * 1e-3  # the layer set's quantize phase per step
    achieved = ops / q_s_total
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha") == source_digest():
            traffic = tr.get("bytes_per_layer_set")
    roof = {"bound": "alu", "achieved": achieved / 1e12, "peak": PEAK_FP64_ALU / 1e12, "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP64_ALU, "traffic": traffic,
            "kernel": "hqq_quantize (solve + stop decision + fix-up), 7 layers on %d stream(s)" % nqs,
            "ops_per_weight": "%d per evaluated round + %d" % (OPS_PER_ROUND, OPS_FIXED),
            "rounds_evaluated": rounds, "seconds_per_layer_set": q_s_total}
    g1 = legs["gemv_b1"]
    roof_gemv = {"bound": "hbm", "achieved": g1["GB/s"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                 "frac": g1["frac_hbm"], "traffic": gemv_traffic(),
                 "kernel": "hqq_gemv_w4a16 batch 1 (k_gemv_valu), 8192x8192 4-bit g64, fp16 step and zero",
                 "us": g1["us"], "bytes": g1["bytes"],
                 "read_floor_us": legs["gemv_read_floor"]["us"],
                 "frac_of_read_floor": g1["frac_of_read_floor"]}
    alg_bytes_q = sum(t.rows * t.cols * (2 + qp.nbits / 8) + 4 * t.rows * t.cols / qp.group_size
                      for t, *_ in layers)

    res = {
        "metric": METRIC,
        "value": n_weights / (step_ms * 1e-3) / 1e9,
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded; N(0,0.02) + 0.1% +/-10 sigma outliers; activations N(0,1))",
        "config": {"workload": "llama7b_layers quantize+pack+dequant (4x4096x4096 + 3x11008x4096, 4-bit g64 "
                               "axis=1, 20 rounds) + fused W4A16 8192x8192 at batch 1/8/256",
                   "weights": n_weights, "nbits": qp.nbits, "group_size": qp.group_size, "axis": qp.axis,
                   "iters": qp.iters, "gemv_copies_rotated": ncopy},
        "quantize_gweights_per_s": n_weights / q_s_total / 1e9,
        "quantize_hbm_frac": alg_bytes_q / q_s_total / PEAK_HBM,
        "stop_index_per_layer": stops,
        "legs": legs,
        "roofline": roof,
        "roofline_gemv_b1": roof_gemv,
        "wall_s": wall,
    }
    if not a.no_cpu_baseline:
        log("timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(spec["tensors"][0], qp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
