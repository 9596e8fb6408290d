"""Write tests/golden/oracle_workloads.json: the whole-tensor oracle's results on every
tensor of every workload in ``synth.WORKLOADS``.

It calls only the oracle and the input generator.  Per tensor and quantizer setting it
stores the number of rounds the method evaluates, the index of the kept zero, the MAE of
each evaluated round (exact, as float.hex), and SHA-256 digests of the input bits, the
codes, the packed bytes, the fp64 zeros and the stored fp16 metadata.  The full-size GPU
tests compare the stop decision and the MAE trace with these, and recompute codes and
zeros group by group with the oracle at test time.

Usage: python tests/golden/make_oracle_golden.py [--jobs 8] [--only WORKLOAD ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from multiprocessing import Pool

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_workloads.json")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def one(job):
    wname, ti, qi = job
    spec = synth.WORKLOADS[wname]
    t = spec["tensors"][ti]
    qp = spec["quant"][qi]
    W = t.make()
    o = oracle.get()
    t0 = time.time()
    r = o.quantize(W, nbits=qp.nbits, group_size=qp.group_size, axis=qp.axis, iters=qp.iters, p=qp.p,
                   beta0=qp.beta0, kappa=qp.kappa)
    dt = time.time() - t0
    packed = o.pack(r["codes"], qp.nbits)
    mae = r["mae"]
    gaps = [(mae[k] - mae[k - 1]) / mae[k - 1] for k in range(1, len(mae))]
    rec = {
        "workload": wname, "tensor": t.name, "rows": t.rows, "cols": t.cols,
        "nbits": qp.nbits, "group_size": qp.group_size, "axis": qp.axis, "iters": qp.iters,
        "p": qp.p, "beta0": qp.beta0, "kappa": qp.kappa, "tiny": oracle.TINY_RANGE,
        "rounds": r["rounds"], "kout": r["kout"],
        "mae_hex": [float(v).hex() for v in mae],
        "min_abs_rel_gap": float(np.min(np.abs(gaps))) if gaps else None,
        "last_rel_gap": float(gaps[-1]) if gaps else None,
        "sha_input_f16": sha(W.view(np.uint16)),
        "sha_codes": sha(r["codes"]), "sha_packed": sha(packed),
        "sha_z_f64": sha(r["z"]), "sha_delta_f64": sha(r["delta"]),
        "sha_delta16": sha(r["delta16"]), "sha_zero16": sha(r["zero16"]),
        "oracle_seconds": dt,
    }
    print("%-16s %-10s b%d g%d ax%d  rounds=%d kout=%d  %.1fs" % (wname, t.name, qp.nbits, qp.group_size, qp.axis,
                                                                 r["rounds"], r["kout"], dt), flush=True)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--only", nargs="*")
    a = ap.parse_args()
    oracle.build()
    synth.build()
    jobs = []
    for wname, spec in synth.WORKLOADS.items():
        if a.only and wname not in a.only:
            continue
        for ti in range(len(spec["tensors"])):
            for qi in range(len(spec["quant"])):
                jobs.append((wname, ti, qi))
    # biggest first
    jobs.sort(key=lambda j: -synth.WORKLOADS[j[0]]["tensors"][j[1]].rows * synth.WORKLOADS[j[0]]["tensors"][j[1]].cols)
    old = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            for rec in json.load(f)["records"]:
                old[(rec["workload"], rec["tensor"], rec["nbits"], rec["group_size"], rec["axis"])] = rec
    with Pool(a.jobs) as pool:
        recs = pool.map(one, jobs, chunksize=1)
    for rec in recs:
        old[(rec["workload"], rec["tensor"], rec["nbits"], rec["group_size"], rec["axis"])] = rec
    out = {"generator": "tests/golden/make_oracle_golden.py (oracle + synth only)",
           "records": sorted(old.values(), key=lambda r: (r["workload"], r["tensor"], r["nbits"]))}
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
