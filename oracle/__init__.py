"""ctypes wrapper of the HQQ fp64 oracle (``hqq_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the product path never does.  It shares no code with
the HIP library.  See ``hqq_oracle.h`` for the page sections each function
follows.

Every function takes and returns numpy arrays.  fp16 inputs are widened to
fp64 with numpy's exact conversion before they reach the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hqq_oracle.c")
_HDR = os.path.join(_HERE, "hqq_oracle.h")
_LIB = os.path.join(_HERE, "libhqq_oracle.so")

# The range at or below which s = 1 (the page names no number; 1e-4 is used here).
TINY_RANGE = 1e-4

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False, plant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc.  `plant` > 0 builds a deliberately wrong variant
    (for the test that checks the pins catch such mistakes) into a temporary file."""
    if plant:
        out = out or os.path.join(tempfile.mkdtemp(prefix="hqq_oracle_plant"), "lib.so")
        subprocess.check_call(["gcc", *CFLAGS, "-DHQQ_ORACLE_PLANT=%d" % plant, "-o", out, _SRC, "-lm"])
        return out
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _declare(lib):
    i64, i32, dbl, p = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    sig = {
        "hqq_oracle_half_to_double": (dbl, [ctypes.c_uint16]),
        "hqq_oracle_double_to_half": (ctypes.c_uint16, [dbl]),
        "hqq_oracle_doubles_to_halves": (None, [p, i64, p]),
        "hqq_oracle_group_elem": (i64, [i64, i64, i32, i32, i64, i32]),
        "hqq_oracle_sum": (dbl, [p, i64]),
        "hqq_oracle_init_group": (None, [p, i32, i32, dbl, p, p, p]),
        "hqq_oracle_shrink": (dbl, [dbl, dbl, dbl]),
        "hqq_oracle_round_group": (None, [p, i32, i32, dbl, dbl, dbl, dbl, dbl, p, p, p, p]),
        "hqq_oracle_stop_check": (i32, [i32, dbl, dbl]),
        "hqq_oracle_stop_iter": (i32, [p, i32, i32, p]),
        "hqq_oracle_stop_iter_rule": (i32, [p, i32, i32, i32, p]),
        "hqq_oracle_quantize": (i32, [p, i64, i64, i32, i32, i32, i32, dbl, dbl, dbl, dbl, p, p, p, p, p, p, p]),
        "hqq_oracle_quantize_rule": (i32, [p, i64, i64, i32, i32, i32, i32, dbl, dbl, dbl, dbl, i32, p, p, p, p, p,
                                           p, p]),
        "hqq_oracle_quantize_groups": (i32, [p, i64, i32, i32, i32, dbl, dbl, dbl, dbl, p, p, p, p, p, p]),
        "hqq_oracle_quantize_v2": (i32, [p, i64, i64, i32, i32, i32, i32, dbl, dbl, dbl, dbl, p, i32, p, p, p, p,
                                         p]),
        "hqq_oracle_packed_bytes": (i64, [i64, i32]),
        "hqq_oracle_pack": (i32, [p, i64, i32, p]),
        "hqq_oracle_unpack": (i32, [p, i64, i32, p]),
        "hqq_oracle_dequant": (i32, [p, p, p, i64, i64, i32, i32, i32, p, p]),
        "hqq_oracle_gemv": (i32, [p, p, p, i64, i64, i32, p, i64, p, i64, p]),
        "hqq_oracle_gemv_fmt": (i32, [p, p, p, i64, i64, i32, i32, i32, p, i64, p, i64, p]),
        "hqq_oracle_gemv_t": (i32, [p, p, p, i64, i64, i32, i32, i32, p, i64, p, i64, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


class Oracle:
    """One loaded build of the oracle (the normal one, or a planted-mistake variant)."""

    def __init__(self, path: str):
        self.lib = _declare(ctypes.CDLL(path))

    # ---------------------------------------------------------------- scalars
    def half_to_double(self, h: int) -> float:
        return self.lib.hqq_oracle_half_to_double(h)

    def double_to_half(self, x: float) -> int:
        return self.lib.hqq_oracle_double_to_half(x)

    def to_half_bits(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.hqq_oracle_doubles_to_halves(x.ctypes.data, x.size, out.ctypes.data)
        return out

    def sum(self, v) -> float:
        v = np.ascontiguousarray(v, dtype=np.float64)
        return self.lib.hqq_oracle_sum(v.ctypes.data, v.size)

    def group_elem(self, rows, cols, g, axis, j, i) -> int:
        return self.lib.hqq_oracle_group_elem(rows, cols, g, axis, j, i)

    def shrink(self, r: float, beta: float, p: float) -> float:
        return self.lib.hqq_oracle_shrink(r, beta, p)

    def init_group(self, w, nbits: int, tiny: float = TINY_RANGE):
        w = np.ascontiguousarray(w, dtype=np.float64)
        s, d, z = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        self.lib.hqq_oracle_init_group(w.ctypes.data, w.size, nbits, tiny, ctypes.byref(s), ctypes.byref(d),
                                       ctypes.byref(z))
        return s.value, d.value, z.value

    def round_group(self, w, nbits, s, delta, z, beta, p):
        """One proximal round of one group: returns (err_sum, z_next, q, e)."""
        w = np.ascontiguousarray(w, dtype=np.float64)
        q = np.empty_like(w)
        e = np.empty_like(w)
        err, zn = ctypes.c_double(), ctypes.c_double()
        self.lib.hqq_oracle_round_group(w.ctypes.data, w.size, nbits, s, delta, z, beta, p, ctypes.byref(err),
                                        ctypes.byref(zn), q.ctypes.data, e.ctypes.data)
        return err.value, zn.value, q, e

    def stop_iter(self, mae, iters: int, rule: int = 0):
        """(index of the kept zero, rounds evaluated) for a MAE sequence; rule as
        hqq_oracle_stop_iter_rule (0: the page's rollback)."""
        mae = np.ascontiguousarray(mae, dtype=np.float64)
        r = ctypes.c_int()
        if rule == 0:
            k = self.lib.hqq_oracle_stop_iter(mae.ctypes.data, mae.size, iters, ctypes.byref(r))
        else:
            k = self.lib.hqq_oracle_stop_iter_rule(mae.ctypes.data, mae.size, iters, rule, ctypes.byref(r))
        return k, r.value

    # ---------------------------------------------------------------- quantizer
    def quantize(self, W, nbits=4, group_size=64, axis=1, iters=20, p=0.7, beta0=10.0, kappa=1.01,
                 tiny=TINY_RANGE, stop_rule: int = 0) -> dict:
        """Whole-tensor HQQ.  W: 2-D array (fp16 or fp64 values).  Returns codes [rows, cols]
        (uint8), s / delta / z per group (fp64), the MAE of each evaluated round, the number
        of rounds evaluated and the index of the kept zero, plus the stored fp16 metadata."""
        rows, cols = W.shape
        W64 = np.ascontiguousarray(W, dtype=np.float64)
        N = rows * cols
        G = N // group_size
        codes = np.empty((rows, cols), dtype=np.uint8)
        s = np.empty(G)
        d = np.empty(G)
        z = np.empty(G)
        mae = np.full(max(iters, 1), np.nan)
        rounds, kout = ctypes.c_int(), ctypes.c_int()
        if stop_rule == 0:
            rc = self.lib.hqq_oracle_quantize(W64.ctypes.data, rows, cols, nbits, group_size, axis, iters, p, beta0,
                                              kappa, tiny, codes.ctypes.data, s.ctypes.data, d.ctypes.data,
                                              z.ctypes.data, mae.ctypes.data, ctypes.byref(rounds), ctypes.byref(kout))
        else:
            rc = self.lib.hqq_oracle_quantize_rule(W64.ctypes.data, rows, cols, nbits, group_size, axis, iters, p,
                                                   beta0, kappa, tiny, stop_rule, codes.ctypes.data, s.ctypes.data,
                                                   d.ctypes.data, z.ctypes.data, mae.ctypes.data,
                                                   ctypes.byref(rounds), ctypes.byref(kout))
        if rc != 0:
            raise ValueError("oracle quantize rejected the arguments (rc=%d)" % rc)
        return {"codes": codes, "s": s, "delta": d, "z": z, "mae": mae[:rounds.value].copy(),
                "rounds": rounds.value, "kout": kout.value,
                "delta16": self.to_half_bits(d), "zero16": self.to_half_bits(z)}

    def quantize_v2(self, W, grid, nbits=4, group_size=64, iters=20, p=0.7, beta0=10.0, kappa=1.01,
                    tiny=TINY_RANGE, axis=1) -> dict:
        """Scale search per group over multipliers `grid` of the min-max scale; the reading
        is in hqq_oracle.c (parity unpinned as to the reference project).  Returns codes, s /
        delta / z per group, the chosen multiplier's index per group and the fp16 metadata."""
        rows, cols = W.shape
        W64 = np.ascontiguousarray(W, dtype=np.float64)
        G = rows * cols // group_size
        gr = np.ascontiguousarray(grid, dtype=np.float64)
        codes = np.empty((rows, cols), dtype=np.uint8)
        s, d, z = np.empty(G), np.empty(G), np.empty(G)
        choice = np.empty(G, dtype=np.uint8)
        rc = self.lib.hqq_oracle_quantize_v2(W64.ctypes.data, rows, cols, nbits, group_size, axis, iters, p, beta0,
                                             kappa, tiny, gr.ctypes.data, gr.size, codes.ctypes.data, s.ctypes.data,
                                             d.ctypes.data, z.ctypes.data, choice.ctypes.data)
        if rc != 0:
            raise ValueError("oracle quantize_v2 rejected the arguments (rc=%d)" % rc)
        return {"codes": codes, "s": s, "delta": d, "z": z, "choice": choice,
                "delta16": self.to_half_bits(d), "zero16": self.to_half_bits(z)}

    def quantize_groups(self, Wg, nbits, kout, p=0.7, beta0=10.0, kappa=1.01, tiny=TINY_RANGE,
                        trajectories: bool = False) -> dict:
        """Per-group steps for Wg [n, g] with a fixed number of rounds `kout`."""
        Wg = np.ascontiguousarray(Wg, dtype=np.float64)
        n, g = Wg.shape
        codes = np.empty((n, g), dtype=np.uint8)
        s, d, z = np.empty(n), np.empty(n), np.empty(n)
        zt = np.empty((n, kout + 1)) if trajectories else None
        et = np.empty((n, max(kout, 1))) if trajectories else None
        rc = self.lib.hqq_oracle_quantize_groups(Wg.ctypes.data, n, g, nbits, kout, p, beta0, kappa, tiny,
                                                 codes.ctypes.data, s.ctypes.data, d.ctypes.data, z.ctypes.data,
                                                 zt.ctypes.data if trajectories else None,
                                                 et.ctypes.data if trajectories else None)
        if rc != 0:
            raise ValueError("oracle quantize_groups rejected the arguments (rc=%d)" % rc)
        out = {"codes": codes, "s": s, "delta": d, "z": z}
        if trajectories:
            out["z_traj"] = zt
            out["err_traj"] = et[:, :kout]
        return out

    # ---------------------------------------------------------------- storage
    def packed_bytes(self, N: int, nbits: int) -> int:
        return self.lib.hqq_oracle_packed_bytes(N, nbits)

    def pack(self, codes, nbits: int) -> np.ndarray:
        c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
        out = np.empty(self.packed_bytes(c.size, nbits), dtype=np.uint8)
        if self.lib.hqq_oracle_pack(c.ctypes.data, c.size, nbits, out.ctypes.data) != 0:
            raise ValueError("bad nbits")
        return out

    def unpack(self, packed, N: int, nbits: int) -> np.ndarray:
        pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        out = np.empty(N, dtype=np.uint8)
        if self.lib.hqq_oracle_unpack(pk.ctypes.data, N, nbits, out.ctypes.data) != 0:
            raise ValueError("bad nbits")
        return out

    def dequant(self, packed, delta, zero, rows, cols, nbits, group_size, axis):
        """Returns (W_hat fp64 [rows, cols], W_hat fp16 bits [rows, cols]).  delta / zero are the
        stored metadata (any float dtype; widened exactly)."""
        pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        dl = np.ascontiguousarray(delta, dtype=np.float64).reshape(-1)
        zr = np.ascontiguousarray(zero, dtype=np.float64).reshape(-1)
        o64 = np.empty((rows, cols), dtype=np.float64)
        o16 = np.empty((rows, cols), dtype=np.uint16)
        rc = self.lib.hqq_oracle_dequant(pk.ctypes.data, dl.ctypes.data, zr.ctypes.data, rows, cols, nbits,
                                         group_size, axis, o64.ctypes.data, o16.ctypes.data)
        if rc != 0:
            raise ValueError("oracle dequant rejected the arguments (rc=%d)" % rc)
        return o64, o16

    def gemv(self, packed, delta, zero, N, K, group_size, x, rows_sel=None) -> np.ndarray:
        """y = x @ W_hat^T in fp64 (4-bit, axis=1).  x: [batch, K].  Returns [batch, n_sel]."""
        pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        dl = np.ascontiguousarray(delta, dtype=np.float64).reshape(-1)
        zr = np.ascontiguousarray(zero, dtype=np.float64).reshape(-1)
        x = np.ascontiguousarray(x, dtype=np.float64)
        B = x.shape[0]
        if rows_sel is None:
            sel, nsel = None, N
        else:
            sel = np.ascontiguousarray(rows_sel, dtype=np.int64)
            nsel = sel.size
        y = np.empty((B, nsel), dtype=np.float64)
        rc = self.lib.hqq_oracle_gemv(pk.ctypes.data, dl.ctypes.data, zr.ctypes.data, N, K, group_size,
                                      x.ctypes.data, B, None if sel is None else sel.ctypes.data, nsel,
                                      y.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gemv rejected the arguments (rc=%d)" % rc)
        return y

    def gemv_fmt(self, packed, delta, zero, N, K, nbits, group_size, axis, x, rows_sel=None) -> np.ndarray:
        """y = x @ W_hat^T in fp64 for any stored format (2/3/4-bit, axis 0 or 1)."""
        pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        dl = np.ascontiguousarray(delta, dtype=np.float64).reshape(-1)
        zr = np.ascontiguousarray(zero, dtype=np.float64).reshape(-1)
        x = np.ascontiguousarray(x, dtype=np.float64)
        B = x.shape[0]
        if rows_sel is None:
            sel, nsel = None, N
        else:
            sel = np.ascontiguousarray(rows_sel, dtype=np.int64)
            nsel = sel.size
        y = np.empty((B, nsel), dtype=np.float64)
        rc = self.lib.hqq_oracle_gemv_fmt(pk.ctypes.data, dl.ctypes.data, zr.ctypes.data, N, K, nbits, group_size,
                                          axis, x.ctypes.data, B, None if sel is None else sel.ctypes.data, nsel,
                                          y.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gemv_fmt rejected the arguments (rc=%d)" % rc)
        return y

    def gemv_t(self, packed, delta, zero, N, K, nbits, group_size, axis, dy, cols_sel=None) -> np.ndarray:
        """dX = dY @ W_hat in fp64 (the input gradient of the product).  dy: [batch, N].
        Returns [batch, n_sel] for the columns cols_sel (all K by default)."""
        pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        dl = np.ascontiguousarray(delta, dtype=np.float64).reshape(-1)
        zr = np.ascontiguousarray(zero, dtype=np.float64).reshape(-1)
        dy = np.ascontiguousarray(dy, dtype=np.float64)
        B = dy.shape[0]
        if cols_sel is None:
            sel, nsel = None, K
        else:
            sel = np.ascontiguousarray(cols_sel, dtype=np.int64)
            nsel = sel.size
        dx = np.empty((B, nsel), dtype=np.float64)
        rc = self.lib.hqq_oracle_gemv_t(pk.ctypes.data, dl.ctypes.data, zr.ctypes.data, N, K, nbits, group_size, axis,
                                        dy.ctypes.data, B, None if sel is None else sel.ctypes.data, nsel,
                                        dx.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gemv_t rejected the arguments (rc=%d)" % rc)
        return dx


_default: Oracle | None = None


def get() -> Oracle:
    """The normal oracle build (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def group_view(W: np.ndarray, group_size: int, axis: int) -> np.ndarray:
    """[G, g] fp64 copy of the groups, in-group order ("axis" section: reshape([-1, g]) for
    axis=1; reshape([g, -1]) with statistics along axis 0, i.e. columns, for axis=0)."""
    if axis == 1:
        return np.ascontiguousarray(W.reshape(-1, group_size), dtype=np.float64)
    return np.ascontiguousarray(W.reshape(group_size, -1).T, dtype=np.float64)


def quantize_groups_threaded(W: np.ndarray, nbits, group_size, axis, kout, p=0.7, beta0=10.0, kappa=1.01,
                             tiny=TINY_RANGE, threads: int = 16, group_ids=None) -> dict:
    """The oracle's per-group steps over all groups (or `group_ids`) of W with a known number
    of rounds, split over threads (each call is the unchanged single-threaded oracle on a
    disjoint block of groups).  Returns codes [n, g] (in-group order), s, delta, z."""
    o = get()
    Wg = group_view(W, group_size, axis)
    if group_ids is not None:
        Wg = np.ascontiguousarray(Wg[np.asarray(group_ids, dtype=np.int64)])
    n = Wg.shape[0]
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    parts = [(bounds[t], bounds[t + 1]) for t in range(threads) if bounds[t + 1] > bounds[t]]

    def run(b):
        lo, hi = b
        return o.quantize_groups(Wg[lo:hi], nbits, kout, p, beta0, kappa, tiny)

    with ThreadPoolExecutor(max_workers=len(parts)) as ex:
        res = list(ex.map(run, parts))
    return {k: np.concatenate([r[k] for r in res]) for k in ("codes", "s", "delta", "z")}
