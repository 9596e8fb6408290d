"""Pins of the fp64 oracle against facts fixed outside it.

Each pin is a function of one loaded oracle build, raising AssertionError when
the build disagrees with the fact.  ``test_oracle_pins.py`` runs them against
the normal build; ``test_oracle_plants.py`` runs them against builds with a
deliberately wrong step and expects at least one pin to fail for each.

The facts come from the pages (worked example, storage sizes, packing counts),
from mathematics (least squares, monotonicity of alternating minimisation,
the rounding-error bound, soft thresholding at p = 1), from library routines
(numpy's fp16 conversion and reshape, numpy matmul) and from brute force on
tiny inputs.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- fp16 helpers

def pin_half_to_double_exhaustive(o):
    """All 65536 binary16 patterns widen exactly as numpy widens them."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "half->double differs at %s" % bits[~same][:5]


def pin_double_to_half_matches_numpy(o):
    """Round-to-nearest-even to binary16, incl. exact ties and the subnormal range."""
    r = _rng(7)
    x = np.concatenate([
        r.normal(0, 1, 20000), r.normal(0, 1e-5, 20000), r.normal(0, 3e4, 5000),
        np.array([65504.0, 65519.99, 65520.0, 7e4, -65520.0, 0.0, -0.0, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26]),
    ])
    # exact midpoints between neighbouring positive halves (ties), normal and subnormal
    h = np.arange(1, 0x7bff, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2])
    got = o.to_half_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert (got == ref).all(), "double->half differs at %s" % x[got != ref][:5]


# ----------------------------------------------------------------------------- summation

def pin_pairwise_sum(o):
    """Every sum is the balanced pairwise sum in index order (the reading of the unstated
    order): exact on integers, within the pairwise error bound of the exact sum (math.fsum),
    and [1, u, u, u] with u = 2^-53 sums to 1 + 2u (a sequential sum would give 1)."""
    import math
    u = 2.0 ** -53
    assert o.sum([1.0, u, u, u]) == 1.0 + 2 * u
    assert o.sum([]) == 0.0 and o.sum([3.5]) == 3.5
    r = _rng(2)
    for n in (1, 2, 3, 7, 64, 100, 1000, 4097):
        ints = r.integers(-1000, 1000, n).astype(np.float64)
        assert o.sum(ints) == ints.sum()
        v = r.normal(0, 1, n)
        bound = (np.ceil(np.log2(max(n, 2))) + 1) * 2.0 ** -53 * np.abs(v).sum()
        assert abs(o.sum(v) - math.fsum(v)) <= bound


# ----------------------------------------------------------------------------- min-max start

def pin_worked_example(o):
    """[-0.8, 0.7] at 4 bits: s0 = 10, z0 = 8, codes 0 / 8 / 15 (fp64 values as printed)."""
    ex = _load("worked_example.json")
    vals = np.array(ex["values"], dtype=np.float64)
    s, d, z = o.init_group(vals, ex["nbits"])
    assert s == ex["s0"] and z == ex["z0"], (s, z)
    r = o.quantize(vals.reshape(1, -1), nbits=ex["nbits"], group_size=vals.size, axis=1, iters=0)
    assert list(r["codes"].reshape(-1)) == ex["codes"], r["codes"]
    assert r["kout"] == 0 and r["rounds"] == 0


def pin_worked_example_fp16(o):
    """The same example after fp16 storage of W: -0.7998046875 .. 0.7001953125 spans exactly
    1.5, so s0 = 10 exactly and z0 = 7.998046875; the codes are unchanged."""
    ex = _load("worked_example.json")
    vals = np.array(ex["values"], dtype=np.float16).astype(np.float64)
    s, d, z = o.init_group(vals, ex["nbits"])
    assert s == 10.0 and z == 7.998046875, (s, z)
    r = o.quantize(vals.reshape(1, -1), nbits=4, group_size=3, axis=1, iters=0)
    assert list(r["codes"].reshape(-1)) == ex["codes"]


def pin_worked_example_solver(o):
    """Group {-0.8, 0.7, 0 x 62}: q0 - W*s = 8 for every element, so z1 = z0 = 8, round 1
    repeats round 0's MAE, the loop stops at round 1 and keeps z0."""
    w = np.zeros(64)
    w[0], w[1] = -0.8, 0.7
    r = o.quantize(w.reshape(1, 64), nbits=4, group_size=64, axis=1, iters=20)
    assert r["rounds"] == 2 and r["kout"] == 0, (r["rounds"], r["kout"])
    assert r["z"][0] == 8.0 and r["s"][0] == 10.0
    c = r["codes"].reshape(-1)
    assert c[0] == 0 and c[1] == 15 and (c[2:] == 8).all()


def pin_minmax_rtn(o):
    """iters = 0 is asymmetric min-max round-to-nearest: the minimum of every group maps to
    code 0, the maximum to 2^b - 1, and nothing is clipped, so |W - W_hat| <= step/2
    (rounding-error bound of the affine map)."""
    r = _rng(3)
    for nbits, g, axis in [(4, 64, 1), (3, 32, 1), (2, 16, 0), (4, 8, 0)]:
        W = r.normal(0, 0.02, (32, 64)).astype(np.float16).astype(np.float64)
        res = o.quantize(W, nbits=nbits, group_size=g, axis=axis, iters=0)
        qmax = (1 << nbits) - 1
        G = W.size // g
        for j in range(G):
            idx = [o.group_elem(32, 64, g, axis, j, i) for i in range(g)]
            vals = W.reshape(-1)[idx]
            codes = res["codes"].reshape(-1)[idx]
            assert codes[np.argmin(vals)] == 0 and codes[np.argmax(vals)] == qmax
        w64, _ = o.dequant(o.pack(res["codes"], nbits), res["delta"], res["z"], 32, 64, nbits, g, axis)
        dj = np.array([res["delta"][_group_of(i, 32, 64, g, axis)] for i in range(W.size)]).reshape(W.shape)
        assert (np.abs(W - w64) <= dj / 2 * (1 + 1e-9)).all()


def _group_of(idx, rows, cols, g, axis):
    return idx // g if axis == 1 else idx % (rows * cols // g)


def pin_rounding_ties_to_even(o):
    """Range [0, 15] at 4 bits gives s = 1, z0 = 0, so 2.5 lands exactly on a tie; round
    half to even sends it to 2 (and 3.5 to 4)."""
    w = np.array([0.0, 2.5, 3.5, 15.0])
    r = o.quantize(w.reshape(1, 4), nbits=4, group_size=4, axis=1, iters=0)
    assert list(r["codes"].reshape(-1)) == [0, 2, 4, 15], r["codes"]
    _, _, q, _ = o.round_group(w, 4, 1.0, 1.0, 0.0, 10.0, 0.7)
    assert list(q) == [0, 2, 4, 15], q


def pin_degenerate_groups(o):
    """Constant group: s = 1, z = -c, code 0, exact reconstruction.  All-zero group: s = 1,
    z = 0.  Tiny range (<= 1e-4): s = 1.  Small range: s limited to 2e4."""
    for c in (0.375, -1.25, 0.0):
        w = np.full(16, c)
        res = o.quantize(w.reshape(1, 16), nbits=4, group_size=16, axis=1, iters=5)
        assert res["s"][0] == 1.0 and res["z"][0] == -c and (res["codes"] == 0).all()
        w64, _ = o.dequant(o.pack(res["codes"], 4), res["delta"], res["z"], 1, 16, 4, 16, 1)
        assert (w64 == c).all()
    s, d, z = o.init_group(np.array([0.0, 5e-5]), 4)
    assert s == 1.0
    s, d, z = o.init_group(np.array([0.0, 2e-4]), 4)
    assert s == 2.0e4 and d == 5e-5
    s, d, z = o.init_group(np.array([-0.005, 0.005]), 4)
    assert s == 1500.0


# ----------------------------------------------------------------------------- shrink

def pin_shrink_values(o):
    """Values of the reading e = sign(r) max(|r| - |r|^(p-1)/beta, 0) at p=0.7, beta=10,
    zero below the threshold beta^(-1/(2-p)), and plain soft thresholding at p = 1."""
    assert abs(o.shrink(1.0, 10.0, 0.7) - 0.9) < 1e-15
    assert abs(o.shrink(-1.0, 10.0, 0.7) + 0.9) < 1e-15
    assert abs(o.shrink(0.5, 10.0, 0.7) - (0.5 - 0.5 ** -0.3 / 10)) < 1e-15
    assert abs(o.shrink(0.5, 10.0, 0.7) - 0.37688555866550837) < 1e-14
    assert o.shrink(0.1, 10.0, 0.7) == 0.0 and o.shrink(0.0, 10.0, 0.7) == 0.0
    for beta in (10.0, 12.2, 30.0):
        thr = beta ** (-1.0 / 1.3)
        for a in (thr * (1 - 1e-6), thr * 0.5, 1e-9):
            assert o.shrink(a, beta, 0.7) == 0.0 and o.shrink(-a, beta, 0.7) == 0.0
        for a in (thr * (1 + 1e-6), thr * 2, 3.0):
            v = o.shrink(a, beta, 0.7)
            assert 0.0 < v < a
    r = np.linspace(-2, 2, 401)
    soft = np.sign(r) * np.maximum(np.abs(r) - 1 / 10.0, 0)
    got = np.array([o.shrink(x, 10.0, 1.0) for x in r])
    assert np.allclose(got, soft, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- zero update

def _lsq_check(w, q, e, s, z_next, h=1e-4, width=2.0):
    f = lambda z: np.sum((q - z - (w - e) * s) ** 2)  # noqa: E731
    grid = z_next + np.arange(-width, width + h / 2, h)
    vals = np.array([f(z) for z in grid])
    zbest = grid[np.argmin(vals)]
    assert abs(zbest - z_next) <= h * 0.51, (zbest, z_next)
    f0 = f(z_next)
    assert f0 <= f(z_next + 1e-6) and f0 <= f(z_next - 1e-6)


def pin_zero_update_least_squares(o):
    """For the round's own q, e and fixed s, the new zero minimises sum (q - z - (W-e)s)^2
    (brute force over a grid, and the two neighbours), i.e. it is the group mean of the
    per-element suggestions q - (W-e)s.  Checked with the shrink inactive (sigma 0.02)
    and active (sigma 1)."""
    r = _rng(11)
    for sigma in (0.02, 1.0):
        for trial in range(6):
            g = 8
            nbits = 4 if sigma < 0.5 else 2
            w = r.normal(0, sigma, g)
            s, d, z0 = o.init_group(w, nbits)
            z = z0 + r.uniform(-1.5, 1.5)
            err, zn, q, e = o.round_group(w, nbits, s, d, z, 10.0, 0.7)
            if sigma == 1.0 and trial == 0:
                assert np.any(e != 0)
            _lsq_check(w, q, e, s, zn)


def pin_l2_monotone(o):
    """Without the shrink (all residuals below its threshold) each round is one step of
    alternating minimisation of sum (W - (q - z)/s)^2 over z (closed form) and q (nearest
    grid point within the clip range), so that error never increases from round to round."""
    r = _rng(5)
    for nbits in (2, 3, 4):
        for trial in range(10):
            w = r.normal(0, 0.02, 64)
            w[r.integers(0, 64)] = 0.2
            s, d, z = o.init_group(w, nbits)
            prev = np.inf
            beta = 10.0
            for k in range(20):
                err, zn, q, e = o.round_group(w, nbits, s, d, z, beta, 0.7)
                assert (e == 0).all()
                l2 = np.sum((w - (q - z) / s) ** 2)
                assert l2 <= prev * (1 + 1e-12), (nbits, trial, k, l2, prev)
                prev, z, beta = l2, zn, beta * 1.01


def pin_beta_schedule(o):
    """beta grows by the factor kappa each round (beta_k = beta0 kappa^k): with the shrink
    active, round k of the oracle's loop is reproduced by one round at that beta and not by
    one at beta0."""
    r = _rng(17)
    W = r.normal(0, 1.0, (4, 64))
    res = o.quantize_groups(W, 2, 6, trajectories=True)
    for j in range(4):
        for k in (3, 5):
            zk = res["z_traj"][j, k]
            _, z_ok, _, e = o.round_group(W[j], 2, res["s"][j], res["delta"][j], zk, 10.0 * 1.01 ** k, 0.7)
            _, z_bad, _, _ = o.round_group(W[j], 2, res["s"][j], res["delta"][j], zk, 10.0, 0.7)
            assert np.any(e != 0)
            assert abs(z_ok - res["z_traj"][j, k + 1]) <= 1e-12
            assert abs(z_bad - res["z_traj"][j, k + 1]) > 1e-9


# ----------------------------------------------------------------------------- stop rule

def pin_stop_rule(o):
    """Hand-built MAE sequences: strictly decreasing never stops (keep z_iters); a tie or an
    increase at round k stops there and keeps z_(k-1); round 0 is always accepted."""
    assert o.stop_iter([5, 4, 3, 2, 1], 5) == (5, 5)
    assert o.stop_iter([5, 4, 4, 2, 1], 5) == (1, 3)
    assert o.stop_iter([5, 6, 1, 0, 0], 5) == (0, 2)
    assert o.stop_iter([5, 4, 3, 3.0000001, 1], 5) == (2, 4)
    assert o.stop_iter([1.0], 1) == (1, 1)
    assert o.stop_iter([], 0) == (0, 0)


def pin_stop_in_solver(o):
    """A tensor whose groups all reach a fixed point: the loop stops on the first repeated
    MAE and keeps the zero that reached it; the codes equal those of the kept zero."""
    r = _rng(23)
    W = r.normal(0, 0.02, (8, 64)).astype(np.float16).astype(np.float64)
    res = o.quantize(W, nbits=4, group_size=64, axis=1, iters=30)
    k = res["kout"]
    assert res["rounds"] == k + 2 and k + 2 <= 30
    assert not (res["mae"][k + 1] < res["mae"][k])
    assert all(res["mae"][i + 1] < res["mae"][i] for i in range(k))
    g = o.quantize_groups(W.reshape(-1, 64), 4, k)
    assert np.array_equal(g["z"], res["z"])
    assert np.array_equal(g["codes"].reshape(W.shape), res["codes"])


def pin_stop_rule_variants(o):
    """The alternative readings of the rollback on hand-built MAE sequences: on a stop at round
    k the kept zero is z_(k-1) (rule 0), z_k (1) or z_(k+1) (2); flag 4 changes only the result
    of a loop that never stops (z_(iters-1) instead of z_iters); the rounds evaluated never
    depend on the rule."""
    cases = [([5, 4, 3, 3.5, 2], 5, 3), ([5, 4, 4], 3, 2), ([5, 6, 1], 3, 1)]
    for mae, iters, kstar in cases:
        for rule in (0, 1, 2, 4, 5, 6):
            assert o.stop_iter(mae, iters, rule) == (kstar - 1 + (rule & 3), kstar + 1), (mae, rule)
    for rule, expect in ((0, 4), (1, 4), (2, 4), (4, 3), (5, 3), (6, 3)):
        assert o.stop_iter([5, 4, 3, 2], 4, rule) == (expect, 4)
        assert o.stop_iter([], 0, rule) == (0, 0)


def pin_stop_rule_zero_choice(o):
    """Each rule keeps the zero it names: the codes and zeros equal those of the per-group steps
    run for exactly that many rounds with no stop decision (k* - 1, k*, k* + 1 on a tensor that
    stops at k*; iters - 1 under flag 4 on one that never stops)."""
    r = _rng(23)
    W = r.normal(0, 0.02, (8, 64)).astype(np.float16).astype(np.float64)
    base = o.quantize(W, nbits=4, group_size=64, axis=1, iters=30)
    kstar = base["rounds"] - 1
    assert kstar + 1 <= 30 and base["kout"] == kstar - 1
    for rule in (0, 1, 2):
        res = o.quantize(W, nbits=4, group_size=64, axis=1, iters=30, stop_rule=rule)
        assert res["kout"] == kstar - 1 + rule and res["rounds"] == base["rounds"]
        assert np.array_equal(res["mae"], base["mae"])
        g = o.quantize_groups(W.reshape(-1, 64), 4, kstar - 1 + rule)
        assert np.array_equal(g["z"], res["z"]) and np.array_equal(g["codes"].reshape(W.shape), res["codes"])
    W2 = r.normal(0, 0.02, (4, 128)).astype(np.float16).astype(np.float64)
    full = o.quantize(W2, nbits=3, group_size=64, axis=1, iters=2)
    assert full["rounds"] == 2 and full["kout"] == 2  # too few rounds to stop
    res = o.quantize(W2, nbits=3, group_size=64, axis=1, iters=2, stop_rule=4)
    g = o.quantize_groups(W2.reshape(-1, 64), 3, 1)
    assert res["kout"] == 1 and np.array_equal(g["z"], res["z"])
    assert np.array_equal(g["codes"].reshape(W2.shape), res["codes"])


# ----------------------------------------------------------------------------- group view

def pin_group_view(o):
    """axis=1 groups are reshape([-1, g]) rows; axis=0 groups are the columns of
    reshape([g, -1]) (numpy's reshape of the row-major tensor)."""
    rows, cols = 16, 24
    flat = np.arange(rows * cols)
    for g in (4, 8, 16):
        if cols % g == 0:
            v1 = flat.reshape(-1, g)
            for j in range(v1.shape[0]):
                assert [o.group_elem(rows, cols, g, 1, j, i) for i in range(g)] == list(v1[j])
        v0 = flat.reshape(g, -1)
        for j in range(v0.shape[1]):
            assert [o.group_elem(rows, cols, g, 0, j, i) for i in range(g)] == list(v0[:, j])


def pin_axis0_statistics(o):
    """axis=0 quantisation takes min/max over columns of reshape([g, -1]): for a tensor whose
    column structure differs from its row structure, each group's min maps to 0."""
    r = _rng(29)
    W = r.normal(0, 0.02, (32, 16))
    W[:, 3] += 1.0
    res = o.quantize(W, nbits=4, group_size=16, axis=0, iters=0)
    view = W.reshape(16, -1)
    cview = res["codes"].reshape(16, -1)
    for j in range(view.shape[1]):
        assert cview[np.argmin(view[:, j]), j] == 0 and cview[np.argmax(view[:, j]), j] == 15


# ----------------------------------------------------------------------------- packing

def pin_pack_exhaustive(o):
    """4-bit: every (c0, c1) pair gives byte c0 + 16 c1 and unpacks back ([1, 2] -> 0x21).
    2-bit: every quad gives sum c_t 4^t.  3-bit: every value in every slot of a word lands at
    bits 3t, bits 30-31 stay zero, the tail is padded with zeros."""
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    codes = np.stack([a.reshape(-1), b.reshape(-1)], 1).reshape(-1).astype(np.uint8)
    pk = o.pack(codes, 4)
    assert (pk == (a + 16 * b).reshape(-1)).all()
    assert (o.unpack(pk, codes.size, 4) == codes).all()
    assert o.pack(np.array([1, 2], np.uint8), 4)[0] == 0x21
    quads = np.array([[(v >> (2 * t)) & 3 for t in range(4)] for v in range(256)], np.uint8).reshape(-1)
    pk2 = o.pack(quads, 2)
    assert (pk2 == np.arange(256)).all() and (o.unpack(pk2, quads.size, 2) == quads).all()
    for t in range(10):
        for v in range(8):
            c = np.zeros(10, np.uint8)
            c[t] = v
            word = int.from_bytes(o.pack(c, 3).tobytes(), "little")
            assert word == v << (3 * t) and word >> 30 == 0
    r = _rng(31)
    for n in range(1, 41):
        c = r.integers(0, 8, n).astype(np.uint8)
        pk3 = o.pack(c, 3)
        assert pk3.size == 4 * ((n + 9) // 10)
        assert (o.unpack(pk3, n, 3) == c).all()
        words = pk3.view("<u4")
        assert (words >> 30 == 0).all()
        if n % 10:
            assert words[-1] >> (3 * (n % 10)) == 0


def pin_storage_sizes(o):
    """4-bit g64 with fp16 scale and zero costs 36 bytes per 64 weights = 4.5 bits/weight;
    the INT4 g128 scale-only overhead is 2/128 B/param = 3.125 %, ~3.6 GB for 7B."""
    f = _load("storage_sizes.json")
    h = f["hqq_group_cost"]
    N, g = 64 * 1024, h["group_size"]
    G = N // g
    packed = o.packed_bytes(N, h["nbits"])
    assert packed // G == h["code_bytes_per_group"]
    assert (packed * 8 + G * h["meta_bits_per_group"]) / N == h["bits_per_weight"]
    for nbits, (per, size) in f["packing"]["codes_per_container"].items():
        assert o.packed_bytes(per * 1000, int(nbits)) == size * 1000
    i4 = f["int4_g128_scale_only"]
    per_param = o.packed_bytes(1 << 20, 4) / (1 << 20)
    over = i4["scale_bytes"] / i4["group_size"]
    assert over == i4["overhead_bytes_per_param"] and over / per_param == i4["overhead_fraction"]
    assert round(i4["params"] * (per_param + over) / 1e9, 1) == i4["approx_total_gb"]
    # 3-bit g64 with fp16 metadata: 3.2 bits/code + 0.5 = 3.7; 2-bit g16: 2 + 2 = 4.0
    N = 640 * 64
    assert (o.packed_bytes(N, 3) * 8 + (N // 64) * 32) / N == 3.7
    assert (o.packed_bytes(N, 2) * 8 + (N // 16) * 32) / N == 4.0


# ----------------------------------------------------------------------------- dequant / gemv

def pin_dequant(o):
    """Dequantisation is linear in the code: W_hat = (q - z) delta; fp16 output is the
    nearest-even rounding of the exact value (numpy's conversion); a constant group comes
    back exactly."""
    r = _rng(37)
    for nbits, g, axis in [(4, 64, 1), (3, 64, 1), (2, 16, 1), (4, 16, 0)]:
        rows, cols = 32, 128
        codes = r.integers(0, 1 << nbits, (rows, cols)).astype(np.uint8)
        G = rows * cols // g
        delta = r.uniform(1e-3, 0.1, G).astype(np.float16).astype(np.float64)
        zero = r.uniform(-2, 17, G).astype(np.float16).astype(np.float64)
        w64, w16 = o.dequant(o.pack(codes, nbits), delta, zero, rows, cols, nbits, g, axis)
        assert (w16 == w64.astype(np.float16).view(np.uint16)).all()
        # the value at code 0 of each group is -z*delta; each code step adds delta
        for j in range(0, G, 7):
            idx = [o.group_elem(rows, cols, g, axis, j, i) for i in range(g)]
            vals = w64.reshape(-1)[idx]
            cds = codes.reshape(-1)[idx].astype(np.float64)
            A = np.stack([cds, np.ones(g)], 1)
            sol = np.linalg.lstsq(A, vals, rcond=None)[0]
            assert abs(sol[0] - delta[j]) <= 1e-12 * max(1, delta[j]) and \
                abs(sol[1] + zero[j] * delta[j]) <= 1e-12 * max(1.0, abs(zero[j] * delta[j]))


def pin_gemv(o):
    """y = x W_hat^T: a one-hot x returns a column of W_hat exactly; y is linear in x; it
    equals numpy's matmul of the dequantised weight; a row selection returns the same rows."""
    r = _rng(41)
    N, K, g = 24, 256, 64
    codes = r.integers(0, 16, (N, K)).astype(np.uint8)
    delta = r.uniform(1e-3, 0.05, N * K // g).astype(np.float16).astype(np.float64)
    zero = r.uniform(0, 15, N * K // g).astype(np.float16).astype(np.float64)
    pk = o.pack(codes, 4)
    w64, _ = o.dequant(pk, delta, zero, N, K, 4, g, 1)
    onehot = np.zeros((3, K))
    for b, k in enumerate((0, 77, 255)):
        onehot[b, k] = 1.0
    y = o.gemv(pk, delta, zero, N, K, g, onehot)
    assert (y == w64[:, [0, 77, 255]].T).all()
    x1 = r.normal(0, 1, (2, K)).astype(np.float16).astype(np.float64)
    x2 = r.normal(0, 1, (2, K)).astype(np.float16).astype(np.float64)
    y1, y2 = o.gemv(pk, delta, zero, N, K, g, x1), o.gemv(pk, delta, zero, N, K, g, x2)
    y12 = o.gemv(pk, delta, zero, N, K, g, 2 * x1 + 0.5 * x2)
    assert np.allclose(y12, 2 * y1 + 0.5 * y2, rtol=1e-12, atol=1e-12)
    assert np.allclose(y1, x1 @ w64.T, rtol=1e-12, atol=1e-12)
    sel = np.array([5, 0, 23])
    assert np.array_equal(o.gemv(pk, delta, zero, N, K, g, x1, rows_sel=sel), y1[:, sel])


def pin_gemv_formats(o):
    """The product for every stored format (2-, 3-, 4-bit; axis 1 and axis 0): it equals the
    plain matmul of the dequantised weight, a one-hot x returns a column of W_hat exactly, and
    at 4 bits axis 1 it equals the 4-bit product above.  Shapes where the 3-bit rows start
    inside a word (K not a multiple of 10) and where axis-0 groups stride over rows."""
    r = _rng(47)
    cases = [(4, 64, 1, 16, 256), (4, 128, 0, 256, 96), (4, 16, 0, 32, 64), (2, 16, 1, 12, 128), (2, 32, 0, 64, 32),
             (3, 64, 1, 9, 192), (3, 16, 0, 48, 40)]
    for nbits, g, axis, N, K in cases:
        G = N * K // g
        codes = r.integers(0, 2 ** nbits, (N, K)).astype(np.uint8)
        delta = r.uniform(1e-3, 0.05, G).astype(np.float16).astype(np.float64)
        zero = r.uniform(0, 2 ** nbits - 1, G).astype(np.float16).astype(np.float64)
        pk = o.pack(codes, nbits)
        w64, _ = o.dequant(pk, delta, zero, N, K, nbits, g, axis)
        w64 = w64.reshape(N, K)
        x = r.normal(0, 1, (3, K)).astype(np.float16).astype(np.float64)
        y = o.gemv_fmt(pk, delta, zero, N, K, nbits, g, axis, x)
        assert np.allclose(y, x @ w64.T, rtol=1e-12, atol=1e-12), (nbits, g, axis)
        onehot = np.zeros((2, K))
        onehot[0, 0] = onehot[1, K - 1] = 1.0
        y1 = o.gemv_fmt(pk, delta, zero, N, K, nbits, g, axis, onehot)
        assert (y1 == w64[:, [0, K - 1]].T).all(), (nbits, g, axis)
        if nbits == 4 and axis == 1:
            assert np.array_equal(y, o.gemv(pk, delta, zero, N, K, g, x))


def pin_gemv_transposed(o):
    """The input gradient dX = dY W_hat (every stored format): the adjoint of the forward
    product (<dY, W_hat x> = <dY W_hat, x> with the forward product computed by its own code
    path), one-hot rows of dY return rows of W_hat exactly, and selected columns equal the full
    result's columns."""
    r = _rng(53)
    cases = [(4, 64, 1, 16, 256), (4, 128, 0, 256, 96), (2, 16, 1, 12, 128), (3, 64, 1, 9, 192), (3, 16, 0, 48, 40)]
    for nbits, g, axis, N, K in cases:
        G = N * K // g
        codes = r.integers(0, 2 ** nbits, (N, K)).astype(np.uint8)
        delta = r.uniform(1e-3, 0.05, G).astype(np.float16).astype(np.float64)
        zero = r.uniform(0, 2 ** nbits - 1, G).astype(np.float16).astype(np.float64)
        pk = o.pack(codes, nbits)
        dy = r.normal(0, 1, (3, N))
        x = r.normal(0, 1, (1, K))
        dx = o.gemv_t(pk, delta, zero, N, K, nbits, g, axis, dy)
        y = o.gemv_fmt(pk, delta, zero, N, K, nbits, g, axis, x)  # [1, N]
        lhs = dy @ y[0]
        rhs = dx @ x[0]
        assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10), (nbits, g, axis)
        w64, _ = o.dequant(pk, delta, zero, N, K, nbits, g, axis)
        w64 = w64.reshape(N, K)
        onehot = np.zeros((2, N))
        onehot[0, 0] = onehot[1, N - 1] = 1.0
        assert (o.gemv_t(pk, delta, zero, N, K, nbits, g, axis, onehot) == w64[[0, N - 1]]).all(), (nbits, g, axis)
        sel = np.array([K - 1, 0, K // 2])
        assert np.array_equal(o.gemv_t(pk, delta, zero, N, K, nbits, g, axis, dy, cols_sel=sel), dx[:, sel])


def pin_mae_definition(o):
    """Round 0's MAE is the mean |W - W_hat| of the min-max start (the dequantisation of the
    iters=0 codes with fp64 metadata)."""
    r = _rng(43)
    W = r.normal(0, 0.02, (16, 128)).astype(np.float16).astype(np.float64)
    res = o.quantize(W, nbits=4, group_size=64, axis=1, iters=3)
    rtn = o.quantize(W, nbits=4, group_size=64, axis=1, iters=0)
    w64, _ = o.dequant(o.pack(rtn["codes"], 4), rtn["delta"], rtn["z"], 16, 128, 4, 64, 1)
    assert abs(res["mae"][0] - np.abs(W - w64).mean()) <= 1e-15


def pin_codes_in_range(o):
    """Codes stay in [0, 2^b - 1] even when the zero drifts (outliers pull groups)."""
    r = _rng(47)
    for nbits in (2, 3, 4):
        W = r.normal(0, 0.02, (16, 256))
        W[r.integers(0, 16, 20), r.integers(0, 256, 20)] = 0.3
        res = o.quantize(W, nbits=nbits, group_size=32, axis=1, iters=20)
        assert res["codes"].max() <= (1 << nbits) - 1
        w = W[0, :32]
        s, d, z0 = o.init_group(w, nbits)
        for dz in (-3.0, 3.0):
            _, _, q, _ = o.round_group(w, nbits, s, d, z0 + dz, 10.0, 0.7)
            assert q.min() >= 0 and q.max() <= (1 << nbits) - 1
            assert (q.max() if dz > 0 else -q.min()) == (((1 << nbits) - 1) if dz > 0 else 0)


def pin_group_steps_consistent(o):
    """The per-group entry point with the loop's stop index reproduces the whole-tensor
    result (codes and zero), for both axes."""
    r = _rng(53)
    for axis, g in ((1, 64), (0, 16)):
        W = r.normal(0, 0.02, (32, 128)).astype(np.float16).astype(np.float64)
        res = o.quantize(W, nbits=4, group_size=g, axis=axis, iters=20)
        Wg = W.reshape(-1, g) if axis == 1 else W.reshape(g, -1).T
        gr = o.quantize_groups(Wg, 4, res["kout"])
        assert np.array_equal(gr["z"], res["z"])
        cg = gr["codes"] if axis == 1 else gr["codes"].T
        assert np.array_equal(cg.reshape(W.shape), res["codes"])


# ----------------------------------------------------------------------------- scale search

def _group_error(o, Wg, codes, z, delta):
    """Pairwise sum of |W - W_hat| per group for given codes / zero / step."""
    what = (codes.astype(np.float64) - z[:, None]) * delta[:, None]
    return np.array([o.sum(np.abs(Wg[j] - what[j])) for j in range(Wg.shape[0])])


def pin_scale_search_identity(o):
    """With the single multiplier 1 the scale search is the default solver run on each group
    alone: every group of a many-group tensor gets the codes, scale and zero that the default
    whole-tensor solver gives a tensor made of that group only (its MAE is the group's error
    sum divided exactly by g, a power of two, so the global stop is the group's own); iters = 0
    is min-max round-to-nearest."""
    r = _rng(31)
    for nbits, g, iters in ((4, 64, 20), (2, 16, 20), (4, 128, 7), (2, 256, 20), (4, 32, 0)):
        W = r.normal(0, 0.02, (4, 2 * g)).astype(np.float16).astype(np.float64)
        W[1, :g] = r.laplace(0, 0.05, g)  # a heavier-tailed group, where the shrink acts
        v2 = o.quantize_v2(W, [1.0], nbits=nbits, group_size=g, iters=iters)
        Wg = W.reshape(-1, g)
        assert np.all(v2["choice"] == 0)
        for j in range(Wg.shape[0]):
            one = o.quantize(Wg[j:j + 1], nbits=nbits, group_size=g, axis=1, iters=iters)
            assert v2["s"][j] == one["s"][0] and v2["z"][j] == one["z"][0]
            assert np.array_equal(v2["codes"].reshape(-1, g)[j], one["codes"][0])


def pin_scale_search_argmin(o):
    """A grid of several multipliers picks, per group, the candidate whose own single-multiplier
    search has the smallest error sum (the first such one on a tie), and returns exactly that
    candidate's codes, scale and zero; a repeated multiplier is never chosen over its first
    copy."""
    r = _rng(37)
    W = r.normal(0, 0.02, (8, 256)).astype(np.float16).astype(np.float64)
    W[3, 17] = 0.2  # an outlier
    grid = [0.9, 1.0, 1.05, 1.1, 0.95, 1.05]
    full = o.quantize_v2(W, grid, nbits=4, group_size=64)
    Wg = W.reshape(-1, 64)
    singles = [o.quantize_v2(W, [c], nbits=4, group_size=64) for c in grid]
    errs = np.array([_group_error(o, Wg, sg["codes"].reshape(-1, 64), sg["z"], sg["delta"]) for sg in singles])
    best = np.argmin(errs, axis=0)
    assert np.array_equal(full["choice"], best) and np.all(full["choice"] != 5)
    assert len(set(best.tolist())) >= 3  # the grid matters on these groups
    for j, c in enumerate(best):
        sg = singles[c]
        assert full["s"][j] == sg["s"][j] and full["z"][j] == sg["z"][j]
        assert np.array_equal(full["codes"].reshape(-1, 64)[j], sg["codes"].reshape(-1, 64)[j])
    base = _group_error(o, Wg, singles[1]["codes"].reshape(-1, 64), singles[1]["z"], singles[1]["delta"])
    mine = _group_error(o, Wg, full["codes"].reshape(-1, 64), full["z"], full["delta"])
    assert np.all(mine <= base)


def pin_scale_search_axis0(o):
    """Axis-0 groups of a [g, M] tensor are its columns, which are the axis-1 groups of its
    transpose: the scale search gives the same steps, zeros and choices, and the transposed
    codes; for a taller tensor the groups follow reshape([g, -1])."""
    r = _rng(43)
    for nbits, g in ((4, 64), (3, 32), (2, 16)):
        W = r.normal(0, 0.02, (g, 24)).astype(np.float16).astype(np.float64)
        a0 = o.quantize_v2(W, [0.9, 1.0, 1.1], nbits=nbits, group_size=g, axis=0)
        a1 = o.quantize_v2(np.ascontiguousarray(W.T), [0.9, 1.0, 1.1], nbits=nbits, group_size=g, axis=1)
        assert np.array_equal(a0["z"], a1["z"]) and np.array_equal(a0["s"], a1["s"])
        assert np.array_equal(a0["choice"], a1["choice"]) and np.array_equal(a0["codes"], a1["codes"].T)
    W = r.normal(0, 0.02, (128, 16)).astype(np.float16).astype(np.float64)
    a0 = o.quantize_v2(W, [1.0, 1.05], nbits=4, group_size=64, axis=0)
    view = W.reshape(64, -1)
    a1 = o.quantize_v2(np.ascontiguousarray(view.T), [1.0, 1.05], nbits=4, group_size=64, axis=1)
    assert np.array_equal(a0["z"], a1["z"])
    assert np.array_equal(a0["codes"].reshape(64, -1), a1["codes"].T)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
