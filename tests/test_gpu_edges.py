"""GPU parity of the method's edge cases on every quantizer instantiation (2/3/4-bit codes, group
sizes 16..256, axis 0 and 1) at 0, 1, 2 and 20 rounds.

Two inputs per instantiation, both built in the group view and mapped back to the weight layout:
  * degenerate groups (HQQ page, "第一拍": s = 1 for a tiny range, s limited to 2e4): a constant
    group, an all-zero group, a range below the tiny-range threshold, a range that hits the 2e4
    limit at every bit width, a group whose start puts every code on an exact rounding tie
    ("量化公式": round to nearest, ties to even), single outliers, and N(0, 0.02) groups; the
    shrink stays exactly zero on all of them, so codes, steps, zeros and the MAE trace must be
    bit-identical to the oracle;
  * sigma-1 and sigma-3 groups among N(0, 0.02) ones ("shrink 不是删除极值"): residuals pass the
    shrink threshold beta^(-1/(2-p)), so the solver's pow() slow path runs; pow() may differ in its
    last bit between the device and the host library, so zeros and steps are held to 1e-5
    relative and codes to >= 99.99 % equal, the stop round exactly.
The shapes span two full solve tiles and a ragged third (axis 1: 4 GPW groups per block; axis 0:
the same number of columns per block)."""
import numpy as np
import pytest

import oracle
from tests.gpu_common import compare_quant, gpu_quantize, say

pytestmark = pytest.mark.gpu

GROUPS = (16, 32, 64, 128, 256)
BITS = (2, 3, 4)
ITERS = (0, 1, 2, 20)


def groups_per_block(g: int) -> int:
    """Groups one solve block holds: 4 waves x 64 / L groups, L = lanes per group."""
    lanes = {16: 4, 32: 4, 64: 8, 128: 16, 256: 16}[g]
    return 4 * 64 // lanes


def layout(V: np.ndarray, g: int, axis: int, rows: int, cols: int) -> np.ndarray:
    """Weight [rows, cols] whose group view (axis 1: reshape([-1, g]); axis 0: columns of
    reshape([g, -1])) is V [G, g]."""
    if axis == 1:
        return V.reshape(rows, cols)
    return np.ascontiguousarray(V.T).reshape(rows, cols)


def shape_for(g: int, axis: int, min_groups: int):
    """rows, cols with at least min_groups groups and a ragged last tile."""
    gpb = groups_per_block(g)
    G = max(min_groups, 2 * gpb + gpb // 2 + 3)
    if axis == 1:
        cols = 2 * g
        rows = (G + 1) // 2
        return rows, cols
    # axis 0: rows = 2 g (two row phases), M = 2 cols groups; (rows / g) cols % 8 == 0
    cols = (G // 2 + 3) // 4 * 4
    if (2 * cols) % gpb == 0:
        cols += 4
    return 2 * g, cols


def degenerate_groups(g: int, nbits: int, G: int, seed: int) -> np.ndarray:
    r = np.random.default_rng(seed)
    qmax = (1 << nbits) - 1
    V = r.normal(0.0, 0.02, (G, g))
    i = np.arange(g)
    V[0] = 0.375                                        # constant: s = 1, z = -c, exact
    V[1] = 0.0                                          # all zero
    V[2] = 0.01 + r.uniform(0.0, 5e-5, g)               # range <= 5e-5: below the threshold, s = 1
    base = float(np.float16(0.02))                      # fp16 grid step near 0.02 is 2^-16
    V[3] = base + 2.0 ** -16 * (i % 9)                  # range 8 * 2^-16 = 1.22e-4: qmax / d > 2e4
    u = 2.0 ** -6                                       # start s = 1/u, z = 0: t = W/u
    V[4] = u * ((i % qmax) + 0.5)                       # every t on a half-integer tie ...
    V[4, 0], V[4, 1] = 0.0, qmax * u                    # ... with min 0 and max qmax u
    V[5, g // 3] = 0.3                                  # single outliers
    V[6, g - 1] = -0.25
    V[7] = -V[4]                                        # ties mirrored (negative range)
    return V


def shrink_groups(g: int, G: int, seed: int) -> np.ndarray:
    r = np.random.default_rng(seed)
    V = r.normal(0.0, 0.02, (G, g))
    sel = r.permutation(G)
    V[sel[: G // 2]] = r.normal(0.0, 1.0, (G // 2, g))
    V[sel[G // 2: G // 2 + G // 4]] = r.normal(0.0, 3.0, (G // 4, g))
    return V


def _quantize_both(W16, nbits, g, axis, iters):
    ref = oracle.get().quantize(W16.astype(np.float64), nbits=nbits, group_size=g, axis=axis, iters=iters)
    gq = gpu_quantize(W16, nbits, g, axis, iters, meta="f64")
    return ref, gq


@pytest.mark.parametrize("iters", ITERS)
@pytest.mark.parametrize("axis", (1, 0))
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("nbits", BITS)
def test_degenerate_groups(nbits, g, axis, iters):
    rows, cols = shape_for(g, axis, 0)
    G = rows * cols // g
    V = degenerate_groups(g, nbits, G, seed=31 * g + nbits)
    W = layout(V, g, axis, rows, cols).astype(np.float16)
    say("degenerate groups", nbits, g, axis, iters, rows, cols)
    ref, gq = _quantize_both(W, nbits, g, axis, iters)
    # the inputs do what they are for (read off the oracle's steps, delta = 1/s)
    assert ref["delta"][0] == 1.0 and ref["delta"][1] == 1.0 and ref["delta"][2] == 1.0
    assert ref["delta"][3] == 1.0 / 2.0e4
    assert ref["delta"][4] == 2.0 ** -6
    compare_quant(W, ref, gq, nbits, g, axis, exact_codes=True, exact=True)


@pytest.mark.parametrize("iters", ITERS)
@pytest.mark.parametrize("axis", (1, 0))
@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("nbits", BITS)
def test_shrink_active(nbits, g, axis, iters):
    rows, cols = shape_for(g, axis, 24576 // g)
    G = rows * cols // g
    V = shrink_groups(g, G, seed=17 * g + nbits)
    W = layout(V, g, axis, rows, cols).astype(np.float16)
    say("shrink active", nbits, g, axis, iters, rows, cols)
    ref, gq = _quantize_both(W, nbits, g, axis, iters)
    if iters:
        # round 0's residuals of the min-max start pass the shrink threshold somewhere
        o = oracle.get()
        Wg = oracle.group_view(W.astype(np.float64), g, axis)
        thr = 10.0 ** (-1.0 / (2.0 - 0.7))
        big = 0
        for j in range(0, Wg.shape[0], max(1, Wg.shape[0] // 64)):
            s, d, z = o.init_group(Wg[j], nbits)
            q = np.clip(np.rint(Wg[j] * s + z), 0, (1 << nbits) - 1)
            big += int(np.sum(np.abs(Wg[j] - (q - z) * d) > thr))
        assert big > 0, "no residual reaches the shrink"
    agree = compare_quant(W, ref, gq, nbits, g, axis, exact_codes=False, exact=False)
    say("  codes agree %.6f" % agree)
