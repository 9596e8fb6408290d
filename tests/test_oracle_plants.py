"""Each deliberately wrong oracle build (one step changed: a sign, an exponent, a dropped
term, a transposed index, a wrong rounding, a missing clamp, ...) fails at least one pin."""
import pytest

import oracle
from tests import oracle_pins

PLANTS = {
    1: "zero point of the min-max start with the wrong sign",
    2: "shrink exponent p instead of p-1",
    3: "zero update drops the shrink term e",
    4: "axis=0 groups taken as axis=1 rows",
    5: "4-bit nibble order swapped",
    6: "stop keeps the zero of the failing round",
    7: "rounding half up instead of half to even",
    8: "no upper clip at 2^b-1",
    9: "dequantisation adds the zero",
    10: "GEMV reads the transposed weight",
    11: "beta not grown between rounds",
    12: "mean divides by g-1",
    13: "qmax = 2^b",
    14: "3-bit slots shifted by one bit",
    15: "scale not limited to 2e4",
    16: "sums accumulated sequentially instead of pairwise",
    17: "product for all formats takes axis-0 groups as axis-1 runs",
    18: "input gradient multiplies by the transposed weight (column index as row)",
    19: "the stop rule that keeps the failing round's zero keeps its update instead",
    20: "the scale search keeps the candidate with the larger error",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: "plant%d" % p)
def test_planted_mistake_is_caught(plant):
    o = oracle.Oracle(oracle.build(plant=plant))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
        except ValueError:
            failed.append(pin.__name__)
    assert failed, "no pin caught plant %d (%s)" % (plant, PLANTS[plant])
