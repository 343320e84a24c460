"""Each planted mistake in the oracle (ccl_oracle.c built with -DORACLE_MUTANT=k)
must be caught by at least one pin: the pins are strong enough to matter."""
import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    1: "up-right neighbour dropped",
    2: "rows wrap (flat-index neighbours)",
    3: "node re-pointed instead of its leader",
    4: "larger leader wins",
    5: "numbers start at 0",
    6: "up-left neighbour dropped",
    7: "32-bit colours compared on the low byte",
    8: "a diagonal joined in 4-connectivity",
    9: "ignored pixels counted as regions",
    10: "the ignored colour still labelled",
    11: "RGB pixels compared on two of their three bytes",
    12: "bounding boxes end one row late",
    13: "column sums take the row index",
    14: "the 64-bit entry point drops the ignored colour",
}


@pytest.fixture(scope="module")
def ref_lib():
    return oracle.load()


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(ref_lib, mutant):
    lib = oracle.load(oracle.build(mutant=mutant))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        kwargs = {}
        if pin in (oracle_pins.pin_random_vs_c_bfs, oracle_pins.pin_exhaustive):
            kwargs["ref_lib"] = ref_lib      # flood fill from the unmodified source
        try:
            pin(lib, **kwargs)
        except (AssertionError, ValueError):
            # a disagreement, or output the oracle's own checks reject (a
            # mutant's leader image that numbers into labels out of range)
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
