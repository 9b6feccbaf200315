"""Plant a mistake in the oracle (on the CPU) and check that a pin catches it.

Each mutant is the oracle source rebuilt with -DKVCO_MUTANT=n, which switches
on one plausible error: a dropped term, a wrong index, an off-by-one, a
transposed operand.  The pins must reject every one of them."""
import os

import pytest

import oracle
from oracle import build as obuild
import oracle_pins

MUTANTS = {
    1: "own key excluded from the mask",
    2: "scale dropped",
    3: "query head mapped to kv head h % Hkv",
    4: "slot index reversed inside a block",
    5: "append one position late",
    6: "K used in place of V",
    7: "softmax normaliser dropped",
    8: "cached-length offset ignored in the mask",
    9: "row offset of the sequence ignored for q",
    10: "block table ignored",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_mutant(mutant, tmp_path):
    lib = obuild.build(str(tmp_path / f"liboracle_m{mutant}.so"), mutant=mutant)
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:  # ValueError: oracle refused
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"
