"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is the oracle C source built with one ``ORACLE_MUTANT`` value;
nothing here touches the GPU path.
"""
import os

import pytest

import oracle
import oracle_pins as P

MUTANTS = {
    1: "ties broken towards the higher index",
    2: "NaN ranked below everything",
    3: "-0 ranked below +0",
    4: "end treated as inclusive",
    5: "short rows NaN-checked",
    6: "padding index 0 instead of -1",
    7: "value copied from the wrong column",
    8: "sorted_index ignored",
    9: "gather batch offset dropped",
    10: "gather position off by one",
    11: "ascending instead of descending",
    12: "input row stride ignored",
    13: "value order reversed",
    14: "masked fill lets position len through",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_catch_planted_mistake(tmp_path, mutant):
    lib = oracle.compile_oracle(os.path.join(str(tmp_path), f"liboracle_m{mutant}.so"), mutant=mutant)
    bad = oracle.Oracle(lib)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(bad)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant}: {MUTANTS[mutant]}"
