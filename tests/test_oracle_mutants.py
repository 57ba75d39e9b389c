"""Mutation test: each planted mistake in the oracle must be caught by some pin.

The mistakes are compiled into separate copies of the C oracle (ORACLE_MUTANT=n)
on the CPU; the real oracle is untouched. A mutant that no pin catches means the
pins are too weak to vouch for the oracle.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    1: "sink left out of the softmax denominator",
    2: "index -1 read as the last row",
    3: "softmax scale dropped",
    5: "duplicate slots collapsed",
    6: "mask word index off by one",
    7: "mask bit order reversed",
    8: "key start stored in word 0",
    9: "mask ignored by masked attention",
    10: "keys used as values in masked attention",
    11: "every head uses head 0's query",
    12: "masked attention scale applied twice",
    13: "chunked form ignores key_start",
    14: "chunked form reads key_start from the query's own row",
    15: "chunked form reads the reserved word as mask bits",
    16: "candidate blocks counted from column 0 instead of the start",
    17: "candidate edge flag ignored",
    18: "FP8 scale tile index off by one",
    19: "e4m3 exponent bias 8",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(tmp_path, mutant):
    path = os.path.join(str(tmp_path), f"liboracle_m{mutant}.so")
    oracle.build(path, mutant=mutant, openmp=False)
    o = oracle.Oracle(oracle._bind(__import__("ctypes").CDLL(path)))
    caught = []
    for check in pins.ALL_PINS:
        try:
            check(o)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
