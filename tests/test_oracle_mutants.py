"""Planted mistakes in the oracle must be caught by at least one pin.

Each mutant is oracle.c compiled with -DMXO_MUTANT=k, which plants one
plausible error: a wrong GQA head mapping, a top-left causal mask, a wrong
scale, a dropped channel in the dot product, an off-by-one V row, a missing
normalisation, an lse without its max term, K used in place of V.
"""
import os
import tempfile

import pytest

import oracle
import pins

MUTANTS = {
    1: "GQA head h -> h % Hkv",
    2: "causal mask aligned top-left",
    3: "scale 1/D instead of 1/sqrt(D)",
    4: "last channel dropped from q.k",
    5: "V row j+1 used for key j",
    6: "output not divided by l",
    7: "lse without the max term",
    8: "K rows used as values",
}


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"mutant{m}")
def test_some_pin_catches_mutant(mutant, mutant_dir):
    path = oracle.compile_oracle(os.path.join(mutant_dir, f"libm{mutant}.so"), mutant)
    assert oracle.load(path).mxo_mutant_id() == mutant
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(path)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mutant}: {MUTANTS[mutant]}"
