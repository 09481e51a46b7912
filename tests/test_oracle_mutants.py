"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is the oracle compiled with one deliberate error (a transposed operand,
a dropped term, a wrong sign, a missing scale, a wrong slot index, a dropped rank
row).  The pin suite has to fail on every one of them and pass on the real build.
"""
import os
import tempfile

import pytest

import oracle
from tests import pins

MUTANTS = {1: "transposed A", 2: "dropped input feature", 3: "wrong sign", 4: "scale ignored",
           5: "neighbouring slot's B", 6: "last rank-row dropped"}


@pytest.fixture(scope="module", autouse=True)
def _build_mutants():
    for m in MUTANTS:
        path = oracle.lib_path(m)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(oracle._SRC):
            oracle.build(m)
    yield


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_mutant(mutant):
    assert pins.failures(mutant), f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"


def test_real_oracle_passes_all_pins():
    assert pins.failures(0) == []
