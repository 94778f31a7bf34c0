"""The CPU oracle against the pages' printed values, closed forms, invariants
and a library routine (see oracle_pins.py for what each pin checks)."""
import pytest

import oracle
from oracle_pins import FORMULA_PINS, ORACLE_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ORACLE_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", FORMULA_PINS, ids=lambda f: f.__name__)
def test_formula_pin(pin):
    pin()
