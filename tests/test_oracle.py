"""CPU pins of the fp64 oracle (no GPU): each pin compares the oracle with something other than
itself (the pages' worked example, library routines, brute force, closed forms, invariants)."""

import pytest

import oracle.gdla_grad as grad
import oracle.gdla_ref as ref
from tests.oracle_pins import ALL_PINS, GRAD_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(ref)


@pytest.mark.parametrize("pin", GRAD_PINS, ids=[p.__name__ for p in GRAD_PINS])
def test_backward_oracle_pin(pin):
    pin(grad)
