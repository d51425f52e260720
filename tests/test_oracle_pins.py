"""The CPU oracle against its pins (closed forms, brute force, invariants, fixtures)."""
import pytest

import oracle
import oracle_pins as pins  # noqa: E402


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle.instance())


def test_generator_gate_moments():
    pins.check_gate_moments(oracle.instance())
