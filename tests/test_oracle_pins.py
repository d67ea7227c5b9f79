"""The float64 oracle against closed forms, brute force, hand-derived examples,
an independent chunked algorithm and invariants (see ``oracle_pins.py``)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle._load()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)
