"""The oracle against its pins (pages' printed values, closed forms,
invariances, library routines). CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.default()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_pin(orc, check):
    check(orc)
