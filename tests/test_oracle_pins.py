"""The fp64 oracle against its pins (worked examples, closed forms, brute force,
library routines, invariants). CPU only."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(O, name):
    PINS[name](O)
