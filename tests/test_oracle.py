"""The CPU oracle against its pins (closed forms, invariants, library routines,
brute force, the pages' figures). CPU only."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)
