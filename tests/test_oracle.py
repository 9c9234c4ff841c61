"""The CPU oracle against its pins (library routines, exact integer arithmetic,
a dense formulation and identities of the method).  No GPU needed."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
