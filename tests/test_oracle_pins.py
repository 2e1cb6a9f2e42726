"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle.gqa_oracle as O
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)
