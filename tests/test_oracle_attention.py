"""The attention oracle against its pins (CPU)."""
import pytest

import oracle.attention as at
from tests import oracle_attention_pins as pins


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_attention_oracle_pin(check):
    check(at)
