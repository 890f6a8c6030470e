"""The oracle against mathematics-fixed pins (CPU only)."""
import pytest

import oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    msgs = pin(O)
    assert not msgs, "\n".join(msgs)
