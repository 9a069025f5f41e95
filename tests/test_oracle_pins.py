"""The CPU oracle against its pins (closed forms, invariants, brute force, and
torch's SDPA in float64).  CPU only."""
import pytest

from oracle.attention_ref import attention_forward
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(attention_forward)
