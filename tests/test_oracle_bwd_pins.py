"""The CPU backward oracle against its pins (finite differences through the pinned
forward oracle, float64 torch autograd, closed forms and invariants)."""
import pytest

from oracle.attention_bwd_ref import attention_backward
from tests.oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=[p.__name__ for p in ALL_BWD_PINS])
def test_backward_oracle_pin(pin):
    pin(attention_backward)
