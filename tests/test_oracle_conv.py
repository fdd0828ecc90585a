"""The CPU reference convolution and im2col against their pins (CPU only)."""
import pytest

import oracle
from tests import oracle_conv_pins


@pytest.mark.parametrize("pin", oracle_conv_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_conv_pin(pin):
    pin(oracle.load())
