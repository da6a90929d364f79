"""The fp64 reference convolution checked against closed forms, invariants,
brute force, torch's float64 convolution and hand-worked examples."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_mod):
    pin(oracle_mod._load())
