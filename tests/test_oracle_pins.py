"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.QUICK_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_exhaustive_alphabet_2_n8(o):
    pins.pin_bruteforce_exhaustive(o, max_n=8, alphabet_size=2)


def test_float_transform_roundtrip_exhaustive(o):
    pins.pin_float_transform_roundtrip_exhaustive(o)
