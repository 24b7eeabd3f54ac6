"""The oracle against its pins (CPU only): see ``oracle_pins.py`` for what each pins."""

import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_rejects_contract_violations(o):
    x = np.zeros((1, 24), dtype=np.float16)           # K % 16 != 0
    with pytest.raises(ValueError):
        o.linear(x, np.zeros((3, 8), dtype=np.int32), np.ones((1, 8), np.float16), -1)
    x = np.zeros((1, 16), dtype=np.float16)
    with pytest.raises(ValueError):                     # N % 8 != 0
        o.linear(x, np.zeros((2, 12), dtype=np.int32), np.ones((1, 12), np.float16), -1)
    with pytest.raises(ValueError):                     # group size outside the set
        o.linear(x, np.zeros((2, 8), dtype=np.int32), np.ones((1, 8), np.float16), 48)
    with pytest.raises(ValueError):                     # a code above 15
        o.pack(np.full((8, 8), 16, dtype=np.uint8))


def test_empty_batch(o):
    y = o.linear(np.zeros((0, 32), np.float16), np.zeros((4, 8), np.int32),
                 np.ones((1, 8), np.float16), 32)
    assert y.shape == (0, 8)
