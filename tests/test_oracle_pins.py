"""The CPU oracle against its pins (no GPU needed)."""

import numpy as np
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def O():
    oracle.build(force=False)
    return oracle.get()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(O, check):
    check(O)


def test_rejects_bad_arguments(O):
    x = np.zeros((1, 64), np.uint16)
    w = np.zeros((2, 8), np.uint32)
    s = np.zeros((2, 1), np.uint16)
    with pytest.raises(ValueError):
        O.qmm(x, w, s, s, bits=3)
    with pytest.raises(ValueError):
        O.qmm_points(x, w, s, s, [0], [5], bits=4)
