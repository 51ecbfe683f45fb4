"""The CPU oracle against its pins (closed forms, special matrices, exact
library cases, brute force on exact rationals, invariants).  CPU only."""
import numpy as np
import pytest

import oracle_pins
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_bad_arguments_rejected(orc):
    A = np.ones(16, np.float32)
    with pytest.raises(ValueError):
        orc.sgemm(-1, 4, 4, 1.0, A, 4, A, 4, 0.0, None, 4)
    with pytest.raises(ValueError):
        orc.sgemm(4, 4, 4, 1.0, A, 3, A, 4, 0.0, None, 4)  # lda < k
    with pytest.raises(ValueError):
        orc.sgemm(4, 4, 4, 1.0, A, 4, A, 4, 0.0, None, 4, rows=[4])


def test_empty_is_noop(orc):
    C = np.full(12, 7.0, np.float32)
    A = np.ones(12, np.float32)
    out = orc.sgemm(0, 3, 4, 1.0, A, 4, A, 3, 0.0, C, 3)["C"]
    assert np.array_equal(out, C)
    out = orc.sgemm(4, 0, 3, 1.0, A, 3, A, 1, 0.0, C, 3)["C"]
    assert np.array_equal(out, C)


def test_pin_module_lists_every_pin():
    names = {n for n in dir(oracle_pins) if n.startswith("pin_")}
    assert names == {p.__name__ for p in ALL_PINS}
