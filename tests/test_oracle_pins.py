"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_argument_errors(orc):
    assert orc.raw_step_code(1, 3, 2, 1, 4, 2, 2) == oracle.Oracle(orc.path).raw_step_code(1, 3, 2, 1, 4, 2, 2)
    assert orc.raw_step_code(1, 3, 2, 1, 4, 2, 2) == -1  # Hq not a multiple of Hk
    assert orc.raw_step_code(0, 2, 2, 1, 4, 2, 2) == -1  # B < 1
    assert orc.raw_step_code(1, 2, 2, -1, 4, 2, 2) == -1  # Q < 0
    assert orc.raw_step_code(1, 2, 2, 1, 0, 2, 2) == -1  # M < 1
    assert orc.raw_step_code(1, 2, 2, 1, 4, 2, 2, dtype=7) == -3
    assert orc.raw_step_code(1, 2, 2, 1, 4, 2, 2, has_scale=1, scale=-2.0) == -2
