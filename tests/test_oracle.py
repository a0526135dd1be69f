"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_bad_arguments_rejected(orc):
    import numpy as np
    Q = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        orc.fwd(Q, np.zeros((1, 1, 2, 3)), np.zeros((1, 1, 2, 3)), 1.0)
    with pytest.raises(RuntimeError):
        orc.online_row([1.0], [[1.0]], tile=0)
    with pytest.raises(RuntimeError):
        orc.fwd_rows(Q, Q, Q, [[5]], 1.0)
