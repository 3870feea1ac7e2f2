"""The CPU oracle against values and identities the pages and the mathematics fix."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_inputs(orc):
    import numpy as np
    q = np.zeros((4, 2, 8), np.float32)
    k = np.zeros((4, 1, 8), np.float32)
    with pytest.raises(oracle.OracleError) as e:
        orc.prefill(q, k, k, [0, 3, 2, 4], 2, 1, 8, "f32")
    assert e.value.code == -3
    with pytest.raises(oracle.OracleError) as e:
        orc.prefill(q, k, k, [0, 4], 3, 2, 8, "f32")
    assert e.value.code == -1
    pool = np.zeros((2, 2, 1, 4, 8), np.float32)
    qd = np.zeros((1, 2, 8), np.float32)
    kn = np.zeros((1, 1, 8), np.float32)
    with pytest.raises(oracle.OracleError) as e:
        orc.decode(qd, pool, [0], [5], kn, kn, 2, "f32")
    assert e.value.code == -4
    with pytest.raises(oracle.OracleError) as e:
        orc.decode(qd, pool, [2], [1], kn, kn, 2, "f32")
    assert e.value.code == -5
