"""The CPU oracle against facts fixed by the pages and by mathematics
(tile-ledger worked example, exact brute force, closed forms, library
special cases).  No GPU needed."""
import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.timeout(300)


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np
    A = np.zeros((4, 31), np.uint8)
    B = np.zeros((31, 4), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm_mxfp8(A, B, np.zeros((4, 0), np.uint8), np.zeros((4, 0), np.uint8))
    with pytest.raises(ValueError):
        orc.gemm_bf16(np.zeros((2, 3), np.uint16), np.zeros((4, 2), np.uint16))
