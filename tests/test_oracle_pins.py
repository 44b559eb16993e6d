"""The fp64 oracle against its pins (CPU only)."""
import pytest

from pins import PINS
from pins_backward import BACKWARD_PINS
from pins_ex import EX_PINS
from pins_rowsparse import ROWSPARSE_PINS

ALL = PINS + ROWSPARSE_PINS + EX_PINS + BACKWARD_PINS


@pytest.mark.parametrize("pin", ALL, ids=[p.__name__ for p in ALL])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)
