"""The CPU oracle against facts outside itself (CPU only)."""
import pytest

import oracle
from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.mqa_oracle)


from pins_mla import MLA_PINS  # noqa: E402


@pytest.mark.parametrize("pin", MLA_PINS, ids=lambda p: p.__name__)
def test_mla_oracle_pin(pin):
    pin(oracle.sparse_mla_oracle)
