"""The CPU oracle against its pins (no GPU)."""

import pytest

from oracle import accounting, allocator, attention, fp8
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ACCOUNTING_PINS, ids=lambda f: f.__name__)
def test_accounting_pin(pin):
    pin(accounting)


@pytest.mark.parametrize("pin", P.ALLOCATOR_PINS, ids=lambda f: f.__name__)
def test_allocator_pin(pin):
    pin(allocator)


@pytest.mark.parametrize("pin", P.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(attention)


@pytest.mark.parametrize("pin", P.FP8_PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin(fp8)
