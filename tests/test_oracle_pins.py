"""The oracle against its pins (library routines, brute force, closed forms,
invariances).  CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def ref():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(ref, pin):
    pin(ref)


def test_threads_reported(ref):
    assert ref.num_threads() >= 1
