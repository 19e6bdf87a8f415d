"""The CPU oracle against its pins (brute force, library routine, invariants,
closed forms, hand-worked examples, pair counts)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib_path():
    oracle.lib()
    return oracle._LIB


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib_path):
    fails = pin(lib_path)
    assert not fails, "\n".join(fails[:20])
