"""The CPU oracle against facts fixed by the pages and by mathematics
(hand-worked matrices, the pages' worked example, closed forms, exact
integer arithmetic, invariants, numpy's own decoding, brute-force argmax)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
