"""The oracle against the pages' printed values, closed forms, invariants,
brute force over block partitions and an independent library softmax."""

import pytest

import oracle.reference as R
from pin_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(R)
