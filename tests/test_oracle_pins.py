"""The CPU oracle against its pins (tests/pins.py): conversions against numpy
and torch casts, codes against brute force, error bounds, exact round trips of
zero and constant blocks, the FP closed form, and hand-worked fixtures."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.QUICK_CHECKS + [pins.check_h2f_exhaustive],
                         ids=lambda c: c.__name__)
def test_pin(oracle_lib, check):
    check(oracle_lib)


def test_constants_exhaustive(oracle_lib):
    pins.check_constants_exhaustive(oracle_lib)
