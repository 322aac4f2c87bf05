"""The CPU oracle against its pins (closed forms, exhaustive enumeration,
brute force, hand-derived containers, the pages' worked example)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(ref, check):
    check(ref)
