"""The oracle against what the pages, the format specs and mathematics fix.

Each test runs one check from pins.py; the mutation tests plant mistakes in
the oracle and expect these same checks to fail.
"""

import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
