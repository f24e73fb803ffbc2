"""The fp64 oracle against the pages' worked example, closed forms and
invariants (CPU only)."""
import pytest

import oracle as O
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
