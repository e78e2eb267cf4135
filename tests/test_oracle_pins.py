"""The CPU oracle checked against facts fixed outside itself (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL, ids=[c.__name__[6:] for c in pins.ALL])
def test_pin(check):
    check()
