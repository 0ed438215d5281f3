"""The CPU oracle against its pins (see tests/pins.py for what pins what)."""
import pytest

import pins


@pytest.mark.parametrize("name,fn,args", pins.ALL_PINS, ids=[p[0] for p in pins.ALL_PINS])
def test_pin(name, fn, args):
    fn(*args)
