"""The CPU oracle against its pins (library decoders, the OCP E2M1 table,
numpy/torch float64 references, Python sorting and closed-form cases)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)
