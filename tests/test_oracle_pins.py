"""The fp64 oracle against facts fixed independently of it (CPU only)."""
import pytest

import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check, orc):
    check()
