"""The fp64 oracle against brute force, library routines, closed forms and invariants."""
import pytest

from tests import pins


@pytest.mark.parametrize("name", sorted(pins.ALL_CHECKS))
def test_oracle_pin(name):
    err = pins.ALL_CHECKS[name]()
    assert err <= pins.TOL, f"{name}: discrepancy {err:.3e}"
