"""The CPU oracle against its pins (hand-worked values, brute force by the
stock FSDP2 path, closed forms, invariants, error bounds)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check, oracle_mod):
    check(oracle_mod.Oracle())


def test_plan_rejects_bad_shapes(oracle_mod):
    orc = oracle_mod.Oracle()
    with pytest.raises(oracle_mod.OracleError):
        orc.plan(4, [()])  # 0-d parameter
    with pytest.raises(oracle_mod.OracleError):
        orc.plan(4, [(3, -1)])
    with pytest.raises(oracle_mod.OracleError):
        orc.plan(0, [(3,)])
    with pytest.raises(oracle_mod.OracleError):
        orc.plan(2, [(2**62, 2**3)])  # D*K overflows int64


def test_plan_allows_empty_dims(oracle_mod):
    geo = oracle_mod.Oracle().plan(4, [(0, 5), (3, 0), (2,)])
    assert list(geo["R"]) == [0, 1, 1]
    assert list(geo["n"]) == [0, 0, 1]
    assert geo["S"] == 1
