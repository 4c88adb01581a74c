"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_model_table_shapes():
    """FFN width 4H with an MoE layer in every other layer reproduces the page's
    parameter counts (within 1%, under one of the two counting conventions)."""
    for m in P.load_golden("model_table.json")["models"]:
        H, L, E, dense = m["hidden"], m["layers"], m["experts"], m["dense_billions"] * 1e9
        moe_layers = L // 2
        expert_params = moe_layers * E * 2 * H * (4 * H)
        added = dense + expert_params
        replaced = dense - moe_layers * 8 * H * H + expert_params
        target = m["billions"] * 1e9
        best = min(abs(added - target), abs(replaced - target)) / target
        assert best < 0.01, (m["name"], added / 1e9, replaced / 1e9)
