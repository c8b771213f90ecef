"""Host-side control of a decode step (TokenButler model card, Method and Memory
requirements), without a GPU: the layer plan the bench and the chain tests run from is
checked against the golden slot table derived from the model card and against the
oracle's producer / slot functions (written separately), and the fixed_<N>pc knob against
the golden policy table."""
import os

import pytest

import oracle
from query_aware_sparse_imp_amd import control

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    return [ln.split() for ln in open(os.path.join(GOLDEN, name))
            if ln.strip() and not ln.startswith("#")]


def test_layer_plan_matches_golden_slot_table():
    plan = control.layer_plan(32, 4)
    rows = _rows("slot_map_g4.txt")
    assert len(plan) == len(rows) == 32
    for role, (layer, producer, slot, dense) in zip(plan, rows):
        assert (role.layer, role.producer, role.slot, role.dense) == \
            (int(layer), int(producer), int(slot), bool(int(dense)))
        assert role.produces == (role.layer == role.producer)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_layer_plan_matches_oracle_for_other_frequencies(G):
    for role in control.layer_plan(32, G):
        assert role.producer == oracle.producer_of(role.layer, G)
        assert role.slot == oracle.slot_of(role.layer, G)
        assert 0 <= role.slot < G and role.producer <= role.layer
        # a producer serves itself (slot G - 1) and the next G - 1 layers (slots 0 .. G-2)
        if role.produces:
            assert role.slot == G - 1


def test_fixed_pc_matches_golden_policy_table():
    for policy, num, den, L, x in _rows("fixed_pc_policy.txt"):
        assert control.fixed_pc(policy) == (int(num), int(den))
        assert (int(L) * int(num)) // int(den) == int(x)
    with pytest.raises(ValueError):
        control.fixed_pc("top_50pc")
    with pytest.raises(ValueError):
        control.layer_plan(0, 4)
