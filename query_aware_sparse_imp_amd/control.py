"""Host-side control of a decode step: no kernels, integers only.

TokenButler model card, section Method: producer layers sit at 0, G, 2G, ...; a producer
predicts importance queries for itself and the next G - 1 layers, G slots of Q_imp, and
consumer layer l reads slot (l - 1) mod G of its producer's output.  Section Memory
requirements: the first layer stays dense, the policy ``fixed_<N>pc`` prunes N% of the
tokens (it retains 100 - N percent), with a sink prefix (``min_sparse_index``) and a
recent window (``sliding_window``) always kept.

The caller turns a layer's role into the arguments of the C ABI: the producer's Q_imp
buffer and ``slot`` for butler_score / butler_project_and_score, the budget fraction for
butler_select_topk / butler_select_attend (budget 1/1 for the dense layer).
"""
from __future__ import annotations

from typing import List, NamedTuple, Tuple


class LayerRole(NamedTuple):
    layer: int
    producer: int      # the layer whose Q_imp this layer scores with
    slot: int          # which of the producer's G slots
    produces: bool     # this layer runs f_theta (its Q_imp serves itself and the next G-1)
    dense: bool        # attends to every token (no selection)


def layer_plan(n_layers: int, G: int) -> List[LayerRole]:
    """Role of every layer of an n_layers model with producer frequency G."""
    if n_layers <= 0 or G <= 0:
        raise ValueError("n_layers and G must be positive")
    plan = []
    for layer in range(n_layers):
        first_of_block = layer - layer % G          # producers at 0, G, 2G, ...
        plan.append(LayerRole(layer=layer, producer=first_of_block,
                              slot=(layer + G - 1) % G, produces=layer % G == 0,
                              dense=layer == 0))
    return plan


def fixed_pc(policy: str) -> Tuple[int, int]:
    """'fixed_<N>pc' -> the retained fraction (100 - N) / 100 as (num, den), the budget
    arguments of the selection calls (x = floor(L * num / den))."""
    if not (policy.startswith("fixed_") and policy.endswith("pc")):
        raise ValueError(f"not a fixed_<N>pc policy: {policy!r}")
    n = int(policy[len("fixed_"):-len("pc")])
    if not 0 <= n <= 100:
        raise ValueError(f"pruned percentage out of range: {n}")
    return 100 - n, 100
