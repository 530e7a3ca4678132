"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

This shows the pins are not vacuous: a dropped term, a wrong tie rule, a wrong
GELU form, a missing renormalisation or a wrong capacity rule each fails at
least one of them.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import test_oracle_pins as P
from tests import test_oracle_router_extras as RX
from tests import test_oracle_shared_experts as SX
from tests import test_oracle_capacity as CX


def _tanh_gelu(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _no_renorm(p, idx, renormalize):
    return np.take_along_axis(p, idx, axis=-1)


def _ties_to_higher(g, k):
    E = g.shape[-1]
    rev = g[:, ::-1]
    order = E - 1 - np.argsort(-rev, axis=-1, kind="stable")
    idx = order[:, :k]
    ranked = np.take_along_axis(g, order, axis=-1)
    last = min(k + 1, E)
    margin = (ranked[:, :last - 1] - ranked[:, 1:last]).min(axis=-1) if last >= 2 else np.full(g.shape[0], np.inf)
    return idx, margin


def _keep_last(idx, n_experts, capacity):
    T, k = idx.shape
    keep = np.ones((T, k), dtype=bool)
    if capacity:
        seen = np.zeros(n_experts, dtype=np.int64)
        for t in reversed(range(T)):
            e = idx[t, 0]
            keep[t, 0] = seen[e] < capacity
            seen[e] += 1
    return keep


def _aux_all_slots(idx, p, n_experts):
    T = idx.shape[0]
    cnt = np.bincount(idx.ravel(), minlength=n_experts)
    f = cnt / T
    P_ = p.mean(axis=0)
    return float(n_experts * np.sum(f * P_)), f, P_, cnt


def _ffn_no_out_bias(rows64, w1e, b1e, w2e, b2e):
    h = rows64 @ w1e.T
    if b1e is not None:
        h += b1e[None, :]
    return O.gelu_erf(h) @ w2e.T


def _ffn_transposed(rows64, w1e, b1e, w2e, b2e):
    # second matrix applied with the wrong orientation (square only when d == d_ff)
    h = O.gelu_erf(rows64 @ w1e.T + (b1e[None, :] if b1e is not None else 0))
    o = h @ w2e.T[::-1, ::-1]
    return o + (b2e[None, :] if b2e is not None else 0)


def _z_no_square(g):
    m = g.max(axis=-1, keepdims=True)
    return float(np.mean(m[:, 0] + np.log(np.exp(g - m).sum(axis=-1))))


def _selection_ignores_bias(g, b_select64=None):
    return g


def _selection_subtracts_bias(g, b_select64=None):
    return g if b_select64 is None else g - b_select64[None, :]


def _shared_half(inputs, x64_rows):
    r = O.expert_ffn(x64_rows, O.widen(inputs["w1_shared"]), O.widen(inputs.get("b1_shared")),
                     O.widen(inputs["w2_shared"]), O.widen(inputs.get("b2_shared"))) \
        if inputs.get("w1_shared") is not None else None
    return None if r is None else 0.5 * r


def _keep_slot0_only(idx, n_experts, capacity):
    T, k = idx.shape
    keep = np.ones((T, k), dtype=bool)
    if capacity:
        seen = np.zeros(n_experts, dtype=np.int64)
        for t in range(T):
            e = idx[t, 0]
            keep[t, 0] = seen[e] < capacity
            seen[e] += 1
    return keep


_reroute_true = O.reroute


def _reroute_reverse_order(idx, scores, probs, capacity, renormalize):
    T = idx.shape[0]
    rev = np.arange(T)[::-1]
    served, w, rounds, margin = _reroute_true(idx[rev], scores[rev], probs[rev], capacity, renormalize)
    return served[rev], w[rev], rounds, margin[rev]


def _reroute_new_denominator(idx, scores, probs, capacity, renormalize):
    served, w, rounds, margin = _reroute_true(idx, scores, probs, capacity, renormalize)
    if renormalize:
        ps = np.where(served >= 0, np.take_along_axis(probs, np.maximum(served, 0), axis=1), 0.0)
        w = ps / ps.sum(axis=1, keepdims=True)
    return served, w, rounds, margin


MUTATIONS = [
    ("gelu_erf", _tanh_gelu, [P.test_gelu_against_math_erf_and_identities,
                              P.test_single_expert_reduces_to_dense_mlp]),
    ("routing_weights", _no_renorm, [P.test_eight_expert_example_top2]),
    ("topk_by_logit", _ties_to_higher, [P.test_exact_ties_go_to_lower_index]),
    ("capacity_keep", _keep_last, [P.test_capacity_hand_case]),
    ("aux_loss", _aux_all_slots, [P.test_oracle_matches_the_definition_token_by_token]),
    ("expert_ffn", _ffn_no_out_bias, [P.test_single_expert_reduces_to_dense_mlp]),
    ("expert_ffn", _ffn_transposed, [P.test_oracle_matches_the_definition_token_by_token]),
    ("router_z_loss", _z_no_square, [functools.partial(RX.test_z_loss_of_equal_logits_is_log_E_squared, 8),
                                     RX.test_z_loss_of_one_hot_logits]),
    ("selection_scores", _selection_ignores_bias,
     [RX.test_dominant_selection_bias_picks_expert_with_unbiased_weights]),
    ("selection_scores", _selection_subtracts_bias,
     [RX.test_dominant_selection_bias_picks_expert_with_unbiased_weights]),
    ("shared_expert", _shared_half, [SX.test_shared_expert_is_added_with_weight_one,
                                     SX.test_dropped_token_keeps_the_shared_expert]),
    ("capacity_keep", _keep_slot0_only, [CX.test_drop_with_top2_hand_case]),
    ("reroute", _reroute_reverse_order, [CX.test_reroute_top1_hand_case]),
    ("reroute", _reroute_new_denominator, [functools.partial(CX.test_reroute_invariants, 1, 2, 4)]),
]


@pytest.mark.parametrize("name,fake,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fake, pins):
    from tests import _inputs
    _inputs.inputs_for.cache_clear()
    monkeypatch.setattr(O, name, fake)
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught == len(pins), f"mutation of {name} slipped past {len(pins) - caught} pin(s)"
