"""Pins of the router extras in the oracle: the router z-loss and the
selection-only per-expert bias (web page "Mixture of Experts: Scaling Parameters
Without Scaling Compute", section "The central problem: load balancing": router
z-loss; auxiliary-loss-free balancing with per-expert bias terms).

The pages give no formulas for either; the readings (z = mean over tokens of the
squared log-sum-exp of the logits; the bias only changes which experts are
picked, the weights stay the unbiased softmax) are pinned here against closed
forms, special cases and the two independent variants."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import variants as V


def _tiny(T=6, d=5, F=3, E=4, k=2, seed=3, zero_router=False, b_router=None, b_select=None):
    rng = np.random.default_rng(seed)
    inp = {"x": rng.standard_normal((T, d)).astype(np.float32),
           "w_router": (np.zeros((E, d)) if zero_router else rng.standard_normal((E, d))).astype(np.float32),
           "b_router": None if b_router is None else np.asarray(b_router, np.float32),
           "b_select": None if b_select is None else np.asarray(b_select, np.float32),
           "w1": rng.standard_normal((E, F, d)).astype(np.float32),
           "b1": rng.uniform(-0.1, 0.1, (E, F)).astype(np.float32),
           "w2": rng.standard_normal((E, d, F)).astype(np.float32),
           "b2": rng.uniform(-0.1, 0.1, (E, d)).astype(np.float32)}
    desc = {"tokens": T, "d_model": d, "d_ff": F, "n_experts": E, "top_k": k,
            "renormalize": True, "capacity": 0}
    return inp, desc


@pytest.mark.parametrize("E", [1, 2, 8, 64])
def test_z_loss_of_equal_logits_is_log_E_squared(E):
    """All logits equal (zero router): log-sum-exp = ln E for every token."""
    inp, desc = _tiny(E=E, k=1, zero_router=True)
    assert abs(O.route(inp, desc)["z_loss"] - math.log(E) ** 2) <= 1e-14


def test_z_loss_shifts_with_a_constant_logit_bias():
    """Zero router plus the same bias c on every expert: z = (ln E + c)^2."""
    E, c = 8, 2.5
    inp, desc = _tiny(E=E, k=2, zero_router=True, b_router=np.full(E, c))
    assert abs(O.route(inp, desc)["z_loss"] - (math.log(E) + c) ** 2) <= 1e-13


def test_z_loss_of_one_hot_logits():
    """Token t has logit a_t on one expert and 0 on the others:
    log-sum-exp = ln(e^a_t + E - 1)."""
    E, a = 4, [3.0, -1.0, 0.5, 7.0]
    x = np.eye(4, dtype=np.float32) * np.asarray(a, np.float32)[:, None]
    inp, desc = _tiny(T=4, d=4, E=E, k=1)
    inp["x"], inp["w_router"] = x, np.eye(E, 4, dtype=np.float32)
    want = np.mean([math.log(math.exp(v) + E - 1) ** 2 for v in a])
    assert abs(O.route(inp, desc)["z_loss"] - want) <= 1e-13


def test_z_loss_is_large_for_large_logits_and_ignores_selection_bias():
    inp, desc = _tiny(E=8, k=2)
    z = O.route(inp, desc)["z_loss"]
    inp2 = dict(inp, w_router=inp["w_router"] * np.float32(10.0))
    assert O.route(inp2, desc)["z_loss"] > 10 * z
    inp3 = dict(inp, b_select=np.linspace(-3, 3, 8).astype(np.float32))
    assert O.route(inp3, desc)["z_loss"] == z


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_router_extras_agree_with_both_variants(seed):
    E = 6
    bs = np.random.default_rng(100 + seed).uniform(-1, 1, E)
    inp, desc = _tiny(E=E, k=3, seed=seed, b_router=np.linspace(-0.5, 0.5, E), b_select=bs)
    r = O.forward(inp, desc, check_margin=False)
    dm = V.dense_masked(inp, desc)
    lp = V.loops(inp, desc)
    assert abs(r["z_loss"] - dm["z_loss"]) <= 1e-12 * max(1.0, r["z_loss"])
    assert abs(r["z_loss"] - lp["z_loss"]) <= 1e-12 * max(1.0, r["z_loss"])
    assert np.allclose(r["y"], dm["y"], rtol=1e-12, atol=1e-12)
    assert np.allclose(r["y"], lp["y"], rtol=1e-12, atol=1e-12)
    assert r["topk_idx"][:, 0].tolist() == lp["top1"]
    assert abs(r["aux"] - lp["aux"]) <= 1e-12


def test_zero_selection_bias_changes_nothing():
    inp, desc = _tiny(E=8, k=2, seed=5)
    a = O.route(inp, desc)
    b = O.route(dict(inp, b_select=np.zeros(8, np.float32)), desc)
    for key in ("topk_idx", "topk_w", "aux", "z_loss"):
        assert np.array_equal(a[key], b[key])


def test_dominant_selection_bias_picks_expert_with_unbiased_weights():
    """A bias of +50 on expert j makes j every token's first choice; the weights
    are still the softmax of the logits (renormalised over the chosen), and the
    aux loss has f_j = 1: aux = E * P_j."""
    E, j = 8, 5
    bs = np.zeros(E, np.float32)
    bs[j] = 50.0
    inp, desc = _tiny(T=20, E=E, k=2, seed=7, b_select=bs)
    r = O.route(inp, desc)
    p = r["probs"]
    assert np.all(r["topk_idx"][:, 0] == j)
    second = r["topk_idx"][:, 1]
    # the second choice is the best other expert by (unbiased) logit
    g = r["logits"].copy()
    g[:, j] = -np.inf
    assert np.array_equal(second, np.argmax(g, axis=1))
    tot = p[np.arange(20), j] + p[np.arange(20), second]
    assert np.allclose(r["topk_w"][:, 0], p[:, j] / tot, rtol=1e-15)
    assert abs(r["aux"] - E * p[:, j].mean()) <= 1e-13
    # probabilities themselves do not see the bias
    assert np.array_equal(p, O.route(dict(inp, b_select=None), desc)["probs"])
