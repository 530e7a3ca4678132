"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on a page (fixtures under tests/golden/), a closed form, an
invariant, a special case that reduces to a textbook routine, or brute force.
"""
from __future__ import annotations

import json
import math
import os
import random

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from oracle import variants as V
from tests._inputs import SMALL, inputs_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _route_logits(logits, k, renormalize=True, capacity=0):
    """Route tokens whose router logits are given (x = logits, W_r = identity)."""
    g = np.asarray(logits, dtype=np.float64)
    T, E = g.shape
    inputs = {"x": g, "w_router": np.eye(E), "b_router": None}
    desc = {"tokens": T, "d_model": E, "d_ff": 1, "n_experts": E, "top_k": k,
            "renormalize": renormalize, "capacity": capacity}
    return O.route(inputs, desc)


# --------------------------------------------------------------------------
# Router: worked examples from the pages
# --------------------------------------------------------------------------
def test_eight_expert_example_top2():
    """Eight-expert router example: top-2 goes to the second and fourth experts;
    renormalised weights 0.51/0.82 and 0.31/0.82."""
    gd = _golden("router_eight_experts.json")
    p = np.array(gd["probs"])
    r = _route_logits(np.log(p)[None, :], gd["top_k"])
    assert r["topk_idx"][0].tolist() == gd["expected_idx"]
    assert [i + 1 for i in r["topk_idx"][0]] == gd["expected_experts_one_based"]
    want = [a / b for a, b in gd["expected_weights_fraction"]]
    np.testing.assert_allclose(r["topk_w"][0], want, rtol=0, atol=1e-12)
    # softmax of ln p recovers p (the probabilities sum to 1 on the page)
    np.testing.assert_allclose(r["probs"][0], p / p.sum(), rtol=1e-13)


def test_three_score_example():
    gd = _golden("router_three_scores.json")
    p = np.array(gd["probs"])
    r1 = _route_logits(np.log(p)[None, :], 1)
    assert r1["topk_idx"][0].tolist() == gd["top1_idx"]
    np.testing.assert_allclose(r1["topk_w"][0], [1.0], atol=1e-15)
    r2 = _route_logits(np.log(p)[None, :], 2)
    assert r2["topk_idx"][0].tolist() == gd["top2_idx"]
    np.testing.assert_allclose(r2["topk_w"][0], [a / b for a, b in gd["top2_weights_fraction"]],
                               atol=1e-12)
    # without renormalisation the raw probabilities come back
    r3 = _route_logits(np.log(p)[None, :], 2, renormalize=False)
    np.testing.assert_allclose(r3["topk_w"][0], [0.75, 0.15], atol=1e-12)


def test_topk_on_gaussian_scores_by_definition():
    """Seeded Gaussian scores for 8 experts (the shape of the aiinbed page's router
    demo): every chosen expert's probability is at least every unchosen one's, the
    choices come in descending order, and the renormalised weights are the chosen
    probabilities scaled to sum to 1."""
    rng = random.Random(7)
    scores = np.array([[rng.gauss(0, 1) for _ in range(8)] for _ in range(64)])
    r = _route_logits(scores, 2)
    p = O.softmax(scores)
    for t in range(scores.shape[0]):
        c = r["topk_idx"][t]
        rest = np.setdiff1d(np.arange(8), c)
        assert p[t, c[0]] >= p[t, c[1]] >= p[t, rest].max()
        np.testing.assert_allclose(r["topk_w"][t], p[t, c] / p[t, c].sum(), rtol=1e-12)
        np.testing.assert_allclose(r["topk_w"][t].sum(), 1.0, rtol=1e-15)


def test_exact_ties_go_to_lower_index():
    g = np.array([[1.0, 3.0, 3.0, 0.0, 3.0],
                  [2.0, 2.0, 2.0, 2.0, 2.0],
                  [0.0, 1.0, 0.5, 1.0, 0.5]])
    r = _route_logits(g, 3)
    assert r["topk_idx"].tolist() == [[1, 2, 4], [0, 1, 2], [1, 3, 2]]
    # the brute force (rank counting) agrees
    inputs = {"x": g, "w_router": np.eye(5), "b_router": None,
              "w1": np.zeros((5, 1, 5)), "w2": np.zeros((5, 5, 1)), "b1": None, "b2": None}
    desc = {"tokens": 3, "d_model": 5, "d_ff": 1, "n_experts": 5, "top_k": 3,
            "renormalize": True, "capacity": 0}
    rank = V.dense_masked(inputs, desc)["rank"]
    for t in range(3):
        assert np.argsort(rank[t], kind="stable")[:3].tolist() == r["topk_idx"][t].tolist()


def test_softmax_matches_library_and_sums_to_one():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((200, 16)) * 5
    p = O.softmax(g)
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(g), dim=-1).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-15)


def test_renormalised_weights_sum_to_one():
    spec, inp = inputs_for("mid_small_bf16")
    r = O.route(inp, O.desc_of(spec))
    np.testing.assert_allclose(r["topk_w"].sum(axis=1), 1.0, atol=4 * 2 * np.finfo(float).eps)
    # slot 0 carries the larger weight (rank order)
    assert np.all(r["topk_w"][:, 0] >= r["topk_w"][:, 1])


# --------------------------------------------------------------------------
# Aux loss: closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("E", [2, 8, 64])
def test_aux_uniform_routing_is_one(E):
    r = _route_logits(10.0 * np.eye(E), 1)
    np.testing.assert_allclose(r["f"], 1.0 / E, rtol=0, atol=0)
    np.testing.assert_allclose(r["P"], 1.0 / E, rtol=1e-14)
    assert abs(r["aux"] - 1.0) < 1e-13


def test_aux_uniform_probabilities_is_one():
    # all logits equal: every token picks expert 0 (tie rule), P is uniform
    r = _route_logits(np.zeros((37, 8)), 2)
    assert np.all(r["topk_idx"][:, 0] == 0)
    assert abs(r["aux"] - 1.0) < 1e-14


def test_aux_uniform_fractions_is_one():
    rng = np.random.default_rng(11)
    E = 6
    g = rng.standard_normal((E * 20, E))
    g[np.arange(E * 20), np.arange(E * 20) % E] += 50.0        # token t picks t % E
    r = _route_logits(g, 1)
    np.testing.assert_allclose(r["f"], 1.0 / E)
    assert abs(r["aux"] - 1.0) < 1e-13


@pytest.mark.parametrize("E", [4, 8, 64])
def test_aux_collapse_is_E(E):
    g = np.zeros((50, E))
    g[:, 0] = 50.0
    r = _route_logits(g, 1)
    assert abs(r["aux"] - E) < 1e-12 * E


def test_aux_load_skew_table():
    """The 8,000-token skew table: with P_i = f_i the loss is 8 * sum f_i^2 = 2.995."""
    gd = _golden("load_skew_table.json")
    counts = gd["counts"]
    assert sum(counts) == gd["tokens"] and gd["tokens"] / 8 == gd["balanced_per_expert"]
    top1 = np.repeat(np.arange(8), counts)
    p = np.eye(8)[top1]                       # probabilities one-hot on the choice: P = f
    aux, f, P, cnt = O.aux_loss(top1[:, None], p, 8)
    assert cnt.tolist() == counts
    np.testing.assert_allclose(f, np.array(counts) / 8000, atol=0)
    assert abs(aux - gd["aux_with_P_equal_f"]) < 1e-12


def test_aux_counts_top1_before_capacity():
    # 6 tokens all choosing expert 1 with capacity 2: f still counts all 6
    g = np.zeros((6, 3))
    g[:, 1] = 20.0
    r = _route_logits(g, 1, capacity=2)
    assert r["top1_count"].tolist() == [0, 6, 0]
    assert r["keep"][:, 0].tolist() == [True, True, False, False, False, False]


# --------------------------------------------------------------------------
# Expert FFN and GELU
# --------------------------------------------------------------------------
def test_gelu_against_math_erf_and_identities():
    z = np.linspace(-8, 8, 4001)
    ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z])
    np.testing.assert_allclose(O.gelu_erf(z), ref, rtol=1e-15, atol=1e-15)  # 1+erf cancels for z << 0
    assert O.gelu_erf(np.array([0.0]))[0] == 0.0
    # GELU(-z) = GELU(z) - z   (Phi(-z) = 1 - Phi(z))
    np.testing.assert_allclose(O.gelu_erf(-z), O.gelu_erf(z) - z, atol=1e-14)
    # GELU(1) = Phi(1), the standard normal CDF at 1
    assert abs(O.gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    # not the tanh approximation: they differ by ~1e-4 near |z| = 2
    tanh_form = 0.5 * 2.0 * (1 + math.tanh(math.sqrt(2 / math.pi) * (2.0 + 0.044715 * 8.0)))
    assert abs(O.gelu_erf(np.array([2.0]))[0] - tanh_form) > 1e-5


def test_gelu_matches_torch_exact_gelu():
    z = np.random.default_rng(5).standard_normal(10000) * 4
    np.testing.assert_allclose(O.gelu_erf(z), F.gelu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-15)


def test_single_expert_reduces_to_dense_mlp():
    """E = 1, k = 1 with renormalisation: y = W2 GELU(W1 x + b1) + b2, the dense MLP."""
    spec, inp = inputs_for("dense_mlp_fp32")
    r = O.forward(inp, O.desc_of(spec))
    x = torch.from_numpy(inp["x"].astype(np.float64))
    h = F.gelu(F.linear(x, torch.from_numpy(inp["w1"][0].astype(np.float64)),
                        torch.from_numpy(inp["b1"][0].astype(np.float64))))
    y = F.linear(h, torch.from_numpy(inp["w2"][0].astype(np.float64)),
                 torch.from_numpy(inp["b2"][0].astype(np.float64))).numpy()
    np.testing.assert_allclose(r["y"], y, rtol=1e-12, atol=1e-13)
    assert abs(r["aux"] - 1.0) < 1e-15


# --------------------------------------------------------------------------
# Capacity and dispatch layout
# --------------------------------------------------------------------------
def test_capacity_hand_case():
    top1 = [0, 0, 1, 0, 0, 1, 0, 1, 1, 1]
    idx = np.array(top1)[:, None]
    keep = O.capacity_keep(idx, 2, 3)
    assert keep[:, 0].tolist() == [True, True, True, True, False, True, False, True, False, False]
    counts, offsets, dest, src = O.dispatch_layout(idx, keep, 2)
    assert counts.tolist() == [3, 3] and offsets.tolist() == [0, 3, 6]
    assert dest[:, 0].tolist() == [0, 1, 3, 2, -1, 4, -1, 5, -1, -1]
    assert src.tolist() == [0, 1, 3, 2, 5, 7]


def test_capacity_invariants_on_switch_shape():
    spec, inp = inputs_for("switch_small_bf16")
    r = O.route(inp, O.desc_of(spec))
    C = spec.capacity
    demand = np.bincount(r["topk_idx"][:, 0], minlength=spec.n_experts)
    assert r["counts"].tolist() == np.minimum(demand, C).tolist()
    assert demand.max() > C                        # the shape does drop tokens
    for e in range(spec.n_experts):                 # kept tokens are the lowest indices
        toks = np.flatnonzero(r["topk_idx"][:, 0] == e)
        assert r["keep"][toks, 0].tolist() == [i < C for i in range(toks.size)]


def test_dispatch_layout_invariants():
    spec, inp = inputs_for("mid_small_bf16")
    r = O.route(inp, O.desc_of(spec))
    k = spec.top_k
    R = int(r["offsets"][-1])
    assert R == spec.tokens * k and r["counts"].sum() == R
    assert sorted(r["src"].tolist()) == list(range(R))          # a permutation of assignments
    for row, a in enumerate(r["src"]):
        assert r["dest"][a // k, a % k] == row
    for e in range(spec.n_experts):
        seg = r["src"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(r["topk_idx"][seg // k, seg % k] == e)
        assert np.all(np.diff(seg // k) > 0)                    # token order, no repeats


# --------------------------------------------------------------------------
# Whole layer against independent formulations
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["toy_fp32", "mid_small_bf16", "switch_small_bf16",
                                  "top1_norenorm_fp32", "topk_eq_e_bf16", "capacity_one_bf16",
                                  "decode_small_bf16"])
def test_oracle_equals_dense_masked(name):
    spec, inp = inputs_for(name)
    desc = O.desc_of(spec)
    r = O.forward(inp, desc)
    b = V.dense_masked(inp, desc)
    rms = np.sqrt(np.mean(b["y"] ** 2))
    assert np.max(np.abs(r["y"] - b["y"])) <= 1e-12 * max(rms, 1e-300)
    assert abs(r["aux"] - b["aux"]) <= 1e-13 * abs(b["aux"])
    # the dense mask marks exactly the oracle's kept choices
    m = np.zeros((spec.tokens, spec.n_experts), bool)
    for s in range(spec.top_k):
        m[np.arange(spec.tokens)[r["keep"][:, s]], r["topk_idx"][r["keep"][:, s], s]] = True
    assert np.array_equal(m, b["mask"])


@pytest.mark.parametrize("k,renorm,cap", [(2, True, 0), (1, False, 2), (3, True, 0), (1, True, 1)])
def test_oracle_equals_scalar_loops(k, renorm, cap):
    from synth import workloads as W
    from tests._inputs import repair
    spec = W.Workload("tiny", 7, 6, 9, 5, k, renorm, cap, True, "f32", router_bias=True, seed=k)
    rb = np.array([0.3, -0.2, 0.0, 0.1, -0.4], np.float32)
    import synth
    inp = synth.make_inputs(spec, redraw=repair(spec, rb), router_bias=rb, params={})
    desc = O.desc_of(spec)
    r = O.forward(inp, desc)
    lp = V.loops(inp, desc)
    np.testing.assert_allclose(r["y"], lp["y"], rtol=1e-12, atol=1e-14)
    assert abs(r["aux"] - lp["aux"]) < 1e-13
    assert r["topk_idx"][:, 0].tolist() == lp["top1"]


def _layer_by_definition(inp, E, k):
    """The layer written straight from its definition, token by token, in torch fp64:
    p = softmax(W_r x); the k largest p (torch.topk); weights p_i / sum of the chosen
    p; y = sum over the chosen experts of w_i (W2_i GELU(W1_i x + b1_i) + b2_i) with
    the exact erf GELU; aux = E * sum_i f_i P_i with f_i the share of tokens whose
    first choice is i and P_i the mean of p_i."""
    t = lambda a: torch.from_numpy(O.widen(a))
    x, wr = t(inp["x"]), t(inp["w_router"])
    w1, w2, b1, b2 = t(inp["w1"]), t(inp["w2"]), t(inp["b1"]), t(inp["b2"])
    T = x.shape[0]
    p = torch.softmax(x @ wr.T, dim=-1)
    y = torch.zeros_like(x)
    chosen = []
    for tok in range(T):
        pv, idx = torch.topk(p[tok], k)
        chosen.append(idx.tolist())
        for wgt, e in zip((pv / pv.sum()).tolist(), idx.tolist()):
            y[tok] += wgt * (w2[e] @ F.gelu(w1[e] @ x[tok] + b1[e]) + b2[e])
    f = torch.bincount(torch.tensor([c[0] for c in chosen]), minlength=E).double() / T
    aux = E * torch.dot(f, p.mean(0))
    return y, aux, np.array(chosen)


def test_oracle_matches_the_definition_token_by_token():
    spec, inp = inputs_for("toy_fp32")
    desc = O.desc_of(spec)
    r = O.forward(inp, desc)
    y, aux, chosen = _layer_by_definition(inp, spec.n_experts, spec.top_k)
    assert np.array_equal(chosen, r["topk_idx"])
    np.testing.assert_allclose(r["y"], y.numpy(), rtol=1e-12, atol=1e-13)
    assert abs(r["aux"] - aux.item()) < 1e-12


def test_sampled_tokens_equal_full_forward():
    spec, inp = inputs_for("switch_small_bf16")
    desc = O.desc_of(spec)
    full = O.forward(inp, desc)
    toks = [776, 0, 5, 400, 123]
    part = O.forward(inp, desc, tokens=toks)
    np.testing.assert_allclose(part["y"], full["y"][toks], rtol=1e-12, atol=1e-15)  # BLAS blocking only


def test_expert_outputs_layout_matches_forward():
    spec, inp = inputs_for("mid_small_bf16")
    desc = O.desc_of(spec)
    eo = O.expert_outputs(inp, desc)
    r = eo["route"]
    y = np.zeros((spec.tokens, spec.d_model))
    for t in range(spec.tokens):
        for s in range(spec.top_k):
            y[t] += r["topk_w"][t, s] * eo["o"][r["dest"][t, s]]
    np.testing.assert_allclose(y, O.forward(inp, desc)["y"], rtol=1e-13, atol=1e-15)


def test_active_flops_are_k_over_E_of_dense_bank():
    """Eight experts with top-2 run about 2x the FFN compute of one dense FFN while
    holding 8x its parameters: active FFN flops are exactly k/E of running every
    expert on every token."""
    spec, inp = inputs_for("toy_fp32")
    r = O.route(inp, O.desc_of(spec))
    per_row = 4 * spec.d_model * spec.d_ff            # two matrix products per row
    active = per_row * int(r["offsets"][-1])
    dense_bank = per_row * spec.tokens * spec.n_experts
    assert active * spec.n_experts == dense_bank * spec.top_k
