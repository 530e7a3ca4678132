"""Pins of expert capacity for any k and of the reroute policy in the oracle (web
page "Mixture-of-Experts — making a model wider without using all of it for
every token", section "Experts also have capacity limits": overflow may be
dropped or routed elsewhere; "Mixture of Experts: Scaling Parameters Without
Scaling Compute", section "The central problem: load balancing").

Readings pinned: drop keeps, per expert, the C lowest-index tokens that chose
it in any slot; reroute serves overflow in rounds at each token's next-best
unused expert, requests accepted per expert in token order, and weights a
served slot with the serving expert's probability over the original
denominator."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import variants as V


def _from_logits(logits, k, C, policy="drop", renorm=True, F=3, seed=0):
    """Inputs whose router logits are exactly `logits` (x = logits, W_r = I)."""
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    rng = np.random.default_rng(seed)
    inp = {"x": logits, "w_router": np.eye(E, dtype=np.float32), "b_router": None, "b_select": None,
           "w1": rng.standard_normal((E, F, E)).astype(np.float32), "b1": None,
           "w2": rng.standard_normal((E, E, F)).astype(np.float32), "b2": None}
    desc = {"tokens": T, "d_model": E, "d_ff": F, "n_experts": E, "top_k": k,
            "renormalize": renorm, "capacity": C, "capacity_policy": policy}
    return inp, desc


def test_drop_with_top2_hand_case():
    # choices (rank order): t0 [0,1] t1 [0,2] t2 [1,0] t3 [0,1] t4 [2,1];  C = 2
    L = [[3, 2, 0], [3, 0, 2], [2, 3, 0], [3, 2, 0], [0, 2, 3]]
    inp, desc = _from_logits(L, k=2, C=2)
    r = O.route(inp, desc)
    assert r["topk_idx"].tolist() == [[0, 1], [0, 2], [1, 0], [0, 1], [2, 1]]
    # expert 0: tokens 0, 1, 2, 3 chose it -> keep 0, 1;  expert 1: 0, 2, 3, 4 -> keep 0, 2;
    # expert 2: tokens 1, 4 -> both
    assert r["keep"].tolist() == [[True, True], [True, True], [True, False], [False, False],
                                  [True, False]]
    assert r["counts"].tolist() == [2, 2, 2]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_drop_invariants_any_k(seed):
    rng = np.random.default_rng(seed)
    T, E, k, C = 40, 6, 3, 9
    inp, desc = _from_logits(rng.standard_normal((T, E)), k=k, C=C)
    r = O.route(inp, desc, )
    idx, keep = r["topk_idx"], r["keep"]
    for e in range(E):
        toks = [t for t in range(T) if e in idx[t]]
        kept = [t for t in range(T) for s in range(k) if idx[t, s] == e and keep[t, s]]
        assert kept == toks[:C]
        assert r["counts"][e] == min(len(toks), C)


def test_reroute_top1_hand_case():
    """E = 3, C = 2, everyone prefers expert 0.
    round 0: tokens 0, 1 -> expert 0 (full); 2, 3, 4 rejected.
    round 1: 2 -> 1, 3 -> 2, 4 -> 1 (second choices); all fit.
    """
    L = [[5, 1, 0], [5, 0, 1], [5, 2, 1], [5, 1, 2], [5, 3, 2]]
    inp, desc = _from_logits(L, k=1, C=2, policy="reroute")
    r = O.route(inp, desc)
    assert r["topk_idx"][:, 0].tolist() == [0, 0, 1, 2, 1]
    assert r["keep"].all() and r["reroute_rounds"] == 2
    p = r["probs"]
    for t, e in enumerate([0, 0, 1, 2, 1]):          # k = 1, renorm: denominator p[t, 0]
        assert abs(r["topk_w"][t, 0] - p[t, e] / p[t, 0]) <= 1e-15
    assert r["router_idx"][:, 0].tolist() == [0] * 5 and r["top1_count"].tolist() == [5, 0, 0]


def test_reroute_chain_and_drop():
    """E = 2, C = 1, three tokens all preferring expert 0: token 0 -> 0, token 1
    rerouted to 1, token 2 finds both full and is dropped."""
    L = [[2, 1], [2, 1], [2, 1]]
    inp, desc = _from_logits(L, k=1, C=1, policy="reroute")
    r = O.route(inp, desc)
    assert r["keep"][:, 0].tolist() == [True, True, False]
    assert r["topk_idx"][:2, 0].tolist() == [0, 1]
    y = O.forward(inp, desc, check_margin=False)["y"]
    assert np.all(y[2] == 0.0)


def test_reroute_top2_slots_take_ranks_in_slot_order():
    """k = 2, C = 1, E = 4.  Token 0 takes experts 0 and 1.  Token 1 also chose 0
    and 1: both slots overflow; slot 0 asks for rank 2 (expert 2), slot 1 for
    rank 3 (expert 3)."""
    L = [[4, 3, 2, 1], [4, 3, 2, 1]]
    inp, desc = _from_logits(L, k=2, C=1, policy="reroute")
    r = O.route(inp, desc)
    assert r["topk_idx"].tolist() == [[0, 1], [2, 3]]
    assert r["keep"].all()


def test_reroute_with_room_everywhere_is_uncapped():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((30, 5))
    a = O.route(*_from_logits(L, k=2, C=60, policy="reroute"))
    b = O.route(*_from_logits(L, k=2, C=0))
    assert np.array_equal(a["topk_idx"], b["topk_idx"]) and a["keep"].all()
    assert np.allclose(a["topk_w"], b["topk_w"], rtol=1e-15)


@pytest.mark.parametrize("seed,k,C", [(0, 1, 3), (1, 2, 4), (2, 3, 5), (3, 2, 7)])
def test_reroute_invariants(seed, k, C):
    rng = np.random.default_rng(seed)
    T, E = 25, 6
    inp, desc = _from_logits(rng.standard_normal((T, E)), k=k, C=C, policy="reroute")
    r = O.route(inp, desc)
    idx, keep, ridx = r["topk_idx"], r["keep"], r["router_idx"]
    load = np.zeros(E, int)
    for t in range(T):
        served = [int(idx[t, s]) for s in range(k) if keep[t, s]]
        assert len(set(served)) == len(served)                  # distinct experts per token
        for s in range(k):
            if keep[t, s]:
                load[idx[t, s]] += 1
                if idx[t, s] != ridx[t, s]:                      # rerouted: a non-chosen expert
                    assert idx[t, s] not in ridx[t]
    assert np.all(load <= C) and np.array_equal(load, r["counts"])
    if C * E >= T * k:                                           # room for everyone
        assert keep.all()
    # weights: serving expert's probability over the original denominator
    p = r["probs"]
    den = np.take_along_axis(p, ridx, axis=1).sum(axis=1)
    for t in range(T):
        for s in range(k):
            if keep[t, s]:
                assert abs(r["topk_w"][t, s] - p[t, idx[t, s]] / den[t]) <= 1e-15


@pytest.mark.parametrize("policy,k", [("drop", 2), ("drop", 3), ("reroute", 1), ("reroute", 2)])
def test_capacity_policies_agree_with_loops(policy, k):
    rng = np.random.default_rng(9 + k)
    T, E = 12, 5
    inp, desc = _from_logits(rng.standard_normal((T, E)), k=k, C=3, policy=policy)
    inp["b1"] = rng.uniform(-.1, .1, (E, 3)).astype(np.float32)
    inp["b2"] = rng.uniform(-.1, .1, (E, E)).astype(np.float32)
    r = O.forward(inp, desc, check_margin=False)
    lp = V.loops(inp, desc)
    assert np.allclose(r["y"], lp["y"], rtol=1e-12, atol=1e-12)
    if policy == "drop":
        dm = V.dense_masked(inp, desc)
        assert np.allclose(r["y"], dm["y"], rtol=1e-12, atol=1e-12)
