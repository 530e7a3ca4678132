"""Pins of the shared expert and of fine-grained routing in the oracle (web page
"Mixture of Experts: Scaling Parameters Without Scaling Compute", section
"Design variations": fine-grained experts with larger k; shared experts that are
always active).

Readings pinned here: the shared expert runs on every token (dropped ones
included) and is added after the routed sum with weight 1; several shared
experts are one shared FFN whose hidden layer is theirs side by side."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import variants as V


def _erf_gelu(z):
    return 0.5 * z * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0)))


def _ffn(x, w1, b1, w2, b2):
    """Textbook FFN on float64 arrays (independent of the oracle)."""
    return _erf_gelu(x @ w1.T + b1) @ w2.T + b2


def _tiny(T=7, d=6, F=4, Fs=5, E=4, k=2, capacity=0, seed=11):
    rng = np.random.default_rng(seed)
    f32 = lambda a: np.asarray(a, np.float32)
    inp = {"x": f32(rng.standard_normal((T, d))), "w_router": f32(rng.standard_normal((E, d))),
           "b_router": None, "b_select": None,
           "w1": f32(rng.standard_normal((E, F, d))), "b1": f32(rng.uniform(-.1, .1, (E, F))),
           "w2": f32(rng.standard_normal((E, d, F))), "b2": f32(rng.uniform(-.1, .1, (E, d))),
           "w1_shared": f32(rng.standard_normal((Fs, d))), "b1_shared": f32(rng.uniform(-.1, .1, Fs)),
           "w2_shared": f32(rng.standard_normal((d, Fs))), "b2_shared": f32(rng.uniform(-.1, .1, d))}
    desc = {"tokens": T, "d_model": d, "d_ff": F, "n_experts": E, "top_k": k,
            "renormalize": True, "capacity": capacity}
    return inp, desc


def _no_shared(inp):
    return dict(inp, w1_shared=None, b1_shared=None, w2_shared=None, b2_shared=None)


def test_zero_shared_expert_changes_nothing():
    inp, desc = _tiny()
    z = {k: np.zeros_like(inp[k]) for k in ("w1_shared", "b1_shared", "w2_shared", "b2_shared")}
    a = O.forward(dict(inp, **z), desc, check_margin=False)["y"]
    b = O.forward(_no_shared(inp), desc, check_margin=False)["y"]
    assert np.array_equal(a, b)


def test_shared_expert_is_added_with_weight_one():
    inp, desc = _tiny()
    x = inp["x"].astype(np.float64)
    want = O.forward(_no_shared(inp), desc, check_margin=False)["y"] + _ffn(
        x, *(inp[k].astype(np.float64) for k in ("w1_shared", "b1_shared", "w2_shared", "b2_shared")))
    got = O.forward(inp, desc, check_margin=False)["y"]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_two_shared_experts_equal_one_of_their_joint_width():
    """FFN_a(x) + FFN_b(x) == the FFN with W1 = [W1a; W1b], b1 = [b1a; b1b],
    W2 = [W2a | W2b], b2 = b2a + b2b."""
    inp, desc = _tiny(Fs=3)
    rng = np.random.default_rng(5)
    d = desc["d_model"]
    a = [rng.standard_normal((3, d)), rng.uniform(-.1, .1, 3), rng.standard_normal((d, 3)), rng.uniform(-.1, .1, d)]
    b = [rng.standard_normal((2, d)), rng.uniform(-.1, .1, 2), rng.standard_normal((d, 2)), rng.uniform(-.1, .1, d)]
    a = [v.astype(np.float32) for v in a]
    b = [v.astype(np.float32) for v in b]
    joint = {"w1_shared": np.concatenate([a[0], b[0]]), "b1_shared": np.concatenate([a[1], b[1]]),
             "w2_shared": np.concatenate([a[2], b[2]], axis=1),
             "b2_shared": (a[3].astype(np.float64) + b[3].astype(np.float64))}
    got = O.forward(dict(inp, **joint), desc, check_margin=False)["y"]
    x = inp["x"].astype(np.float64)
    want = O.forward(_no_shared(inp), desc, check_margin=False)["y"] + \
        _ffn(x, *(v.astype(np.float64) for v in a)) + _ffn(x, *(v.astype(np.float64) for v in b))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_dropped_token_keeps_the_shared_expert():
    """Top-1 with capacity 1: every token after the first on an expert is dropped
    and its output is exactly the shared expert's."""
    inp, desc = _tiny(T=9, E=2, k=1, capacity=1)
    r = O.forward(inp, desc, check_margin=False)
    dropped = np.flatnonzero(~r["keep"][:, 0])
    assert dropped.size > 0
    x = inp["x"].astype(np.float64)[dropped]
    sh = _ffn(x, *(inp[k].astype(np.float64) for k in ("w1_shared", "b1_shared", "w2_shared", "b2_shared")))
    assert np.allclose(r["y"][dropped], sh, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("E,k,seed", [(4, 2, 0), (16, 8, 1), (32, 6, 2)])
def test_shared_and_fine_grained_agree_with_both_variants(E, k, seed):
    inp, desc = _tiny(T=6, d=5, F=3, Fs=4, E=E, k=k, seed=seed)
    r = O.forward(inp, desc, check_margin=False)
    dm = V.dense_masked(inp, desc)
    lp = V.loops(inp, desc)
    assert np.allclose(r["y"], dm["y"], rtol=1e-12, atol=1e-12)
    assert np.allclose(r["y"], lp["y"], rtol=1e-12, atol=1e-12)
    assert abs(r["aux"] - lp["aux"]) <= 1e-12
