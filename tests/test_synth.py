"""The seeded generator: rounding, reproducibility, stream independence and the
routing structure each named workload asks for (checked with the oracle)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from synth import workloads as W
from oracle import moe_oracle as O


def test_bf16_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -2.5, 3.0e38, 1e-40],
                    np.float32)
    bits = W.f32_to_bf16_bits(vals)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0
    assert back[1] == 1.0                 # tie -> even mantissa
    assert back[2] == one + 2 * ulp       # tie -> even mantissa (up)
    assert back[3] == 1.0
    assert back[4] == -2.5
    assert np.isfinite(back[5])
    rng = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    b = (W.f32_to_bf16_bits(rng).astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(b - rng) <= np.abs(rng) * 2.0 ** -8 + 1e-45)


def test_reproducible_and_streams_independent():
    s = W.Workload("t", 40, 64, 128, 4, 2, True, 0, True, "bf16")
    a = synth.make_inputs(s, params={})
    b = synth.make_inputs(s, params={})
    for key in ("x", "w_router", "w1", "b1", "w2", "b2"):
        assert np.array_equal(a[key], b[key])
    nb = synth.make_inputs(s.with_(expert_bias=False), params={})
    assert np.array_equal(a["w1"], nb["w1"]) and np.array_equal(a["w2"], nb["w2"])
    other = synth.make_inputs(s.with_(seed=1), params={})
    assert not np.array_equal(a["w1"], other["w1"])
    # a different token count leaves the expert bank alone (prefill/decode pairs share it)
    t = synth.make_inputs(s.with_(tokens=3), params={})
    assert np.array_equal(a["w1"], t["w1"]) and np.array_equal(a["x"][:3], t["x"])


def test_prefill_and_decode_share_the_expert_shape_and_seed():
    p, d = W.WORKLOADS["mixtral_prefill_bf16"], W.WORKLOADS["decode_bf16"]
    assert (p.n_experts, p.d_model, p.d_ff, p.seed, p.dtype) == (d.n_experts, d.d_model, d.d_ff, d.seed, d.dtype)


def test_capacity_formula():
    assert W.capacity_for(8192, 64) == 160
    assert W.WORKLOADS["switch_capacity_bf16"].capacity == 160
    assert W.capacity_for(777, 64) == 16       # ceil(971.25 / 64) = ceil(15.18)
    assert W.capacity_for(64, 8) == 10


def _route_named(name):
    spec = W.WORKLOADS[name]
    inp = synth.make_inputs(spec, with_experts=False)
    return spec, O.route(inp, O.desc_of(spec))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_named_workload_margins(name):
    spec, r = _route_named(name)
    assert r["margin"].min() > O.MARGIN_MIN


def test_mid_loads_near_uniform():
    spec, r = _route_named("mid_bf16")
    mean = spec.tokens * spec.top_k / spec.n_experts
    assert np.all(np.abs(r["counts"] - mean) <= 0.2 * mean)


def test_prefill_zipf_shares():
    spec, r = _route_named("mixtral_prefill_bf16")
    target = 1.0 / np.arange(1, 9)
    target /= target.sum()
    share = r["counts"] / r["counts"].sum()
    assert np.all(np.abs(share - target) <= 0.01)


def test_switch_hot_experts_and_drops():
    spec, r = _route_named("switch_capacity_bf16")
    hot = np.arange(0, 64, 8)
    frac = np.isin(r["topk_idx"][:, 0], hot).mean()
    assert abs(frac - 0.5) <= 0.005
    assert np.all(r["counts"][hot] == spec.capacity)
    assert r["keep"].sum() < spec.tokens


def test_decode_touches_every_expert():
    spec, r = _route_named("decode_bf16")
    assert np.all(r["counts"] >= 1)
