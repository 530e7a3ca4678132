"""Test inputs: the named workloads plus small shapes, all margin-repaired.

Named workloads read their stored router bias and redrawn rows from
``synth/input_params.json``.  Small test shapes are repaired here with the
oracle's routing (the same rule: every top-k logit margin > 1e-3), so the GPU's
fp32 router cannot legitimately choose differently from the fp64 oracle.
"""
from __future__ import annotations

import functools

import numpy as np

import synth
from synth import workloads as W
from oracle import moe_oracle as O

Workload = W.Workload

# Small shapes that still span several tiles and end in a ragged tail.
SMALL = {
    "mid_small_bf16": Workload("mid_small_bf16", 300, 256, 512, 16, 2, True, 0, True, "bf16"),
    "prefill_small_bf16": Workload("prefill_small_bf16", 1000, 512, 1024, 8, 2, True, 0, False,
                                   "bf16", router_bias=True),
    "switch_small_bf16": Workload("switch_small_bf16", 777, 256, 512, 64, 1, False,
                                  W.capacity_for(777, 64), True, "bf16", router_bias=True),
    "decode_small_bf16": Workload("decode_small_bf16", 5, 512, 1024, 8, 2, True, 0, True, "bf16"),
    "top1_norenorm_fp32": Workload("top1_norenorm_fp32", 50, 128, 256, 4, 1, False, 0, True, "f32"),
    "dense_mlp_fp32": Workload("dense_mlp_fp32", 33, 128, 384, 1, 1, True, 0, True, "f32"),
    "topk_eq_e_bf16": Workload("topk_eq_e_bf16", 70, 256, 256, 4, 4, True, 0, True, "bf16"),
    "single_token_bf16": Workload("single_token_bf16", 1, 256, 512, 8, 2, True, 0, True, "bf16"),
    "capacity_one_bf16": Workload("capacity_one_bf16", 64, 128, 256, 8, 1, True, 1, True, "bf16"),
    # selection-only per-expert bias (and the z-loss, computed for every shape)
    "select_bias_bf16": Workload("select_bias_bf16", 300, 256, 512, 16, 4, True, 0, True, "bf16",
                                 selection_bias=True),
    "select_bias_top1_fp32": Workload("select_bias_top1_fp32", 90, 128, 256, 8, 1, False, 0, True,
                                      "f32", selection_bias=True),
    # fine-grained routing (32 experts, top-6) plus a shared expert
    "shared_fine_bf16": Workload("shared_fine_bf16", 500, 256, 256, 32, 6, True, 0, True, "bf16",
                                 d_ff_shared=512),
    # top-1 with capacity: dropped tokens still get the shared expert
    "shared_capacity_bf16": Workload("shared_capacity_bf16", 300, 256, 512, 16, 1, True,
                                     W.capacity_for(300, 16), True, "bf16", router_bias=True,
                                     d_ff_shared=256),
    "shared_fp32": Workload("shared_fp32", 60, 128, 256, 8, 2, True, 0, True, "f32", d_ff_shared=384),
    # widths that are odd multiples of 128 (the tiled kernel's last n-tile is half padding)
    "odd_width_bf16": Workload("odd_width_bf16", 700, 384, 640, 8, 2, True, 0, True, "bf16"),
    "odd_fine_shared_bf16": Workload("odd_fine_shared_bf16", 1200, 256, 384, 16, 6, True, 0, True,
                                     "bf16", d_ff_shared=384),
    # capacity with top-2 (drop), and the reroute policy (top-1 and top-2, bf16 and fp32)
    "capacity_top2_bf16": Workload("capacity_top2_bf16", 400, 256, 512, 16, 2, True, 40, True,
                                   "bf16", router_bias=True),
    "reroute_top1_bf16": Workload("reroute_top1_bf16", 500, 256, 512, 16, 1, False,
                                  W.capacity_for(500, 16), True, "bf16", router_bias=True,
                                  capacity_policy="reroute"),
    "reroute_top2_fp32": Workload("reroute_top2_fp32", 200, 128, 256, 8, 2, True, 40, True, "f32",
                                  router_bias=True, capacity_policy="reroute"),
    # rerouting that fills experts past one 128-row tile (tiled path, split h)
    "reroute_c160_bf16": Workload("reroute_c160_bf16", 1400, 256, 384, 10, 1, False, 160, True,
                                  "bf16", router_bias=True, capacity_policy="reroute"),
    # small batches on the weight-streaming path: bf16 with biases, with a shared
    # expert, with a capacity no expert can reach (drop and reroute), ragged widths
    "batch32_bf16": Workload("batch32_bf16", 32, 512, 1024, 8, 2, True, 0, True, "bf16"),
    "batch48_shared_bf16": Workload("batch48_shared_bf16", 48, 256, 384, 8, 2, True, 0, True,
                                    "bf16", d_ff_shared=256),
    "batch24_cap_bf16": Workload("batch24_cap_bf16", 24, 256, 512, 4, 2, True, 30, True, "bf16"),
    "batch40_reroute_bf16": Workload("batch40_reroute_bf16", 40, 256, 512, 8, 2, True, 40, True,
                                     "bf16", capacity_policy="reroute"),
    "batch64_top1_bf16": Workload("batch64_top1_bf16", 64, 384, 640, 16, 1, False, 0, False,
                                  "bf16"),
    # the small-batch router (64 tokens at most) with many experts and slots, a router
    # bias and a selection bias: 64 experts top-6 (bf16), 24 experts top-3 (fp32)
    "batch20_fine_bias_bf16": Workload("batch20_fine_bias_bf16", 20, 256, 256, 64, 6, True, 0,
                                       True, "bf16", router_bias=True, selection_bias=True),
    "batch57_e24_k3_fp32": Workload("batch57_e24_k3_fp32", 57, 128, 256, 24, 3, True, 0, True,
                                    "f32", selection_bias=True),
    # every token's first choice is one expert (a logit bias of +6 on it): that expert's
    # segment holds all T rows -- the longest run of m-tiles the tile schedule sees --
    # on the stream path (fp32), the 128-row tiled path (top-1) and the 256-row tiled
    # path (top-2, 275 rows per expert on average)
    "one_expert_fp32": Workload("one_expert_fp32", 300, 128, 256, 4, 1, True, 0, True, "f32",
                                router_bias=True),
    "one_expert_top1_bf16": Workload("one_expert_top1_bf16", 700, 256, 512, 8, 1, True, 0, True,
                                     "bf16", router_bias=True),
    "one_expert_top2_bf16": Workload("one_expert_top2_bf16", 1100, 256, 384, 8, 2, True, 0, False,
                                     "bf16", router_bias=True),
    # k ranges of 4096 (d_model for the first product, d_ff for the second): the
    # tiled kernel's last round is split along k and finished by its reduction, for
    # bf16 h (top-2, 256-row tiles) and split h (top-1 without renormalisation,
    # 128-row tiles), first and second product
    "long_d_bf16": Workload("long_d_bf16", 512, 4096, 512, 4, 2, True, 0, True, "bf16"),
    "long_f_bf16": Workload("long_f_bf16", 512, 256, 4096, 4, 2, True, 0, True, "bf16"),
    "long_d_top1_bf16": Workload("long_d_top1_bf16", 600, 4096, 512, 8, 1, False, 0, True,
                                 "bf16"),
    "long_f_top1_bf16": Workload("long_f_top1_bf16", 600, 512, 4096, 8, 1, False, 0, True,
                                 "bf16"),
    # few column blocks and d_model = 4096 on the weight-streaming path: the first
    # product's k range is split over blocks and reduced (top-2 of 2 experts: both hold
    # all 24 rows, two 16-row tiles; top-1 of 4: mostly one tile)
    "split_k_bf16": Workload("split_k_bf16", 24, 4096, 256, 2, 2, True, 0, True, "bf16"),
    "split_k_top1_bf16": Workload("split_k_top1_bf16", 20, 4096, 256, 4, 1, False, 0, True,
                                  "bf16"),
    # the mid-size layer's shapes (4096 tokens, 16 experts) with a selection bias
    "mid_select_bias_bf16": Workload("mid_select_bias_bf16", 4096, 1024, 4096, 16, 2, True, 0, True,
                                     "bf16", selection_bias=True),
}


ONE_EXPERT_HOT = 5     # the expert every token of the one_expert_* shapes picks first


def small_router_bias(spec):
    """A fixed skew for the small skewed shapes (no calibration needed)."""
    E = spec.n_experts
    if spec.name.startswith("one_expert"):
        b = np.zeros(E, np.float32)
        b[ONE_EXPERT_HOT % E] = 6.0
        return b
    if spec.top_k == 1:                     # hot experts: every 8th
        b = np.zeros(E, np.float32)
        b[::8] = 1.0
        return b
    return (-np.log(np.arange(1, E + 1))).astype(np.float32)


def repair(spec, router_bias=None, max_rounds=50):
    """Redraw token rows until every margin the routing decisions depend on
    exceeds 1e-3: the top-k margin of the selection scores and, with rerouting,
    the gaps among the ranks each token's reroutes consulted."""
    wr64 = O.widen(W.make_router(spec))
    b64 = None if router_bias is None else np.asarray(router_bias, np.float32).astype(np.float64)
    bs64 = O.widen(W.make_selection_bias(spec)) if spec.selection_bias else None
    redraw = {}
    for _ in range(max_rounds):
        if spec.capacity_policy == "reroute":
            inp = {"x": W.make_x(spec, redraw), "w_router": W.make_router(spec),
                   "b_router": None if router_bias is None else np.asarray(router_bias, np.float32),
                   "b_select": W.make_selection_bias(spec) if spec.selection_bias else None}
            margin = O.route(inp, O.desc_of(spec))["margin"]
        else:
            g = O.router_logits(O.widen(W.make_x(spec, redraw)), wr64, b64)
            _, margin = O.topk_by_logit(O.selection_scores(g, bs64), spec.top_k)
        bad = np.flatnonzero(margin <= O.MARGIN_MIN)
        if bad.size == 0:
            return redraw
        for r in bad.tolist():
            redraw[r] = redraw.get(r, 0) + 1
    raise RuntimeError("margin repair did not converge")


@functools.lru_cache(maxsize=8)
def inputs_for(name: str, seed: int = 0):
    """(spec, inputs) for a named workload or a small test shape."""
    if name in W.WORKLOADS:
        spec = W.WORKLOADS[name]
        if seed != 0:
            spec = spec.with_(seed=seed)
            rb = small_router_bias(spec) if spec.router_bias else None
            return spec, synth.make_inputs(spec, redraw=repair(spec, rb), router_bias=rb, params={})
        return spec, synth.make_inputs(spec)
    spec = SMALL[name].with_(seed=seed)
    rb = small_router_bias(spec) if spec.router_bias else None
    return spec, synth.make_inputs(spec, redraw=repair(spec, rb), router_bias=rb, params={})


def desc_of(spec):
    return O.desc_of(spec)
