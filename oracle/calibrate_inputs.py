"""Decide the data-dependent input parameters of the named workloads.

TEST INFRASTRUCTURE: run by hand (``python -m oracle.calibrate_inputs``); it
writes ``synth/input_params.json``, which the seeded generator reads.  It uses
only the oracle's own routing (fp64 on the stored, dtype-rounded values).

Per workload it records:
  router_bias  fp32 logit bias (skewed workloads only):
               - Mixtral-shaped prefill: expert e's share of the 2T top-2
                 assignments follows normalised Zipf(1), 1/(e+1) / H_E, each
                 share within 1 percentage point.  Start b_e = -ln(e+1) and
                 iterate b <- b + 0.5 (ln target - ln share).
               - Switch-style layer: beta on the 8 hot experts (every 8th
                 expert), 0 elsewhere; bisect beta until the hot experts take
                 50% +- 0.5 pp of the top-1 choices.
  redraw       {row: attempt}: token rows redrawn from their own stream until
               every top-k logit margin (consecutive ranked gaps among ranks
               0..k) exceeds 1e-3, so the GPU's fp32 logits cannot reorder any
               choice; with the reroute policy, every gap among the ranks a
               token's reroutes consulted as well.
  stats        achieved loads, drops and the smallest margin (report only).
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synth  # noqa: E402
from synth import workloads as W  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402


def _logits(spec, x_stored, wr64, bias):
    return O.router_logits(O.widen(x_stored), wr64,
                           None if bias is None else np.asarray(bias, np.float32).astype(np.float64))


def _shares(spec, g):
    idx, _ = O.topk_by_logit(g, spec.top_k)
    return np.bincount(idx.ravel(), minlength=spec.n_experts) / idx.size, idx


def calibrate_zipf(spec, x_stored, wr64, tol=0.01, max_iter=200):
    E = spec.n_experts
    target = 1.0 / np.arange(1, E + 1)
    target /= target.sum()
    b = (-np.log(np.arange(1, E + 1))).astype(np.float32)
    for _ in range(max_iter):
        share, _ = _shares(spec, _logits(spec, x_stored, wr64, b))
        if np.all(np.abs(share - target) <= tol):
            return b, share, target
        b = (b.astype(np.float64) + 0.5 * (np.log(target) - np.log(np.maximum(share, 1e-9)))).astype(np.float32)
    raise RuntimeError(f"zipf calibration did not converge: {share} vs {target}")


def calibrate_hot(spec, x_stored, wr64, hot, target=0.5, tol=0.005):
    lo, hi = 0.0, 4.0
    for _ in range(60):
        beta = 0.5 * (lo + hi)
        b = np.zeros(spec.n_experts, np.float32)
        b[hot] = np.float32(beta)
        g = _logits(spec, x_stored, wr64, b)
        idx, _ = O.topk_by_logit(g, 1)
        frac = np.isin(idx[:, 0], hot).mean()
        if abs(frac - target) <= tol:
            return b, frac
        if frac < target:
            lo = beta
        else:
            hi = beta
    raise RuntimeError("hot-expert calibration did not converge")


def repair_margins(spec, wr64, bias, max_rounds=50):
    """Redraw rows whose top-k margin is <= 1e-3; returns (redraw map, logits)."""
    redraw = {}
    x = W.make_x(spec, redraw)
    for _ in range(max_rounds):
        g = _logits(spec, x, wr64, bias)
        _, margin = O.topk_by_logit(g, spec.top_k)
        if spec.capacity_policy == "reroute":
            r = O.route({"x": x, "w_router": W.make_router(spec), "b_router": bias},
                        O.desc_of(spec))
            margin = np.minimum(margin, r["margin"])
        bad = np.flatnonzero(margin <= O.MARGIN_MIN)
        if bad.size == 0:
            return redraw, g, margin
        for row in bad.tolist():
            redraw[row] = redraw.get(row, 0) + 1
        x = W.make_x(spec, redraw)
    raise RuntimeError("margin repair did not converge")


def calibrate(spec):
    out = {}
    wr64 = O.widen(W.make_router(spec))
    x_raw = W.make_x(spec, {})
    bias = None
    if spec.name == "mixtral_prefill_bf16":
        bias, share, target = calibrate_zipf(spec, x_raw, wr64)
        out["zipf_target"] = target.tolist()
    elif spec.name in ("switch_capacity_bf16", "switch_reroute_bf16"):
        hot = list(range(0, spec.n_experts, 8))
        bias, frac = calibrate_hot(spec, x_raw, wr64, hot)
        out["hot_experts"] = hot
    redraw, g, margin = repair_margins(spec, wr64, bias)
    share, idx = _shares(spec, g)
    out["redraw"] = {str(k): int(v) for k, v in sorted(redraw.items())}
    if bias is not None:
        out["router_bias"] = [float(v) for v in np.asarray(bias, np.float32)]
    keep = O.capacity_keep(idx, spec.n_experts, spec.capacity)
    counts = np.array([np.sum((idx == e) & keep) for e in range(spec.n_experts)])
    out["stats"] = {
        "assignment_share": [round(float(s), 6) for s in share],
        "kept_rows_per_expert": counts.tolist(),
        "dropped": int(idx.size - keep.sum()),
        "min_margin": float(margin.min()),
        "redrawn_rows": len(redraw),
    }
    if spec.capacity_policy == "reroute":
        r = O.route({"x": W.make_x(spec, redraw), "w_router": W.make_router(spec),
                     "b_router": bias}, O.desc_of(spec))
        out["stats"]["reroute"] = {"rounds": int(r["reroute_rounds"]),
                                   "rerouted": int(((r["topk_idx"] != r["router_idx"]) & r["keep"]).sum()),
                                   "dropped": int((~r["keep"]).sum())}
    if spec.name in ("switch_capacity_bf16", "switch_reroute_bf16"):
        out["stats"]["hot_top1_fraction"] = float(np.isin(idx[:, 0], out["hot_experts"]).mean())
    # Workload-level properties the descriptions ask for.
    demand = np.bincount(idx.ravel(), minlength=spec.n_experts)
    if spec.name == "mid_bf16":
        mean = spec.top_k * spec.tokens / spec.n_experts
        assert np.all(np.abs(demand - mean) <= 0.2 * mean), demand
    if spec.name == "decode_bf16":
        assert np.all(demand >= 1), demand
    return out


def main():
    params = {}
    for name, spec in W.WORKLOADS.items():
        params[name] = calibrate(spec)
        print(name, json.dumps(params[name]["stats"]))
    with open(W._PARAMS_PATH, "w") as f:
        json.dump(params, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
