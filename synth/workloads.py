"""Seeded synthetic inputs for the sparsely-gated MoE layer forward.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
bench.  It only draws random numbers and stores them in the dtype a workload
asks for.  It holds none of the layer's arithmetic: no router product, no
softmax, no top-k, no expert FFN.  The two data-dependent adjustments a named
workload needs (the fp32 router logit bias that creates the load skew, and the
list of token rows redrawn so that every top-k logit margin exceeds 1e-3) are
read from ``input_params.json``; that file is written by a script under
``oracle/`` which decides them with the oracle's own routing.

Layouts (row-major, nn.Linear ``[out][in]`` for weights):
  x          [T][d]                  f32 or bf16
  w_router   [E][d]                  f32 or bf16
  b_router   [E]                     f32 (only for the skewed workloads) or None
  b_select   [E]                     f32 selection-only bias (workloads that ask for it) or None
  w1_shared  [Fs][d], b1_shared [Fs], w2_shared [d][Fs], b2_shared [d]
                                     the shared expert (workloads with d_ff_shared > 0)
  w1         [E][d_ff][d]            f32 or bf16
  b1         [E][d_ff]               f32 or bf16, or None
  w2         [E][d][d_ff]            f32 or bf16
  b2         [E][d]                  f32 or bf16, or None
bf16 arrays are numpy ``uint16`` holding the bf16 bit patterns.

Random streams.  Every tensor has its own child stream, ``default_rng([seed,
tensor_id, sub])``, so adding or removing one tensor shifts no other draw, and
two workloads with the same expert shapes and seed share one expert bank (the
prefill and decode workloads below are such a pair).  Expert tensors use one
stream per expert (``sub`` = expert index), which also lets them be drawn in
parallel threads.  A token row that must be redrawn takes its replacement from
``default_rng([seed, 6, row, attempt])``.

Distributions: x ~ N(0, 1); weights ~ N(0, 1/fan_in) with fan_in = d for the
router and the first expert matrix and d_ff for the second; biases ~
U(-0.01, 0.01).  Every value is drawn in fp32 and, for bf16 workloads, rounded
to the nearest bf16 (ties to even).
"""
from __future__ import annotations

import dataclasses
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_X, STREAM_WR, STREAM_W1, STREAM_B1, STREAM_W2, STREAM_B2, STREAM_REDRAW = range(7)
STREAM_BSEL = 8             # per-expert selection bias (stream 7 is the calibration sample)
STREAM_W1S, STREAM_B1S, STREAM_W2S, STREAM_B2S = 9, 10, 11, 12   # shared expert

_PARAMS_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_params.json")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and routing options of one MoE layer instance."""

    name: str
    tokens: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    renormalize: bool
    capacity: int          # 0 = unlimited
    expert_bias: bool      # b1/b2 present
    dtype: str             # "f32" or "bf16"
    router_bias: bool = False  # fp32 logit bias drawn by calibration (skewed workloads)
    seed: int = 0
    selection_bias: bool = False  # fp32 per-expert bias added to the scores used to pick experts
    d_ff_shared: int = 0          # hidden width of the always-active shared expert (0: none)
    capacity_policy: str = "drop" # overflow beyond capacity: "drop" or "reroute"

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def capacity_for(tokens: int, n_experts: int, factor_num: int = 5, factor_den: int = 4) -> int:
    """Expert capacity = ceil(capacity_factor * tokens / experts), in exact integers.

    The capacity factor 1.25 is 5/4; the ceiling is taken in integer arithmetic.
    """
    return (factor_num * tokens + factor_den * n_experts - 1) // (factor_den * n_experts)


# The five workloads of the layer, named by what they are.
WORKLOADS = {
    "toy_fp32": Workload("toy_fp32", 64, 256, 1024, 8, 2, True, 0, True, "f32"),
    "mid_bf16": Workload("mid_bf16", 4096, 1024, 4096, 16, 2, True, 0, True, "bf16"),
    "mixtral_prefill_bf16": Workload("mixtral_prefill_bf16", 16384, 4096, 14336, 8, 2, True, 0,
                                     False, "bf16", router_bias=True),
    "switch_capacity_bf16": Workload("switch_capacity_bf16", 8192, 2048, 8192, 64, 1, False,
                                     capacity_for(8192, 64), True, "bf16", router_bias=True),
    # the same layer and tokens with the overflow rerouted instead of dropped
    "switch_reroute_bf16": Workload("switch_reroute_bf16", 8192, 2048, 8192, 64, 1, False,
                                    capacity_for(8192, 64), True, "bf16", router_bias=True,
                                    capacity_policy="reroute"),
    "decode_bf16": Workload("decode_bf16", 32, 4096, 14336, 8, 2, True, 0, True, "bf16"),
    # fine-grained experts (64 experts of width 1408, top-6) plus a shared expert of
    # width 2816 (two of width 1408 side by side); no router skew
    "finegrained_shared_bf16": Workload("finegrained_shared_bf16", 8192, 2048, 1408, 64, 6, True, 0,
                                        False, "bf16", d_ff_shared=2816),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def _normal(key, shape, scale: float) -> np.ndarray:
    a = _rng(*key).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def _uniform_bias(key, shape) -> np.ndarray:
    u = _rng(*key).random(shape, dtype=np.float32)
    return u * np.float32(0.02) - np.float32(0.01)


def load_params() -> dict:
    if not os.path.exists(_PARAMS_PATH):
        return {}
    with open(_PARAMS_PATH) as f:
        return json.load(f)


def draw_x_rows(spec: Workload, redraw: dict | None) -> np.ndarray:
    """Token activations in fp32 before dtype rounding, with redrawn rows applied."""
    x = _normal((spec.seed, STREAM_X), (spec.tokens, spec.d_model), 1.0)
    for row, attempt in (redraw or {}).items():
        row = int(row)
        x[row] = _normal((spec.seed, STREAM_REDRAW, row, int(attempt)), (spec.d_model,), 1.0)
    return x


def make_selection_bias(spec: Workload) -> np.ndarray:
    """Per-expert selection bias, U(-1, 1) in fp32 (router logits are ~N(0, 1),
    so it changes a fair share of the choices)."""
    u = _rng(spec.seed, STREAM_BSEL).random(spec.n_experts, dtype=np.float32)
    return u * np.float32(2.0) - np.float32(1.0)


def make_router(spec: Workload) -> np.ndarray:
    return _store(_normal((spec.seed, STREAM_WR), (spec.n_experts, spec.d_model),
                          1.0 / np.sqrt(spec.d_model)), spec.dtype)


def make_x(spec: Workload, redraw: dict | None = None) -> np.ndarray:
    return _store(draw_x_rows(spec, redraw), spec.dtype)


def make_expert_bank(spec: Workload, threads: int | None = None) -> dict:
    """Expert weights and biases, one stream per (tensor, expert), drawn in parallel."""
    E, d, F = spec.n_experts, spec.d_model, spec.d_ff
    el = np.uint16 if spec.dtype == "bf16" else np.float32
    w1 = np.empty((E, F, d), el)
    w2 = np.empty((E, d, F), el)
    b1 = np.empty((E, F), el) if spec.expert_bias else None
    b2 = np.empty((E, d), el) if spec.expert_bias else None
    s1, s2 = 1.0 / np.sqrt(d), 1.0 / np.sqrt(F)

    def one(e):
        w1[e] = _store(_normal((spec.seed, STREAM_W1, e), (F, d), s1), spec.dtype)
        w2[e] = _store(_normal((spec.seed, STREAM_W2, e), (d, F), s2), spec.dtype)
        if spec.expert_bias:
            b1[e] = _store(_uniform_bias((spec.seed, STREAM_B1, e), (F,)), spec.dtype)
            b2[e] = _store(_uniform_bias((spec.seed, STREAM_B2, e), (d,)), spec.dtype)

    nthreads = threads or min(E, max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(one, range(E)))
    return {"w1": w1, "b1": b1, "w2": w2, "b2": b2}


def make_shared_expert(spec: Workload) -> dict:
    """The shared expert's weights (same laws as the routed experts; biases iff
    the routed experts have them)."""
    d, Fs = spec.d_model, spec.d_ff_shared
    out = {"w1_shared": _store(_normal((spec.seed, STREAM_W1S), (Fs, d), 1.0 / np.sqrt(d)), spec.dtype),
           "w2_shared": _store(_normal((spec.seed, STREAM_W2S), (d, Fs), 1.0 / np.sqrt(Fs)), spec.dtype),
           "b1_shared": None, "b2_shared": None}
    if spec.expert_bias:
        out["b1_shared"] = _store(_uniform_bias((spec.seed, STREAM_B1S), (Fs,)), spec.dtype)
        out["b2_shared"] = _store(_uniform_bias((spec.seed, STREAM_B2S), (d,)), spec.dtype)
    return out


def make_inputs(spec: Workload, redraw: dict | None = None, router_bias=None,
                with_experts: bool = True, params: dict | None = None) -> dict:
    """All inputs of one layer call.

    For a named workload, ``redraw`` and ``router_bias`` default to the stored
    values in ``input_params.json`` (pass ``params={}`` to get the raw draw).
    """
    if params is None:
        params = load_params().get(spec.name, {}) if spec.name in WORKLOADS and \
            WORKLOADS[spec.name] == spec else {}
    if redraw is None:
        redraw = params.get("redraw", {})
    if router_bias is None and spec.router_bias and "router_bias" in params:
        router_bias = params["router_bias"]
    out = {
        "x": make_x(spec, redraw),
        "w_router": make_router(spec),
        "b_router": None if router_bias is None else np.asarray(router_bias, np.float32),
        "b_select": make_selection_bias(spec) if spec.selection_bias else None,
    }
    if with_experts:
        out.update(make_expert_bank(spec))
        if spec.d_ff_shared:
            out.update(make_shared_expert(spec))
    return out
