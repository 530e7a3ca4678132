"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one moe_forward (route -> permute -> grouped FFN -> combine) over one
batch of synthetic tokens already resident in HBM.  Prints ONE JSON line with
tokens/s, the roofline of the dominant kernel (timed live with HIP events on
the stream it runs on) and the fp64 CPU oracle timed on a bounded sample.

    python bench.py --summarize --stats-csv KS.csv --fetch-csv F.csv --write-csv W.csv \
        --workload NAME --copy-probe-mib N --command "..."

reduces rocprofv3 output (kernel_stats.csv of a --kernel-trace --stats run and
counter_collection.csv of a FETCH_SIZE run and of a WRITE_SIZE run, all written
with --output-format csv) to the markdown summary kept beside the results.  The
counter runs pass --copy-probe-mib so that one plain copy of known size is
measured by the same counters; its reading scales them to bytes.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer tokens/sec + % of bf16 MFMA peak (prefill) / % HBM BW (decode)"
COPY_KERNEL_TAG = "neg_kernel"   # torch.neg: reads N bytes, writes N bytes


def sources_sha256() -> str:
    """Hash of the library's sources: a traffic figure measured on other sources is stale."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "sparse_mixture_experts_49_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "moe_mi355x.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(entry: str, workload: str):
    """HBM bytes per launch of `entry` on `workload` from the committed counter summaries,
    or None if there is none for the current sources."""
    sha = sources_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            m = re.match(r"<!-- traffic (\{.*\}) -->", line.strip())
            if not m:
                continue
            rec = json.loads(m.group(1))
            if rec["entry"] == entry and rec["workload"] == workload and rec["sources_sha256"] == sha:
                return rec["bytes_per_launch"]
    return None


def _to_dev(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _time_events(fn, reps, warmup=2):
    """Average duration (ms) of fn() over reps launches, HIP events on the current stream
    (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def cpu_baseline(spec, inp, sample_tokens):
    """The fp64 oracle as it stands, on a bounded token sample of the same workload.
    Returns the baseline record and the oracle's result on that sample."""
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(spec.tokens, size=min(sample_tokens, spec.tokens), replace=False))
    t0 = time.perf_counter()
    ref = O.forward(inp, O.desc_of(spec), tokens=toks)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"value": round(len(toks) / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(toks)} of {spec.tokens} tokens (routing of all tokens, expert FFNs of "
                      f"the sampled tokens), fp64 NumPy/BLAS, {dt:.1f} s"}, ref


def parity_of(spec, ref, y, aux, routing):
    """The timed run's outputs against the oracle's on the CPU-baseline sample: y's
    max|err|/RMS over the sampled tokens, aux's relative error, routing exactness."""
    toks = ref["tokens"]
    yg = y.cpu().numpy().astype(np.float64)[toks]
    yr = ref["y"]
    rms = float(np.sqrt(np.mean(yr ** 2)))
    idx = routing.topk_idx.cpu().numpy()
    want = ref["topk_idx"] if spec.capacity_policy != "reroute" else np.where(ref["keep"], ref["topk_idx"], -1)
    return {"tokens_compared": int(toks.size),
            "y_max_err_over_rms": float(np.max(np.abs(yg - yr)) / rms),
            "y_tol": 2e-2 if spec.dtype == "bf16" else 1e-4,
            "aux_rel_err": abs(float(aux.item()) - ref["aux"]) / abs(ref["aux"]),
            "routing_exact": bool(np.array_equal(idx, want)
                                  and np.array_equal(routing.counts.cpu().numpy(), ref["counts"])
                                  and np.array_equal(routing.dest.cpu().numpy(), ref["dest"]))}


def stream_read_gbs(dev, mib=1792, reps=20):
    """The library's plain streaming-read probe over `mib` MiB (about the decode
    layer's expert bank) on the same GPU: the practical HBM read ceiling next to
    the 8 TB/s grade."""
    import torch
    import sparse_mixture_experts_49_amd as moe
    buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ms = _time_events(lambda: moe.moe_read_probe(buf, sink), reps)
    del buf
    return round(mib * (1 << 20) / (ms * 1e-3) / 1e9, 1)


def kernel_bytes(spec, R, active, h_elem):
    """Algorithmic HBM bytes of one launch of each expert kernel: the weights (and biases)
    of the experts that received rows, read once, plus the activations each reads and
    writes once at their stored widths (o is fp32)."""
    s = 2 if spec.dtype == "bf16" else 4
    d, F = spec.d_model, spec.d_ff
    bias = 1 if spec.expert_bias else 0
    up = active * (F * d + bias * F) * s + R * d * s + R * F * h_elem
    down = active * (d * F + bias * d) * s + R * F * h_elem + R * d * 4
    return up, down


def measure(spec, args, dev, steps, with_cpu):
    """One workload: moe_forward timed over `steps` steps, its expert products timed
    alone in the launch configuration moe_forward uses, the roofline of the dominant
    one, the routing's loads and drops, and (with_cpu) the oracle on a bounded sample
    with the timed run's parity against it."""
    import torch
    import sparse_mixture_experts_49_amd as moe
    import synth

    inp = synth.make_inputs(spec)
    desc = moe.Desc(spec.tokens, spec.d_model, spec.d_ff, spec.n_experts, spec.top_k,
                    spec.renormalize, spec.capacity, spec.dtype, spec.expert_bias,
                    d_ff_shared=spec.d_ff_shared, capacity_policy=spec.capacity_policy)
    x = _to_dev(inp["x"], dev)
    w = moe.Weights(**{name: _to_dev(inp.get(name), dev) for name in (
        "w_router", "w1", "w2", "b_router", "b1", "b2", "b_select", "w1_shared", "b1_shared",
        "w2_shared", "b2_shared")})
    ws = moe.alloc_workspace(desc, dev)
    y = torch.empty(spec.tokens, spec.d_model, dtype=torch.float32, device=dev)
    aux = torch.empty((), dtype=torch.float32, device=dev)
    routing = moe.Routing.allocate(desc, dev)

    def step():
        moe.moe_forward(desc, x, w, y, aux, routing, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    y_out = y.clone()
    aux_out = aux.clone()

    # The expert products alone, as moe_forward launches them: the first reads each
    # dispatched row's token from x through src, the second reads h.
    Tk = spec.tokens * spec.top_k
    h = moe.alloc_h(desc, dev)
    o = torch.empty(Tk, spec.d_model, dtype=torch.float32, device=dev)
    R = int(routing.offsets[-1].item())
    counts = routing.counts.cpu().numpy()
    active = int((counts > 0).sum())
    up_ms = _time_events(lambda: moe.moe_ffn_up_gather(desc, x, routing.src, routing.offsets, w, h, ws),
                         args.kernel_reps)
    down_ms = _time_events(lambda: moe.moe_ffn_down(desc, h, routing.offsets, w, o, ws), args.kernel_reps)
    r2 = moe.Routing.allocate(desc, dev)
    route_ms = _time_events(lambda: moe.moe_route(desc, x, w, r2, None, ws), args.kernel_reps)
    shared_ms = None
    if spec.d_ff_shared:
        o_sh = torch.empty(spec.tokens, spec.d_model, dtype=torch.float32, device=dev)
        shared_ms = _time_events(lambda: moe.moe_shared_ffn(desc, x, w, o_sh, ws), args.kernel_reps)

    plan = moe.moe_query_plan(desc)
    h_elem = h.element_size() * (2 if h.dim() == 3 else 1)
    bf16 = spec.dtype == "bf16"
    flops_one = 2.0 * R * spec.d_ff * spec.d_model          # each of the two products
    up_bytes, down_bytes = kernel_bytes(spec, R, active, h_elem)
    peak_flops = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    # The FFN is MFMA-bound when its arithmetic intensity exceeds the ridge point.
    mfma_bound = 2 * flops_one / (up_bytes + down_bytes) > peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    dom, dom_ms, dom_bytes = ("moe_ffn_up", up_ms, up_bytes) if up_ms >= down_ms else \
        ("moe_ffn_down", down_ms, down_bytes)
    traffic = recorded_traffic(dom, spec.name)
    if mfma_bound:
        achieved = flops_one / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(achieved / peak_flops, 4)}
    else:
        achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": traffic, "kernel": dom, "kernel_ms": round(dom_ms, 4),
                 "algorithmic_bytes": dom_bytes, "algorithmic_flops": flops_one})
    # Every byte one step must move at least once: x, the router and the touched
    # experts' weights and biases, y (fp32).
    s_el = 2 if bf16 else 4
    step_bytes = (spec.tokens * spec.d_model * s_el + spec.n_experts * spec.d_model * s_el
                  + active * (2 * spec.d_ff * spec.d_model + (spec.d_ff + spec.d_model) * spec.expert_bias) * s_el
                  + spec.tokens * spec.d_model * 4)
    out = {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(spec.tokens / (ms * 1e-3), 1),
        "config": {"workload": spec.name, "tokens": spec.tokens, "d_model": spec.d_model,
                   "d_ff": spec.d_ff, "n_experts": spec.n_experts, "top_k": spec.top_k,
                   "capacity": spec.capacity, "capacity_policy": spec.capacity_policy,
                   "kept_rows": R, "active_experts": active,
                   "ffn_path": {1: "tiled", 2: "stream"}[plan["ffn_path"]],
                   "h_mode": {0: "f32", 1: "bf16", 2: "split"}[plan["h_mode"]]},
        "roofline": roof,
        "layer": {"route_ms": round(route_ms, 4),
                  "ffn_up_ms": round(up_ms, 4), "ffn_down_ms": round(down_ms, 4),
                  "ffn_tflops": round(2 * flops_one / ((up_ms + down_ms) * 1e-3) / 1e12, 1),
                  "ffn_frac_peak": round(2 * flops_one / ((up_ms + down_ms) * 1e-3) / 1e12 / peak_flops, 4),
                  "ffn_gbs": round((up_bytes + down_bytes) / ((up_ms + down_ms) * 1e-3) / 1e9, 1),
                  "step_min_bytes": int(step_bytes),
                  "step_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                  "step_frac_hbm": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "loads": {"kept_per_expert": counts.tolist(), "dropped": int(Tk - R)},
    }
    if shared_ms is not None:
        sh_flops = 4.0 * spec.tokens * spec.d_model * spec.d_ff_shared
        out["layer"].update({"shared_ffn_ms": round(shared_ms, 4),
                             "shared_ffn_tflops": round(sh_flops / (shared_ms * 1e-3) / 1e12, 1)})
    if with_cpu:
        base, ref = cpu_baseline(spec, inp, args.cpu_sample)
        out["cpu_baseline"] = base
        out["parity"] = parity_of(spec, ref, y_out, aux_out, routing)
    del x, w, ws, h, o
    torch.cuda.empty_cache()
    return out


def run(args):
    import synth

    dev = "cuda:0"
    if args.copy_probe_mib:
        # One plain copy of known size for scaling the HBM byte counters (see the module doc).
        import torch
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    main = measure(synth.WORKLOADS[args.workload], args, dev, args.steps, not args.no_cpu_baseline)
    out = {
        "metric": METRIC,
        "value": main["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": synth.WORKLOADS[args.workload].dtype,
        "data": "synthetic",
        "config": main["config"],
        "roofline": main["roofline"],
        "layer": main["layer"],
        "loads": main["loads"],
    }
    for key in ("parity", "cpu_baseline"):
        if key in main:
            out[key] = main[key]
    if args.decode_workload and args.decode_workload != args.workload:
        # The decode half of the metric: the small-batch layer, HBM-bound, timed in the
        # same run (more steps: one step is a few hundred microseconds).
        dec = measure(synth.WORKLOADS[args.decode_workload], args, dev, args.decode_steps,
                      not args.no_cpu_baseline)
        out["decode"] = {k: dec[k] for k in ("ms_per_step", "tokens_per_s", "config", "roofline",
                                            "layer", "loads", "parity", "cpu_baseline") if k in dec}
        out["decode"]["steps"] = args.decode_steps
    out["stream_read_gbs"] = stream_read_gbs(dev)
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------------------
# rocprofv3 output -> markdown summary

def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _entry_of(kernel_name: str):
    """Entry point that launches a HIP kernel of this library (by kernel name)."""
    m = re.search(r"moe::(\w+)<(.*)>\(", kernel_name) or re.search(r"moe::(\w+)\(", kernel_name)
    if not m:
        return None
    base = m.group(1)
    if base.startswith("ffn_"):
        up = re.search(r"\b(true|false)\b", m.group(2)).group(1) == "true"
        return "moe_ffn_up" if up else "moe_ffn_down"
    if base.startswith(("router", "aux", "reroute")):
        return "moe_route"
    if base.startswith("perm"):
        return "moe_permute"
    if base.startswith("combine"):
        return "moe_combine"
    return None


def _short(name: str, n=90):
    name = re.sub(r"\(.*", "", name)
    return name if len(name) <= n else name[:n - 3] + "..."


def _counter_avgs(path, counter):
    """Per kernel name: average over dispatches of the counter summed over its instances."""
    per = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        key = r["Kernel_Name"]
        d = per.setdefault(key, {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def summarize(args):
    lines = [f"# rocprofv3 summary: {args.workload}", ""]
    if args.command:
        lines += ["Commands (run from the repository root):", "", "```"] + args.command + ["```", ""]
    if args.stats_csv:
        lines += ["## Kernel durations (`--kernel-trace --stats`)", "",
                  "| kernel | entry point | calls | avg us | min us | max us | share |",
                  "|---|---|---|---|---|---|---|"]
        for r in _rows(args.stats_csv):
            e = _entry_of(r["Name"]) or "-"
            lines.append(f"| `{_short(r['Name'])}` | {e} | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                         f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
        lines.append("")
    if args.mfma_csv:
        # Per kernel name, averaged over its dispatches: shader clock from the
        # GPU-busy cycle count (summed over the 8 XCDs) over the dispatch's duration,
        # and the share of those cycles each SIMD's matrix unit was busy.
        xcds, simds = 8, 1024
        per = {}
        for r in _rows(args.mfma_csv):
            k = r["Kernel_Name"]
            if _entry_of(k) is None:
                continue
            d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        lines += ["## MFMA utilisation and shader clock (`--pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES "
                  "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA`)", "",
                  "Clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration (this counter run's own "
                  "timestamps); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8).",
                  "", "| kernel | entry point | dispatches | clock GHz | MFMA busy | MFMA instructions |",
                  "|---|---|---|---|---|---|"]
        for k, ds in sorted(per.items()):
            vals = [v for v in ds.values() if v.get("GRBM_GUI_ACTIVE") and v["_ns"] > 0]
            if not vals:
                continue
            clk = sum(v["GRBM_GUI_ACTIVE"] / xcds / v["_ns"] for v in vals) / len(vals)
            busy = sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / simds / (v["GRBM_GUI_ACTIVE"] / xcds)
                       for v in vals) / len(vals)
            mi = sum(v.get("SQ_INSTS_MFMA", 0.0) for v in vals) / len(vals)
            if mi == 0:
                continue
            lines.append(f"| `{_short(k)}` | {_entry_of(k)} | {len(vals)} | {clk:.2f} | {busy:.1%} | {mi:.4g} |")
        lines.append("")
    if args.fetch_csv and args.write_csv:
        fetch = _counter_avgs(args.fetch_csv, "FETCH_SIZE")
        write = _counter_avgs(args.write_csv, "WRITE_SIZE")
        copy_kib = args.copy_probe_mib * 1024.0
        cf = [v for k, v in fetch.items() if COPY_KERNEL_TAG in k]
        cw = [v for k, v in write.items() if COPY_KERNEL_TAG in k]
        if not cf or not cw:
            raise SystemExit("the copy probe kernel is missing from the counter runs")
        sf, sw = copy_kib / cf[0][0], copy_kib / cw[0][0]
        lines += ["## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
                  f"Scale: a plain copy of {args.copy_probe_mib} MiB (`torch.neg`, reads and writes "
                  f"{copy_kib:.0f} KiB) reads FETCH_SIZE {cf[0][0]:.0f} KiB and WRITE_SIZE "
                  f"{cw[0][0]:.0f} KiB, so FETCH_SIZE x {sf:.4f} and WRITE_SIZE x {sw:.4f} give bytes "
                  "moved to and from memory.", "",
                  "| kernel | entry point | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | "
                  "scaled bytes per launch |", "|---|---|---|---|---|---|"]
        recs = {}
        for k, (fv, n) in sorted(fetch.items()):
            e = _entry_of(k)
            if e is None:
                continue
            wv = write.get(k, (0.0, 0))[0]
            b = (fv * sf + wv * sw) * 1024.0
            lines.append(f"| `{_short(k)}` | {e} | {n} | {fv:.0f} | {wv:.0f} | {b:.4g} |")
            if e in ("moe_ffn_up", "moe_ffn_down"):   # every kernel the entry point launches
                recs[e] = recs.get(e, 0.0) + b
        lines.append("")
        sha = sources_sha256()
        for e, b in sorted(recs.items()):
            lines.append("<!-- traffic " + json.dumps(
                {"entry": e, "workload": args.workload, "bytes_per_launch": round(b),
                 "sources_sha256": sha}) + " -->")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_prefill_bf16")
    ap.add_argument("--decode-workload", default="decode_bf16",
                    help="measured after the main workload, reported under 'decode' ('' to skip)")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--summarize", action="store_true")
    ap.add_argument("--stats-csv")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--mfma-csv")
    ap.add_argument("--command", action="append")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X; sharding across GPUs "
              "is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
