"""The bench's measurement helpers on the CPU: the kernel-to-entry-point map, the
profile summariser's traffic scaling against a plain copy of known size, the guard
that ignores traffic recorded for other sources, the algorithmic byte counts, and
the refusal of more than one GPU."""
from __future__ import annotations

import csv
import json
import os
import re
import subprocess
import sys
import types

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_names_map_to_their_entry_points():
    e = bench._entry_of
    assert e("void moe::ffn_tiled_kernel<true, false, 256, 256, 2, 3, 1>(unsigned short const*)") == "moe_ffn_up"
    assert e("void moe::ffn_stream_lds_kernel<false, false, 1>(unsigned short const*)") == "moe_ffn_down"
    assert e("void moe::ffn_tile_reduce<false, true, 128, 256>(int const*)") == "moe_ffn_down"
    assert e("void moe::router_part_kernel<unsigned short, 1>(unsigned short const*)") == "moe_route"
    assert e("void moe::router_small_finish_kernel<2, 2>(float const*, int)") == "moe_route"
    assert e("moe::aux_finalize_kernel(double const*, int const*)") == "moe_route"
    assert e("void moe::reroute_kernel<1, 4, 1024>(int const*)") == "moe_route"
    assert e("moe::perm_rank_kernel(int const*)") == "moe_permute"
    assert e("void moe::combine_kernel<false>(float const*)") == "moe_combine"
    assert e("moe::read_probe_kernel(unsigned int const*)") is None
    assert e("void at::native::vectorized_elementwise_kernel<4>(int)") is None


def _write_counters(path, counter, rows):
    """rows: (kernel name, dispatch id, value) -> a counter_collection.csv."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, disp, val in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_summary_scales_counters_by_the_copy_and_sums_an_entry_points_kernels(tmp_path, capsys):
    copy = "void at::native::unrolled_elementwise_kernel<neg_kernel_cuda>(int)"
    up = "void moe::ffn_tiled_kernel<true, false, 256, 256, 2, 3, 1>(unsigned short const*)"
    red = "void moe::ffn_tile_reduce<true, false, 256, 256>(int const*)"
    # A 1 MiB copy reads 1024 KiB and writes 1024 KiB; FETCH_SIZE reports half the reads.
    # The product kernel has two dispatches, each counted over two instances.
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                    [(copy, 1, 512.0), (up, 2, 100.0), (up, 2, 50.0), (up, 3, 150.0), (up, 3, 150.0),
                     (red, 4, 10.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE",
                    [(copy, 1, 1024.0), (up, 2, 40.0), (up, 3, 40.0), (red, 4, 6.0)])
    args = types.SimpleNamespace(workload="toy_fp32", command=None, stats_csv=None, mfma_csv=None,
                                 fetch_csv=str(tmp_path / "f.csv"), write_csv=str(tmp_path / "w.csv"),
                                 copy_probe_mib=1)
    bench.summarize(args)
    out = capsys.readouterr().out
    assert "FETCH_SIZE x 2.0000 and WRITE_SIZE x 1.0000" in out
    recs = [json.loads(m) for m in re.findall(r"<!-- traffic (\{.*\}) -->", out)]
    assert len(recs) == 1 and recs[0]["entry"] == "moe_ffn_up"
    # up: fetch avg (150 + 300) / 2 = 225 KiB x 2, write 40 KiB; reduce: 10 x 2 + 6 KiB.
    assert recs[0]["bytes_per_launch"] == round(((225 * 2 + 40) + (10 * 2 + 6)) * 1024)
    assert recs[0]["sources_sha256"] == bench.sources_sha256()


def test_traffic_recorded_for_other_sources_is_ignored(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"entry": "moe_ffn_up", "workload": "w", "bytes_per_launch": 123,
            "sources_sha256": bench.sources_sha256()}
    stale = dict(good, workload="v", sources_sha256="0" * 64)
    (prof / "a.md").write_text("x\n<!-- traffic " + json.dumps(good) + " -->\n"
                               "<!-- traffic " + json.dumps(stale) + " -->\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_sha256", lambda: good["sources_sha256"])
    assert bench.recorded_traffic("moe_ffn_up", "w") == 123
    assert bench.recorded_traffic("moe_ffn_up", "v") is None
    assert bench.recorded_traffic("moe_ffn_down", "w") is None


def test_algorithmic_bytes_of_the_decode_products():
    """Each touched expert's weights and biases once, activations at their stored widths,
    o in fp32: written out for the decode layer (8 experts, 64 rows, one h plane)."""
    spec = synth.WORKLOADS["decode_bf16"]
    d, F, R, A = spec.d_model, spec.d_ff, 64, 8
    up, down = bench.kernel_bytes(spec, R, A, 2)
    assert up == A * (F * d + F) * 2 + R * d * 2 + R * F * 2
    assert down == A * (d * F + d) * 2 + R * F * 2 + R * d * 4
    assert up == 942_112_768 and down == 942_473_216


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in (res.stdout + res.stderr)
