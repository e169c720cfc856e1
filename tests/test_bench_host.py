"""Host logic of bench.py and of the binding's work counts (CPU only).

- `--gpus N` above 1 is refused before any GPU call;
- rocprofv3 counter CSVs are turned into HBM bytes by the copy kernel's
  calibration (mean over dispatches, largest matching kernel);
- a stored traffic figure is used only while the kernel sources match;
- the layer's algorithmic FLOPs equal the sum of its GEMMs written out one by
  one, 556.0 MFLOP per token at K3 shape.
"""

import argparse
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_moe_transformer_gemm_amd import lmoe  # noqa: E402


def test_gpus_above_one_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, kernel, counter, value])
    return str(path)


def test_summarize_pmc_scales_counts_by_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gv = "gemm3p_kernel<Tile3<...>, ExpertGVProb<...>>"
    up = "gemm3_kernel<Tile3<...>, UpProb<...>>"
    fetch = _counters(tmp_path / "f.csv", [(gv, "FETCH_SIZE", 300), (gv, "FETCH_SIZE", 500), (up, "FETCH_SIZE", 40),
                                           ("other_kernel", "FETCH_SIZE", 9999)])
    write = _counters(tmp_path / "w.csv", [(gv, "WRITE_SIZE", 10), (gv, "WRITE_SIZE", 30), (up, "WRITE_SIZE", 8)])
    # copy kernel of 1 MiB each way: 512 fetch units and 1024 write units
    cfetch = _counters(tmp_path / "cf.csv", [("copy", "FETCH_SIZE", 512), ("tiny", "FETCH_SIZE", 3)])
    cwrite = _counters(tmp_path / "cw.csv", [("copy", "WRITE_SIZE", 1024)])
    a = argparse.Namespace(summarize_pmc=[fetch, write, cfetch, cwrite], copy_bytes=1 << 20, workload="wl")
    bench.summarize_pmc(a)
    with open(tmp_path / "traffic_wl.json") as fh:
        out = json.load(fh)
    assert out["source_hash"] == bench.source_hash()
    assert out["copy_calibration"]["bytes_per_fetch_unit"] == 2048.0
    assert out["copy_calibration"]["bytes_per_write_unit"] == 1024.0
    k = out["kernels"]
    assert set(k) == {"expert_gate_value", "up"}  # kernels with both counters only
    assert k["expert_gate_value"]["fetch_bytes"] == 400 * 2048.0  # mean over the two dispatches
    assert k["expert_gate_value"]["write_bytes"] == 20 * 1024.0
    assert k["up"]["fetch_bytes"] == 40 * 2048.0 and k["up"]["write_bytes"] == 8 * 1024.0


def test_measured_traffic_needs_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("wl", "expert_gate_value") is None  # no file
    rec = {"source_hash": bench.source_hash(),
           "kernels": {"expert_gate_value": {"fetch_bytes": 10.0, "write_bytes": 2.5}}}
    with open(tmp_path / "traffic_wl.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.measured_traffic("wl", "expert_gate_value") == 12.5
    assert bench.measured_traffic("wl", "up") is None  # not counted
    rec["source_hash"] = "0" * 16  # taken on other kernel sources
    with open(tmp_path / "traffic_wl.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.measured_traffic("wl", "expert_gate_value") is None


def test_layer_flops_is_the_sum_of_its_gemms():
    H, L, E, k, I, S, Is = 7168, 3584, 896, 16, 1024, 2, 1024
    sh = lmoe.make_shape(T=3, H=H, L=L, E=E, k=k, I=I, S=S, Is=Is)
    macs_per_token = {
        "router": H * E,
        "down": H * L,
        "expert gate and value": k * 2 * L * I,
        "expert out": k * I * L,
        "up": L * H,
        "shared gate and value": S * 2 * H * Is,
        "shared out": S * Is * H,
    }
    per_token = 2 * sum(macs_per_token.values())
    assert lmoe.layer_flops(sh) == 3 * per_token
    assert round(per_token / 1e6, 1) == 556.0
    # identity projections: no down and no up GEMM
    no_proj = per_token - 2 * (macs_per_token["down"] + macs_per_token["up"])
    assert lmoe.layer_flops(sh, projections=False) == 3 * no_proj
    assert lmoe.layer_flops(sh, tokens=1) == per_token
