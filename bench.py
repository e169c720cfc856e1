"""Benchmark of the Stable Latent MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload k3_t8192]

A step is one full layer call (route GEMM, top-k, permute, expert gate/value
GEMM, expert down GEMM, combine + RMSNorm, up + shared GEMM) over one batch of
seeded synthetic inputs already resident in HBM.  Prints one JSON line:
tokens/s of the prefill workload (K3 shape, T=8192, bf16), its TFLOP/s as a
fraction of the bf16 MFMA peak, per-stage times from HIP events recorded on
the launch stream, the roofline of the dominant kernel (expert gate/value
GEMM, HBM-bound), the decode workload (T=64) in HBM GB/s, and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-MoE layer tokens/s at T=8192 bf16 (% MFMA peak); T=64 decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (about 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "sparse_moe_transformer_gemm_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
GV_KERNEL = "ExpertGVProb"  # substring of the expert gate/value GEMM kernel name


def source_hash():
    """Hash of the kernel sources: counter-based traffic figures are only
    reported while the kernels they were taken on are unchanged."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3_t8192")
    ap.add_argument("--decode-workload", default="k3_decode_t64")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens the oracle runs for cpu_baseline (0: skip)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary lines (Zipf-skewed router at T=16384, e4m3 expert weights at T=8192)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 3 s clock reading (profiler runs)")
    ap.add_argument("--pack", action="store_true",
                    help="pack the routed expert weights once (lmoe_pack_experts) and time the layer on them")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (PMC calibration) and exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of the layer and of the copy "
                         "calibration into profiles/traffic_<workload>.json, then exit")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--quantile", action="store_true",
                    help="time the Quantile Balancing threshold solve (lmoe_quantile_bias) on the workload's "
                         "router-logit shape; prints its own JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="time lmoe_backward (forward recompute + every gradient) instead of the forward; "
                         "prints its own JSON line")
    ap.add_argument("--library-gemms", action="store_true",
                    help="context only: time torch's bf16 GEMMs (hipBLASLt) at the T=8192 layer's dense and "
                         "uniform-load expert shapes; prints its own JSON line")
    return ap.parse_args()


def calibrate_copy(nbytes):
    """One elementwise kernel that reads and writes `nbytes` each (fp32
    negation), so the HBM counters can be scaled to bytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _counter_means(path):
    """{kernel name: {counter: mean over dispatches}} from a counter_collection.csv."""
    acc = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], [])
            d.append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def summarize_pmc(a):
    fetch, write, cfetch, cwrite = (_counter_means(p) for p in a.summarize_pmc)
    # the calibration run holds one copy kernel (the largest dispatch)
    cf = max(v.get("FETCH_SIZE", 0) for v in cfetch.values())
    cw = max(v.get("WRITE_SIZE", 0) for v in cwrite.values())
    f_scale, w_scale = a.copy_bytes / cf, a.copy_bytes / cw
    out = {"workload": a.workload, "source_hash": source_hash(),
           "copy_calibration": {"bytes": a.copy_bytes, "FETCH_SIZE": cf, "WRITE_SIZE": cw,
                                "bytes_per_fetch_unit": f_scale, "bytes_per_write_unit": w_scale},
           "kernels": {}}
    for name, tag in (("expert_gate_value", "ExpertGVProb"), ("expert_down", "ExpertDownProb"),
                      ("route_gemm", "DenseXProb"), ("up", "UpProb"), ("combine_norm", "combine_norm")):
        fk = [v["FETCH_SIZE"] for k, v in fetch.items() if tag in k and "FETCH_SIZE" in v]
        wk = [v["WRITE_SIZE"] for k, v in write.items() if tag in k and "WRITE_SIZE" in v]
        if fk and wk:
            # a dense GEMM runs as two kernels (full waves, then the re-cut
            # last wave): the step's traffic is their sum
            out["kernels"][name] = {"fetch_bytes": sum(fk) * f_scale, "write_bytes": sum(wk) * w_scale,
                                    "FETCH_SIZE": sum(fk), "WRITE_SIZE": sum(wk), "kernels": len(fk)}
    path = os.path.join(PROFILES, f"traffic_{a.workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(path)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash() or kernel not in t.get("kernels", {}):
        return None
    k = t["kernels"][kernel]
    return k["fetch_bytes"] + k["write_bytes"]


def sample_clock(step, seconds=3.0, depth=8, period_s=0.002):
    """The GPU's graphics clock and socket power while the layer runs.  The
    host keeps `depth` calls of `step()` queued for `seconds`, reading amdsmi's
    GPU metrics table between polls of the queued calls' events.  The
    firmware refreshes that table about once a second, so only snapshots that
    carry a new firmware timestamp, taken while calls are queued, count; the
    reading from before the loop never does."""
    import collections
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            xcd = [float(c) for c in m["current_gfxclks"] if isinstance(c, (int, float)) and c > 0]
            return m["firmware_timestamp"], sum(xcd) / len(xcd), float(m["current_socket_power"]), \
                float(m["average_gfx_activity"])
        last = read()[0]
    except Exception as e:  # no amdsmi, no permission or no such field: the field says why
        return {"mhz_mean_over_xcds": None, "error": f"{type(e).__name__}: {e}"}
    pending, snaps, calls = collections.deque(), [], 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        while len(pending) < depth:
            step()
            ev = torch.cuda.Event()
            ev.record()
            pending.append(ev)
            calls += 1
        fw, mhz, watts, busy = read()
        if fw != last and calls > depth:
            snaps.append((mhz, watts, busy))
        last = fw
        while pending and pending[0].query():
            pending.popleft()
        time.sleep(period_s)
    torch.cuda.synchronize()
    if not snaps:
        return {"mhz_mean_over_xcds": None, "error": f"no metrics refresh during the {seconds:.1f} s loop"}
    mhz = sorted(s[0] for s in snaps)
    return {"mhz_mean_over_xcds": round(mhz[len(mhz) // 2]), "mhz_min": round(mhz[0]), "mhz_max": round(mhz[-1]),
            "socket_watts": max(s[1] for s in snaps), "gfx_activity_pct": min(s[2] for s in snaps),
            "snapshots": len(snaps), "layer_calls": calls,
            "source": "amdsmi GPU metrics (current_gfxclks averaged over the XCDs), snapshots refreshed "
                      "by the firmware while layer calls were queued"}


def timed_loop(lmoe, sh, w, x, y, idx, tw, ws, steps, warmup, per_stage):
    import torch
    for _ in range(warmup):
        lmoe.forward(sh, w, x, y, idx, tw, ws)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(lmoe.NUM_STAGES + 1)] for _ in range(steps)] \
        if per_stage else None
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        lmoe.forward(sh, w, x, y, idx, tw, ws, events=evs[i] if per_stage else None)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    stages = None
    if per_stage:
        stages = {}
        for s, name in enumerate(lmoe.STAGES):
            stages[name] = sum(e[s].elapsed_time(e[s + 1]) for e in evs) / steps
    return ms, stages


def main():
    a = parse()
    if a.summarize_pmc:
        summarize_pmc(a)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the layer is measured on a single "
              f"MI355X; multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_moe_transformer_gemm_amd import lmoe
    from synth import get_config, make_inputs
    from synth.inputs import make_x

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    lmoe.load_library()
    dev = torch.device("cuda:0")
    if a.backward:
        bench_backward(a, lmoe, dev)
        return
    if a.quantile:
        bench_quantile(a, lmoe, dev)
        return
    if a.library_gemms:
        bench_library_gemms(a)
        return
    cfg = get_config(a.workload)
    print(f"# generating {cfg.name} inputs on the device", file=sys.stderr, flush=True)
    g = make_inputs(cfg, device=dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    # one-time layout change of the routed expert weights (outside any timing)
    packed = None
    if a.pack and lmoe.packed_bytes(sh) > 0:
        packed = lmoe.pack_experts(sh, w)
        w = lmoe.with_packed(sh, w, packed)
        torch.cuda.synchronize()
    x = g["x"]
    T = cfg.T
    y = torch.empty((T, cfg.H), dtype=x.dtype, device=dev)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    ws = lmoe.alloc_workspace(sh, dev)

    print(f"# timing {a.steps} steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    ms, _ = timed_loop(lmoe, sh, w, x, y, idx, tw, ws, a.steps, a.warmup, per_stage=False)
    # per-stage times from events recorded between the launches (separate pass)
    ms_ev, stages = timed_loop(lmoe, sh, w, x, y, idx, tw, ws, a.steps, 1, per_stage=True)
    touched = int(torch.unique(idx).numel())

    proj = not cfg.identity_proj
    flops = lmoe.layer_flops(sh, projections=proj)
    tflops = flops / (ms * 1e-3) / 1e12
    tok_s = T / (ms * 1e-3)

    # dominant kernel: expert gate/value GEMM.  Algorithmic bytes per launch =
    # the gate and value weights of the touched experts (one expert's unit is
    # 2 * I * L elements); the latent rows it reads and the SiTU-GLU
    # activations it writes are intermediates, reported beside the roofline.
    es = 2 if cfg.act == "bf16" else 4
    gv_bytes = lmoe.expert_bytes(sh, touched, "gv")
    gv_inter = T * cfg.L * es + T * cfg.k * cfg.I * es
    gv_ms = stages["expert_gate_value"]
    gv_gbs = gv_bytes / (gv_ms * 1e-3) / 1e9
    dn_bytes = lmoe.expert_bytes(sh, touched, "down")
    layer_bytes = lmoe.expert_bytes(sh, touched) + lmoe.dense_bytes(sh, projections=proj) + 2 * T * cfg.H * es
    clock = {"mhz_mean_over_xcds": None, "error": "skipped (--no-clock)"} if a.no_clock else \
        sample_clock(lambda: lmoe.forward(sh, w, x, y, idx, tw, ws))

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.w_expert == "bf16" else cfg.w_expert,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, K3 layer shape)",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "L": cfg.L, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "S": cfg.S, "Is": cfg.Is, "act": cfg.act, "w_expert": cfg.w_expert,
                   "expert_act": "f8 (1x128 scales)" if cfg.a8 else cfg.act,
                   "expert_weights": "packed" if packed is not None else "row-major",
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "layer_hbm_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
        "experts_touched": touched,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stages_sum_ms": round(sum(stages.values()), 4),
        "roofline": {
            "kernel": "expert gate/value grouped GEMM + SiTU-GLU",
            "bound": "hbm",
            "achieved": round(gv_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gv_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(cfg.name, "expert_gate_value"),
            "bytes_per_launch": gv_bytes,
            "bytes_unit": "gate + value weights of one touched expert, 2*I*L*%d B" % (1 if cfg.w_expert == "f8" else es),
            "units_per_launch": touched,
            "avg_ms": round(gv_ms, 4),
            "intermediate_bytes": gv_inter,
            "intermediates": "latent rows read once (T*L) + SiTU-GLU activations written once (T*k*I), not in "
                             "achieved",
        },
        "expert_down": {"avg_ms": round(stages["expert_down"], 4), "weight_bytes": dn_bytes,
                        "gbs": round(dn_bytes / (stages["expert_down"] * 1e-3) / 1e9, 1),
                        "frac": round(dn_bytes / (stages["expert_down"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "gpu_clock": clock,
    }

    if not a.no_decode:
        dcfg = get_config(a.decode_workload)
        dsh = lmoe.shape_of(dcfg)
        dx = make_x(dcfg, dev)
        dy = torch.empty((dcfg.T, dcfg.H), dtype=dx.dtype, device=dev)
        di = torch.empty((dcfg.T, dcfg.k), dtype=torch.int32, device=dev)
        dtw = torch.empty((dcfg.T, dcfg.k), dtype=torch.float32, device=dev)
        dws = lmoe.alloc_workspace(dsh, dev)
        dms, _ = timed_loop(lmoe, dsh, w, dx, dy, di, dtw, dws, a.decode_steps, a.warmup, per_stage=False)
        _, dstages = timed_loop(lmoe, dsh, w, dx, dy, di, dtw, dws, a.decode_steps, 1, per_stage=True)
        dtouched = int(torch.unique(di).numel())
        dbytes = lmoe.expert_bytes(dsh, dtouched) + lmoe.dense_bytes(dsh) + 2 * dcfg.T * dcfg.H * es
        out["decode"] = {
            "workload": dcfg.name, "T": dcfg.T, "ms_per_step": round(dms, 4),
            "tokens_per_s": round(dcfg.T / (dms * 1e-3), 1),
            "experts_touched": dtouched, "bytes": dbytes,
            "hbm_gbs": round(dbytes / (dms * 1e-3) / 1e9, 1),
            "hbm_frac": round(dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "stages_ms": {k: round(v, 4) for k, v in dstages.items()},
        }
        del dws

    if not a.no_secondary:
        out["secondary"] = secondary_lines(a, lmoe, dev, g)

    if a.cpu_sample > 0:
        out["cpu_baseline"], out["parity"] = cpu_baseline(cfg, g, idx, y, a.cpu_sample, dev)

    print(json.dumps(out), flush=True)


def secondary_lines(a, lmoe, dev, g_bf16):
    """Two more workloads of the same layer, timed like the headline: the
    Zipf-skewed router at T=16384 (bf16 weights, bias b_e = r_e^-1.1) and e4m3
    expert weights with 128x128 block scales at T=8192 (W8A16)."""
    import torch

    from synth import get_config, make_inputs
    from synth.inputs import make_router_bias, make_x

    res = {}
    for name in ("k3_zipf_t16384", "k3_fp8_t8192"):
        cfg = get_config(name)
        print(f"# secondary: {name}", file=sys.stderr, flush=True)
        if cfg.w_expert == "bf16":
            g = dict(g_bf16)
            g["b_router"] = make_router_bias(cfg, dev)
        else:
            g = make_inputs(cfg, device=dev, with_x=False)
        x = make_x(cfg, dev)
        sh = lmoe.shape_of(cfg)
        w = lmoe.make_weights(sh, g)
        T = cfg.T
        y = torch.empty((T, cfg.H), dtype=x.dtype, device=dev)
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
        ws = lmoe.alloc_workspace(sh, dev)
        steps = max(5, a.steps // 2)
        ms, _ = timed_loop(lmoe, sh, w, x, y, idx, tw, ws, steps, min(a.warmup, 3), per_stage=False)
        _, stages = timed_loop(lmoe, sh, w, x, y, idx, tw, ws, steps, 1, per_stage=True)
        counts = torch.bincount(idx.flatten().long(), minlength=cfg.E)
        flops = lmoe.layer_flops(sh)
        res[name] = {"T": T, "steps": steps, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "w_expert": cfg.w_expert, "bias": cfg.bias,
                     "rows_per_expert": {"max": int(counts.max()), "min": int(counts.min()),
                                         "mean": round(T * cfg.k / cfg.E, 1)},
                     "stages_ms": {k: round(v, 4) for k, v in stages.items()}}
        del ws, y, idx, tw, x, w
        if cfg.w_expert != "bf16":
            g.clear()
        torch.cuda.empty_cache()
    return res


def bench_backward(a, lmoe, dev):
    """One step = one lmoe_backward call: the forward recomputed from x, then
    the fp32 gradients of sum(y * dy) for x and every weight."""
    import numpy as np
    import torch

    from synth import get_config, make_inputs

    cfg = get_config(a.workload)
    print(f"# generating {cfg.name} inputs on the device", file=sys.stderr, flush=True)
    g = make_inputs(cfg, device=dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    x = g["x"]
    T = cfg.T
    gen = torch.Generator(device=dev).manual_seed(77)
    dy = torch.randn((T, cfg.H), generator=gen, device=dev).to(torch.bfloat16)
    grads = {n: torch.empty(shp, dtype=torch.float32, device=dev) for n, shp in lmoe.grad_shapes(sh, w).items()}
    ws = torch.empty(lmoe.backward_workspace_bytes(sh), dtype=torch.uint8, device=dev)
    for _ in range(a.warmup):
        _, idx = lmoe.backward(sh, w, x, dy, grads=grads, ws=ws)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"# timing {a.steps} backward steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(a.steps):
        lmoe.backward(sh, w, x, dy, grads=grads, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(lmoe.BWD_STAGES) + 1)] for _ in range(a.steps)]
    for i in range(a.steps):
        _, idx = lmoe.backward(sh, w, x, dy, grads=grads, ws=ws, events=evs[i])
    torch.cuda.synchronize()
    stages = {n: sum(e[s].elapsed_time(e[s + 1]) for e in evs) / a.steps for s, n in enumerate(lmoe.BWD_STAGES)}
    fl = lmoe.backward_flops(sh, projections=not cfg.identity_proj, up=not cfg.identity_proj)
    total = sum(fl.values())
    tflops = total / (ms * 1e-3) / 1e12
    # the dominant stage, routed expert gradients: HBM-bound at K3 shape (the
    # fp32 gradients of every expert are written: t_HBM > t_MFMA)
    ex_s = stages["expert_grads"] * 1e-3
    ex_bytes = lmoe.backward_expert_bytes(sh)
    t_hbm = ex_bytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = fl["expert_grads"] / (PEAK_BF16_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(ex_bytes / ex_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(t_hbm / ex_s, 4), "bytes_per_launch": ex_bytes}
    else:
        roof = {"bound": "mfma", "achieved": round(fl["expert_grads"] / ex_s / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(t_mfma / ex_s, 4)}
    roof.update(flops_per_launch=fl["expert_grads"], mfma_tflops=round(fl["expert_grads"] / ex_s / 1e12, 1),
                t_hbm_ms=round(t_hbm * 1e3, 3), t_mfma_ms=round(t_mfma * 1e3, 3))
    out = {
        "metric": "latent-MoE layer backward tokens/s (forward recompute + fp32 gradients of x and every weight)",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and dy, N(0,0.02) weights, K3 layer shape)",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "L": cfg.L, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "S": cfg.S, "Is": cfg.Is, "act": cfg.act, "w_expert": cfg.w_expert, "gradients": "fp32",
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stage_gflop": {k: round(v / 1e9, 1) for k, v in fl.items()},
        "roofline": dict({"kernel": "routed expert gradient stage (grouped dgrads + wgrads)", "traffic": None,
                          "avg_ms": round(stages["expert_grads"], 4)}, **roof),
    }
    if a.cpu_sample > 0:
        out["cpu_baseline"], out["parity"] = cpu_baseline_backward(cfg, g, dy, idx, grads["dx"], a.cpu_sample, dev)
    print(json.dumps(out), flush=True)


def bench_library_gemms(a):
    """Context for the GEMM kernels' efficiency, not part of the layer: torch's
    bf16 products (hipBLASLt on ROCm) at the T=8192 K3 shapes.  Dense: route
    GEMM (x [8192, 7168] against the stacked router, W_dn and shared gate/value
    weights, 8576 rows) and up GEMM (K = 3584 + 2048, 7168 rows), weights
    [N, K] as the layer stores them.  Experts: a batched product with a
    uniform 146 rows per expert (the mean load), which the grouped GEMMs
    handle with ragged rows instead."""
    import torch
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(0)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    out = {"metric": "library bf16 GEMM times at the K3 T=8192 shapes (context)", "unit": "ms", "dense": {},
           "batched_experts": {}}
    for name, (M, K, N) in {"route": (8192, 7168, 8576), "up": (8192, 5632, 7168)}.items():
        A = torch.randn(M, K, device=dev, dtype=bf, generator=g)
        W = torch.randn(N, K, device=dev, dtype=bf, generator=g)
        ms = timed(lambda: torch.nn.functional.linear(A, W), 10)
        out["dense"][name] = {"M": M, "K": K, "N": N, "ms": round(ms, 4), "tflops": round(2 * M * K * N / ms / 1e9, 1)}
        del A, W
    for name, (E, M, K, N) in {"gate_value": (896, 146, 3584, 2048), "down": (896, 146, 1024, 3584)}.items():
        A = torch.randn(E, M, K, device=dev, dtype=bf, generator=g)
        B = torch.randn(E, K, N, device=dev, dtype=bf, generator=g)
        ms = timed(lambda: torch.bmm(A, B), 5)
        byt = E * K * N * 2 + E * M * (K + N) * 2
        out["batched_experts"][name] = {"E": E, "rows": M, "K": K, "N": N, "ms": round(ms, 4),
                                        "gbs": round(byt / ms / 1e6, 1)}
        del A, B
        torch.cuda.empty_cache()
    print(json.dumps(out))


def bench_quantile(a, lmoe, dev):
    """One step = one lmoe_quantile_bias call: the per-expert (1 - k/E)
    quantile of the batch's sigmoid scores from fp32 router logits [T, E]
    already in HBM (a skewed router: per-expert offsets of +-4)."""
    import numpy as np
    import torch

    from oracle import lmoe_oracle as O
    from synth import get_config
    from synth.inputs import make_router_logits

    cfg = get_config(a.workload)
    T, E, k = cfg.T, cfg.E, cfg.k
    lg_host = make_router_logits(T, E, seed=13, spread=4.0)
    lg = torch.from_numpy(lg_host).to(dev)
    sh = lmoe.shape_of(cfg)
    bias = torch.empty(E, dtype=torch.float32, device=dev)
    ws = lmoe.alloc_workspace(sh, dev)
    for _ in range(a.warmup):
        lmoe.quantile_bias(sh, lg, out=bias, ws=ws)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(a.steps):
        lmoe.quantile_bias(sh, lg, out=bias, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    # algorithmic bytes: the logits read once, the bias written once
    nbytes = T * E * 4 + E * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "Quantile Balancing threshold solve, tokens/s (per-expert quantile of the batch's router scores)",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0, 1.7^2) router logits with per-expert offsets of +-4)",
        "config": {"workload": f"quantile_bias_T{T}_E{E}_k{k}", "T": T, "E": E, "k": k,
                   "parallelism": "single GPU"},
        "roofline": {
            "kernel": "qb_keys_kernel + qb_select_kernel",
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
            "bytes_per_launch": nbytes,
            "avg_ms": round(ms, 5),
        },
    }
    if a.cpu_sample > 0:
        cores = len(os.sched_getaffinity(0))
        t0c = time.perf_counter()
        ref = O.quantile_bias(lg_host.astype(np.float64), k)
        dt = time.perf_counter() - t0c
        err = float(np.abs(bias.cpu().numpy().astype(np.float64) - ref).max())
        out["cpu_baseline"] = {"value": round(T / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "sample": f"the whole {T}-token batch (numpy sort per expert, fp64), {dt:.2f} s",
                               "seconds": round(dt, 3)}
        out["parity"] = {"max_abs_err": err, "tol": 1e-6, "ok": err <= 1e-6}
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(cfg, g, dy, idx, dx, n, dev):
    """The oracle's backward on a seeded sample of the batch's tokens: its dx
    rows are exact for those tokens (each token's dx depends on that token
    alone), so they double as a parity check of the GPU's dx."""
    import numpy as np
    import torch

    from oracle import lmoe_oracle as O
    from synth import raw_numpy

    cores = len(os.sched_getaffinity(0))
    rows = np.sort(np.random.default_rng(54321).choice(cfg.T, size=min(n, cfg.T), replace=False))
    rt = torch.as_tensor(rows, device=dev)
    forced = idx[rt].cpu().numpy().astype(np.int64)
    touched = sorted(set(forced.ravel().tolist()))

    class Sparse:
        """Expert stack on the host: the sample's experts, zeros elsewhere
        (the sample's gradients never read the others)."""

        def __init__(self, t):
            self.t = t
            self.cache = {e: raw_numpy(t[e]) for e in touched}

        def __len__(self):
            return self.t.shape[0]

        def __getitem__(self, e):
            e = int(e)
            if e not in self.cache:
                self.cache[e] = raw_numpy(self.t[e])
            return self.cache[e]

    inp = {}
    for k, v in g.items():
        if v is None:
            inp[k] = None
        elif k in ("w_gate", "w_value", "w_out"):
            inp[k] = Sparse(v)
        elif k == "x":
            inp[k] = raw_numpy(v[rt])
        else:
            inp[k] = raw_numpy(v)
    dy64 = O.bf16_bits_to_f64(raw_numpy(dy[rt]))
    spec = dict(act=cfg.act, w_expert=cfg.w_expert, k=cfg.k, cap=cfg.cap, eps=cfg.eps)
    print(f"# oracle backward: {len(rows)} tokens on {cores} host cores", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ref = O.backward(inp, spec, dy64, forced_idx=forced, forced_tol=1e-5)
    dt = time.perf_counter() - t0
    got = dx[rt].double().cpu().numpy()
    err = float((np.abs(got - ref["dx"]).max(1) / np.abs(ref["dx"]).max(1)).max())
    base = {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} seeded tokens of the {cfg.T}-token batch, backward (with its forward) in fp64 "
                      f"numpy, {dt:.1f} s", "seconds": round(dt, 2)}
    return base, {"rows": len(rows), "dx_max_row_rel_err": err, "tol": 2e-2, "ok": err <= 2e-2}


def cpu_baseline(cfg, g, idx, y, n, dev):
    """The fp64 oracle, as it stands, on a seeded sample of the workload's
    tokens, on this host's cores.  Its input bytes are copied to host memory
    before the clock starts; the same run gives the sampled parity check."""
    import numpy as np
    import torch

    from oracle import lmoe_oracle as O
    from synth import raw_numpy

    cores = len(os.sched_getaffinity(0))
    rows = np.sort(np.random.default_rng(12345).choice(cfg.T, size=min(n, cfg.T), replace=False))
    rt = torch.as_tensor(rows, device=dev)
    forced = idx[rt].cpu().numpy().astype(np.int64)
    touched = sorted(set(forced.ravel().tolist()))

    class Prefetched:
        """Expert stack on the host for the sample's experts; others fetched on demand."""

        def __init__(self, t):
            self.t = t
            self.cache = {e: raw_numpy(t[e]) for e in touched}

        def __len__(self):
            return self.t.shape[0]

        def __getitem__(self, e):
            e = int(e)
            if e not in self.cache:
                self.cache[e] = raw_numpy(self.t[e])
            return self.cache[e]

    print(f"# oracle: copying {len(touched)} experts to the host", file=sys.stderr, flush=True)
    inp = {}
    for k, v in g.items():
        if v is None:
            inp[k] = None
        elif k in ("w_gate", "w_value", "w_out", "s_gate", "s_value", "s_out"):
            inp[k] = Prefetched(v)
        elif k == "x":
            inp[k] = raw_numpy(v[rt])
        else:
            inp[k] = raw_numpy(v)
    spec = dict(act=cfg.act, w_expert=cfg.w_expert, k=cfg.k, cap=cfg.cap, eps=cfg.eps, a8=cfg.a8)
    print(f"# oracle: {len(rows)} tokens on {cores} host cores", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ref = O.forward(inp, spec, forced_idx=forced, forced_tol=1e-5)
    dt = time.perf_counter() - t0
    y64 = O.bf16_bits_to_f64(raw_numpy(y[rt])) if y.dtype == torch.bfloat16 else raw_numpy(y[rt]).astype(np.float64)
    err = float((np.abs(y64 - ref["y"]).max(1) / np.abs(ref["y"]).max(1)).max())
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:
        blas = "numpy default"
    base = {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} seeded tokens of the {cfg.T}-token batch (rows are independent); "
                      f"fp64 numpy ({blas}), {dt:.1f} s",
            "seconds": round(dt, 2)}
    parity = {"rows": len(rows), "max_row_rel_err": err, "tol": 6e-2 if cfg.w_expert == "f8" else 2e-2,
              "ok": err <= (6e-2 if cfg.w_expert == "f8" else 2e-2)}
    parity["selection"] = selection_stats(cfg, g, idx)
    return base, parity


def selection_stats(cfg, g, idx, gap=1e-3):
    """The GPU's top-k against the oracle's fp64 routing on every token of the
    batch (not timed): strict set mismatches over all tokens, the fraction of
    near-tie tokens (oracle k-th minus (k+1)-th biased score below `gap`),
    and the largest such gap among the mismatches."""
    import numpy as np

    from oracle import lmoe_oracle as O
    from synth import raw_numpy

    print(f"# oracle routing of all {cfg.T} tokens", file=sys.stderr, flush=True)
    r = O.route(O.decode(raw_numpy(g["x"]), cfg.act), O.decode(raw_numpy(g["w_router"]), cfg.act),
                raw_numpy(g["b_router"]).astype(np.float64), cfg.k)
    got = np.sort(idx.cpu().numpy().astype(np.int64), axis=1)
    want = np.sort(r["idx"], axis=1)
    mism = (got != want).any(axis=1)
    return {"tokens": int(cfg.T), "strict_mismatch": int(mism.sum()),
            "near_tie_frac": round(float((r["gap"] < gap).mean()), 4),
            "mismatch_outside_near_ties": int((mism & (r["gap"] >= gap)).sum()),
            "max_gap_among_mismatches": float(r["gap"][mism].max()) if mism.any() else 0.0}


if __name__ == "__main__":
    main()
