#!/usr/bin/env python3
"""Throughput of one MoE layer's forward pass (route -> dispatch -> expert FFN -> combine)
on one MI355X, on the Mixtral-shaped prefill workload (T=4096 tokens, h=4096, 8 experts,
top-2 softmax, SwiGLU inter=14336, bf16 with fp32 accumulation, fp32 router, no capacity
limit), seeded synthetic inputs resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one moe_forward call: every kernel of the layer over one batch. Prints one
JSON line. The dominant kernel (the gate/up grouped GEMM) is timed live with HIP events
that the library records on its launch stream (moe_forward_traced) in the timed region.
The CPU baseline times the fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec per MoE layer (route+dispatch+FFN+combine); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_mixtral_prefill_traffic.json")


def _ffn_source_sha():
    h = hashlib.sha256()
    for f in ("ffn.hip", "moe_internal.h"):
        with open(os.path.join(ROOT, "expert_routing_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary, when it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != _ffn_source_sha() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


CALIB_BYTES = 512 << 20   # the plain copy that scales rocprofv3's FETCH_SIZE / WRITE_SIZE


def summarize_traffic(fetch_csv, write_csv, workload="mixtral_prefill"):
    """Per-launch HBM bytes of the gate/up GEMM from two rocprofv3 --pmc runs of
    `bench.py --calibrate-copy` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by what the same counter reads for the CALIB_BYTES device copy in that run.
    Writes the JSON that bench.py reports as roofline.traffic."""
    import csv

    def per_kernel(path, counter):
        rows = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 float(r["Counter_Value"]) * 1024.0))
        rows.sort()
        first_gemm = min(d for d, n, _ in rows if "ffn_gate_up" in n)
        # the calibration copy is the last device copy before the first layer call
        copies = [v for d, n, v in rows if "copyBuffer" in n and d < first_gemm]
        vals = {"gate_up": [v for _, n, v in rows if "ffn_gate_up" in n],
                "down": [v for _, n, v in rows if "ffn_down" in n],
                "copy": copies[-1:]}
        return {k: (sum(x) / len(x) if x else None) for k, x in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = f["copy"] / CALIB_BYTES
    w_scale = w["copy"] / CALIB_BYTES
    out = {
        "workload": workload,
        "source_sha": _ffn_source_sha(),
        "calibration": {"copy_bytes": CALIB_BYTES, "fetch_counter_bytes": f["copy"],
                        "write_counter_bytes": w["copy"], "fetch_scale": f_scale,
                        "write_scale": w_scale},
        "gate_up": {"fetch_bytes": f["gate_up"] / f_scale, "write_bytes": w["gate_up"] / w_scale},
        "down": {"fetch_bytes": f["down"] / f_scale, "write_bytes": w["down"] / w_scale},
    }
    out["hbm_bytes_per_launch"] = out["gate_up"]["fetch_bytes"] + out["gate_up"]["write_bytes"]
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(cfg, inp, n_tokens, min_seconds=10.0):
    """The fp64 oracle, untuned, on the first n_tokens tokens of the same workload, called
    repeatedly until at least min_seconds of CPU time have passed."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    sub = cfg.with_(T=n_tokens)
    host = {"T": n_tokens, "x": inp["x"][:n_tokens].cpu(), "w_router": inp["w_router"].cpu(),
            "bias": None if inp["bias"] is None else inp["bias"].cpu(),
            "w13": inp["w13"].cpu(), "w2": inp["w2"].cpu(),
            "w13_sh": None if inp["w13_sh"] is None else inp["w13_sh"].cpu(),
            "w2_sh": None if inp["w2_sh"] is None else inp["w2_sh"].cpu()}
    runs, dt = 0, 0.0
    while runs == 0 or dt < min_seconds:   # whole calls, at least min_seconds of CPU work
        t0 = time.perf_counter()
        out = oracle.forward(sub, host)
        dt += time.perf_counter() - t0
        runs += 1
        assert np.isfinite(out["y"]).all()
    del host
    torch.cuda.empty_cache()
    return {"value": runs * n_tokens / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 3), "calls": runs,
            "sample": f"oracle.forward (fp64 numpy) on the first {n_tokens} of {cfg.T} tokens of "
                      f"the same workload, {runs} call(s): routing, dispatch, all {cfg.E_local} "
                      f"experts' SwiGLU FFN on their rows, combine"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the CPU-oracle sample (0: the whole workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one device copy of a known size (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--materialize-xp", action="store_true",
                    help="pass xp, so dispatch copies rows into it (default: no xp; the "
                         "gate/up GEMM reads x through row_src)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, workload=args.workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this build runs one MoE layer on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. Multi-GPU expert parallelism is "
              "design-only here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import expert_routing_amd as moe
    from synth import CONFIGS, make_inputs

    torch.cuda.set_device(0)
    cfg = CONFIGS[args.workload]
    inp = make_inputs(cfg, device="cuda")
    p = moe.problem_from_config(cfg)
    b = moe.alloc_buffers(p, "cuda")
    t = dict(b)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=inp["w13"],
             w2=inp["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"])
    gather = not args.materialize_xp
    if gather:
        t["xp"] = None
    npts = len(moe.TRACE_POINTS)
    ev = moe.HipEvents(npts * args.steps)

    if args.calibrate_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        moe.moe_forward(p, t, b["ws"])
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        moe.moe_forward_traced(p, t, b["ws"], ev.handles[i * npts:(i + 1) * npts])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps

    stage_ms = {name: 0.0 for name in moe.TRACE_POINTS[1:]}
    for i in range(args.steps):
        for j in range(1, npts):
            stage_ms[moe.TRACE_POINTS[j]] += ev.elapsed(i * npts + j - 1, i * npts + j) / args.steps
    ev.close()

    # Work actually done this step (the layout is deterministic, so any step's).
    offsets = b["offsets"].cpu().numpy()
    counts = b["counts"].cpu().numpy()
    R = int(offsets[-1])
    sh = (cfg.T // cfg.n_ep) if cfg.n_shared else 0
    s = cfg.act_bytes
    T, h, E, K, I = cfg.T, cfg.h, cfg.E, cfg.K, cfg.inter
    active = int((np.diff(offsets) > 0).sum())
    gate_up_flops = 4.0 * R * h * I + 4.0 * sh * h * cfg.shared_inter
    down_flops = 2.0 * R * I * h + 2.0 * sh * cfg.shared_inter * h
    route_bytes = T * h * s + E * h * 4 + T * K * 8
    # gathered: dispatch only builds the layout (ids in; dest_row, row_src, counts out) and
    # the rows travel inside the gate/up GEMM's A loads
    dispatch_bytes = (8 * T * K + 4 * R) if gather else (T * h * s + R * h * s + 12 * T * K)
    combine_bytes = R * h * s + T * h * s + 8 * T * K + sh * h * s
    gu = stage_ms["ffn_gate_up"] * 1e-3
    achieved = gate_up_flops / gu / 1e12
    traffic = _traffic(args.workload)

    result = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "h": h, "E": E, "K": K, "inter": I,
                   "score": cfg.score, "capacity_factor": cfg.capacity_factor,
                   "n_ep": cfg.n_ep, "n_shared": cfg.n_shared, "router": "fp32",
                   "xp": "gathered by the gate/up GEMM" if gather else "materialised"},
        "roofline": {"kernel": "ffn_gemm_bf16 gate/up (fused silu*mul)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "flops_per_launch": gate_up_flops,
                     "avg_launch_ms": stage_ms["ffn_gate_up"]},
        "routed_pairs_per_s": (T * K - int(b["n_dropped"].item())) / (ms * 1e-3),
        "layer_tflops": (gate_up_flops + down_flops) / (ms * 1e-3) / 1e12,
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "stage_rates": {
            "route_GBps": route_bytes / (stage_ms["route"] * 1e-3) / 1e9,
            "dispatch_GBps": dispatch_bytes / (stage_ms["dispatch"] * 1e-3) / 1e9,
            "gate_up_TFLOPs": achieved,
            "down_TFLOPs": down_flops / (stage_ms["ffn_down"] * 1e-3) / 1e12,
            "combine_GBps": combine_bytes / (stage_ms["combine"] * 1e-3) / 1e9,
        },
        "layout": {"rows": R, "active_local_experts": active,
                   "balancedness": float(counts.mean() / max(counts.max(), 1)),
                   "dropped": int(b["n_dropped"].item())},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_tokens or T, T))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
