#!/usr/bin/env python3
"""Throughput of one MoE layer's forward pass (route -> dispatch -> expert FFN -> combine)
on one MI355X, seeded synthetic inputs resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu-baseline]
                    [--dtype bf16|mxfp8] [--weights packed|rows]

Default workload: the Mixtral-shaped prefill layer (T=4096 tokens, h=4096, 8 experts, top-2
softmax, SwiGLU inter=14336, bf16 with fp32 accumulation, fp32 router, no capacity limit).
`--workload all` prints one JSON line per workload (Mixtral prefill, DeepSeek-V3 EP=8 share,
Zipf-skewed with and without capacity, DeepSeek-V3 decode).

A step is one moe_forward call: every kernel of the layer over one batch. `value` is the
steady-state rate of K back-to-back steps. Stage times come from HIP events the library
records on its own launch stream between the stages (moe_forward_traced), minus the
measured cost of an empty event pair (`event_pair_us`; an event record occupies the GPU for
a few microseconds); `stages_traced_us` keeps the raw values. The traced steps are run again
with the caches flushed before each one (a 1 GiB buffer is written, which evicts the 4 MB
L2s and the 256 MB Infinity Cache), outside the stage events; `flushed` reports those stage
times and the per-stage rates against the HBM / MFMA rooflines. The CPU baseline times
the fp64 oracle on the same workload; its routing result also gives the near-tie count and
the first-choice skew.

bf16 expert weights are packed once before timing into the MFMA-fragment order the GEMMs
stream straight into registers (moe_pack_weights, a permutation done at load time, like
any kernel-specific weight layout); `--weights rows` times the row-major layout instead.
`--dtype mxfp8` runs the same workload with MX-FP8 expert weights (E4M3 codes and E8M0
block scales, quantised once on the GPU before timing): x is quantised per token inside
the step, both GEMMs run on the FP8 matrix cores, and their rates are taken against the
dense fp8 MFMA peak.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec per MoE layer (route+dispatch+FFN+combine); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the MX-FP8 GEMMs)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
NUM_XCD = 8                 # MI355X: 8 XCDs of 32 CUs (GRBM_GUI_ACTIVE sums over them)
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
ALL = ["mixtral_prefill", "dsv3_ep8", "skew_cap1", "skew_nodrop", "dsv3_decode"]
FLUSH_BYTES = 1 << 30       # written before each flushed step: > L2 (8 x 4 MB) + 256 MB MALL
CALIB_BYTES = 512 << 20     # the plain copy that scales rocprofv3's FETCH_SIZE / WRITE_SIZE
PROFILES = os.path.join(ROOT, "profiles")

# kernel name prefix -> stage of the layer
STAGE_OF = [("router_", "route"), ("select_", "route"), ("logits_", "route"),
            ("disp_", "dispatch"), ("mx_quant", "dispatch"), ("ffn_prep", "ffn_prep"),
            ("ffn_split", "ffn_prep"), ("ffn_gate_up", "ffn_gate_up"),
            ("ffn_down", "ffn_down"), ("combine", "combine")]


def kernel_source_sha():
    """Hash of every HIP source and header the library is built from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "expert_routing_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "moe.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def load_traffic(workload):
    """Per-stage HBM bytes per launch from the committed rocprofv3 counter summary, when it
    was taken on the current kernel sources; else None."""
    try:
        with open(traffic_file(workload)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_sha() or t.get("workload") != workload:
        return None
    return t.get("stages")


def kernel_base_name(kernel_name):
    """The kernel's own name: return type, namespaces and argument list stripped."""
    n = kernel_name[5:] if kernel_name.startswith("void ") else kernel_name
    n = n.replace("moe::(anonymous namespace)::", "").replace("moe::", "")
    return n.split("(", 1)[0]


def stage_of(kernel_name):
    n = kernel_base_name(kernel_name)
    for prefix, stage in STAGE_OF:
        if n.startswith(prefix):
            return stage
    return None


def summarize_traffic(fetch_csv, write_csv, workload):
    """HBM bytes per layer call of every stage from two rocprofv3 --pmc runs of
    `bench.py --calibrate-copy --no-flush` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
    each scaled by what the same counter reads for the CALIB_BYTES device copy in that run.
    Layer calls are counted as the combine kernel's launches (one per call). Writes
    profiles/traffic_<workload>.json."""
    import csv

    def per_stage(path, counter):
        rows = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 float(r["Counter_Value"]) * 1024.0))
        rows.sort()
        # the layer calls start at the first router kernel; earlier library kernels (the
        # MX-FP8 weights' one-time quantisation) and the calibration copy come before
        first = min(d for d, n, _ in rows if stage_of(n) == "route")
        copies = [v for d, n, v in rows if "copyBuffer" in n and d < first]
        tot, kern = {}, {}
        calls = 0
        for d, n, v in rows:
            s = stage_of(n)
            if s is None or d < first:
                continue
            calls += s == "combine"
            tot[s] = tot.get(s, 0.0) + v
            kern.setdefault(kernel_base_name(n), []).append(v)
        return ({s: v / max(calls, 1) for s, v in tot.items()}, copies[-1],
                {k: sum(v) / len(v) for k, v in kern.items()}, calls)

    f, fcopy, fk, calls = per_stage(fetch_csv, "FETCH_SIZE")
    w, wcopy, wk, wcalls = per_stage(write_csv, "WRITE_SIZE")
    assert calls == wcalls and calls > 0, (calls, wcalls)
    fs, ws_ = fcopy / CALIB_BYTES, wcopy / CALIB_BYTES
    out = {
        "workload": workload,
        "source_sha": kernel_source_sha(),
        "layer_calls_per_run": calls,
        "calibration": {"copy_bytes": CALIB_BYTES, "fetch_counter_bytes": fcopy,
                        "write_counter_bytes": wcopy, "fetch_scale": fs, "write_scale": ws_},
        "stages": {s: {"fetch_bytes": f.get(s, 0.0) / fs, "write_bytes": w.get(s, 0.0) / ws_}
                   for s in sorted(set(f) | set(w))},
        "kernels_per_launch": {k: {"fetch_bytes": fk.get(k, 0.0) / fs,
                                   "write_bytes": wk.get(k, 0.0) / ws_}
                               for k in sorted(set(fk) | set(wk))},
    }
    with open(traffic_file(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


PROFILE_SQ = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE "
              "SQ_LDS_BANK_CONFLICT SQ_WAVE_CYCLES SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE")


def summarize_profile(kt_trace_csv, kt_bench_log, sq_csv, workload, dtype, suffix):
    """profiles/<workload>_<dtype>.md from three rocprofv3 runs of this script: the kernel
    trace (--kernel-trace --stats; its kernel_trace.csv and the bench line the profiled run
    printed), and the MFMA / LDS counters of the two GEMMs (PROFILE_SQ, one --pmc run);
    the HBM traffic table comes from profiles/traffic_<workload><suffix>.json
    (--summarize-traffic on the same source)."""
    import csv

    args = f"--workload {workload} --dtype {dtype} --no-cpu-baseline --no-flush"
    cmds = [
        f"rocprofv3 --kernel-trace --stats -f csv -d <out>/kt -o kt -- python3 <repo>/bench.py "
        f"{args} --steps 10 --warmup 3",
        f"rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o fetch -- python3 <repo>/bench.py "
        f"{args} --steps 2 --warmup 1 --calibrate-copy",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o write -- python3 <repo>/bench.py "
        f"{args} --steps 2 --warmup 1 --calibrate-copy",
        f"rocprofv3 --pmc {PROFILE_SQ} --kernel-include-regex \"ffn_gate_up|ffn_down\" -f csv "
        f"-d <out>/sq -o sq -- python3 <repo>/bench.py {args} --steps 2 --warmup 1",
        f"python3 <repo>/bench.py --summarize-traffic <out>/fetch/fetch_counter_collection.csv "
        f"<out>/write/write_counter_collection.csv --workload {workload} --dtype {dtype}",
        f"python3 <repo>/bench.py --summarize-profile <out>/kt/kt_kernel_trace.csv "
        f"<kernel-trace run's stdout> <out>/sq/sq_counter_collection.csv --workload {workload} "
        f"--dtype {dtype}",
    ]
    # per-dispatch durations from the first router kernel on (the MX-FP8 weights' one-time
    # quantisation and the input generation come before the layer calls)
    disp = []
    with open(kt_trace_csv) as fh:
        for r in csv.DictReader(fh):
            if stage_of(r["Kernel_Name"]) is not None:
                disp.append((int(r["Dispatch_Id"]), kernel_base_name(r["Kernel_Name"]),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    first = min(d for d, n, _ in disp if stage_of(n) == "route")
    per = {}
    for d, n, us in disp:
        if d >= first:
            per.setdefault(n, []).append(us)
    kern = [(n, len(v), sum(v) / len(v), min(v), max(v)) for n, v in per.items()]
    kern.sort(key=lambda k: -k[1] * k[2])
    mean_us = {k[0]: k[2] for k in kern}
    line = None
    with open(kt_bench_log) as fh:
        for ln in fh:
            if ln.startswith("{"):
                line = json.loads(ln)
    sq = {}
    with open(sq_csv) as fh:
        for r in csv.DictReader(fh):
            n = kernel_base_name(r["Kernel_Name"])
            sq.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    calls = max((k[1] for k in kern if stage_of(k[0]) == "combine"), default=0)
    out = [f"# Kernel times and counters: {workload} ({dtype})", "",
           "Commands (GPU box, from the repository root; output directory of your choice;",
           "`cd /tmp && export TMPDIR=/tmp` first):", "", "```", *cmds, "```", ""]
    out.append("The bench passes no xp (dispatch builds only the layout; the gate/up GEMM reads "
               "x through row_src); " + ("the expert weights are MX-FP8, quantised once before "
                                         "timing (quantize_mx, omitted below)." if dtype == "mxfp8"
                                         else "bf16 expert weights are packed once before timing "
                                         "(pack_weights, omitted below)."))
    out.append(f"The kernel-trace run makes {calls} layer calls (3 warm-up, 10 timed, 10 traced). "
               "Library kernels of the layer calls (from the first router launch on):")
    out += ["", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    out += [f"| {n} | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} |" for n, c, a, lo, hi in kern]
    if line:
        out += ["", "bench.py's own HIP-event stage times in the same profiled process (us, "
                f"event-pair overhead of {line['event_pair_us']} us removed): "
                f"{json.dumps(line['stages_us'])}; ms_per_step {line['ms_per_step']:.4f}, "
                f"value {line['value']:.4g} tokens/s.",
                f"Roofline object ({line['roofline']['kernel'].split(' (')[0]}): achieved "
                f"{line['roofline']['achieved']:.1f} {line['roofline']['unit']} of "
                f"{line['roofline']['peak']} ({line['roofline']['frac']:.3f})."]
    out += ["", "## MFMA and LDS counters (per launch, averaged over the run's launches)", "",
            "| kernel | GRBM_GUI_ACTIVE (sum of 8 XCDs) | SQ_VALU_MFMA_BUSY_CYCLES | MFMA busy "
            "fraction | SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE | clock under load (GHz) |",
            "|---|---|---|---|---|---|"]
    for n in sorted(sq):
        c = {k: sum(v) / len(v) for k, v in sq[n].items()}
        grbm, busy = c.get("GRBM_GUI_ACTIVE", 0.0), c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        frac = busy / (1024 * grbm / NUM_XCD) if grbm else 0.0
        conf = (c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"]
                if c.get("SQ_LDS_IDX_ACTIVE") else 0.0)
        ghz = grbm / NUM_XCD / (mean_us[n] * 1e3) if n in mean_us and mean_us[n] else 0.0
        out.append(f"| {n} | {grbm:.4g} | {busy:.4g} | {frac:.3f} | {conf:.3f} | {ghz:.2f} |")
    out += ["", "MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / "
            "8 XCDs); the clock is GRBM_GUI_ACTIVE / 8 over the kernel's mean trace duration."]
    try:
        with open(traffic_file(workload + suffix)) as fh:
            t = json.load(fh)
    except OSError:
        t = None
    if t:
        cal = t["calibration"]
        out += ["", "## HBM traffic per layer call (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled)", "",
                f"Each counter is scaled by its reading for a {cal['copy_bytes'] >> 20} MiB "
                f"device copy in the same run: FETCH_SIZE reads {cal['fetch_scale']:.4f} of the "
                f"copy's bytes, WRITE_SIZE {cal['write_scale']:.4f}. Layer calls per run: "
                f"{t['layer_calls_per_run']}. Source hash: {t['source_sha']} (bench.py reports "
                "roofline.traffic only while it matches).", "",
                "| stage | fetched (MB) | written (MB) |", "|---|---|---|"]
        out += [f"| {s} | {v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} |"
                for s, v in sorted(t["stages"].items())]
    path = os.path.join(PROFILES, f"{workload}_{dtype}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("wrote", path)


def measure_peaks(torch, reps=20):
    """Practical ceilings of this GPU, for context beside the published peaks the roofline
    fractions use: a plain bf16 GEMM through torch.matmul (hipBLASLt) at the Mixtral gate/up
    shape (all 8192 routed rows against one 28672 x 4096 weight), the same GEMM per 1024-row
    expert, and a 1 GiB device-to-device copy. Medians of `reps` runs, each timed with HIP
    events."""
    dev = "cuda"

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        fn()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2] * 1e-3   # s

    out = {}
    g = torch.Generator(device=dev).manual_seed(0)
    for name, M in (("gemm_8192x28672x4096", 8192), ("gemm_1024x28672x4096", 1024)):
        a = torch.randn(M, 4096, device=dev, dtype=torch.bfloat16, generator=g)
        w = torch.randn(4096, 28672, device=dev, dtype=torch.bfloat16, generator=g)
        t = timed(lambda: torch.matmul(a, w))
        out[name] = {"TFLOPs": 2.0 * M * 28672 * 4096 / t / 1e12,
                     "frac_of_published": 2.0 * M * 28672 * 4096 / t / 1e12 / PEAK_BF16_TFLOPS}
        del a, w
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src))
    out["copy_1GiB"] = {"GBps": 2.0 * (1 << 30) / t / 1e9,
                        "frac_of_published": 2.0 * (1 << 30) / t / 1e9 / PEAK_HBM_GBS}
    del src, dst
    return {"practical_peaks": out, "published": {"bf16_TFLOPs": PEAK_BF16_TFLOPS,
                                                   "hbm_GBps": PEAK_HBM_GBS}}


def cpu_baseline(cfg, inp, ids_gpu, min_seconds=10.0):
    """The fp64 oracle, untuned, on the whole workload, called repeatedly until at least
    min_seconds have passed; its routing also gives the near-tie count, the number of
    tokens whose GPU expert set differs, and the first-choice load skew."""
    import numpy as np
    import torch

    import oracle
    from oracle import volumes as V
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    host = {"T": cfg.T, "x": inp["x"].cpu(), "w_router": inp["w_router"].cpu(),
            "bias": None if inp["bias"] is None else inp["bias"].cpu(),
            "w13": inp["w13"].cpu(), "w2": inp["w2"].cpu(),
            "w13_sh": None if inp["w13_sh"] is None else inp["w13_sh"].cpu(),
            "w2_sh": None if inp["w2_sh"] is None else inp["w2_sh"].cpu()}
    runs, dt, out = 0, 0.0, None
    while runs == 0 or dt < min_seconds:   # whole calls, at least min_seconds of CPU work
        t0 = time.perf_counter()
        out = oracle.forward(cfg, host)
        dt += time.perf_counter() - t0
        runs += 1
        assert np.isfinite(out["y"]).all()
    rr = out["route"]
    near = (rr.kth_gap < 1e-4) | (rr.group_gap < 1e-4)
    diff = (ids_gpu != rr.ids).any(axis=1)
    first = rr.keys.argmax(axis=1) if cfg.n_groups == 1 else None
    check = {"near_tie_tokens": int(near.sum()),
             "gpu_id_mismatch_tokens": int(diff.sum()),
             "gpu_id_mismatch_off_near_tie": int((diff & ~near).sum())}
    if first is not None:
        check["first_choice_peak_to_mean"] = V.peak_to_mean(np.bincount(first, minlength=cfg.E))
    del host
    torch.cuda.empty_cache()
    return ({"value": runs * cfg.T / dt, "unit": "tokens/s", "cores": int(cores),
             "kind": "oracle", "seconds": round(dt, 3), "calls": runs,
             "sample": f"oracle.forward (fp64 numpy) on all {cfg.T} tokens of the same "
                       f"workload, {runs} call(s): routing, dispatch, the SwiGLU FFN of all "
                       f"{cfg.E_local} local experts on their rows, combine"}, check)


def stage_work(cfg, R, active, gather, mx=False):
    """Algorithmic bytes and flops of each stage of one layer call (what the method must
    move: each operand read once, each result written once). With MX-FP8 weights an
    operand element of the GEMMs is one byte plus a scale byte per 32."""
    s = cfg.act_bytes
    if mx:
        return stage_work_mx(cfg, R, active)
    T, h, E, K, I = cfg.T, cfg.h, cfg.E, cfg.K, cfg.inter
    sh = (T // cfg.n_ep) if cfg.n_shared else 0
    Is = cfg.shared_inter
    n_sh = 1 if cfg.n_shared else 0
    w = {
        "route": {"bytes": T * h * s + E * h * 4 + T * K * 8, "flops": 2.0 * T * h * E},
        # gathered: dispatch moves only the layout (ids in; dest_row, row_src, counts out)
        # and the token rows travel inside the gate/up GEMM's A loads
        "dispatch": {"bytes": (8 * T * K + 4 * R + 4 * E) if gather
                     else (T * h * s + R * h * s + 12 * T * K), "flops": 0.0},
        "ffn_gate_up": {"bytes": 2 * I * h * s * active + 2 * Is * h * s * n_sh
                        + R * h * s + sh * h * s
                        + R * I * s + sh * Is * s,
                        "flops": 4.0 * R * h * I + 4.0 * sh * h * Is},
        "ffn_down": {"bytes": I * h * s * active + Is * h * s * n_sh + R * I * s + sh * Is * s
                     + R * h * s + sh * h * s,
                     "flops": 2.0 * R * I * h + 2.0 * sh * Is * h},
        "combine": {"bytes": R * h * s + T * h * s + 8 * T * K + sh * h * s, "flops": 0.0},
    }
    return w


def stage_work_mx(cfg, R, active):
    T, h, E, K, I = cfg.T, cfg.h, cfg.E, cfg.K, cfg.inter
    sh = (T // cfg.n_ep) if cfg.n_shared else 0
    Is = cfg.shared_inter
    n_sh = 1 if cfg.n_shared else 0
    q = 33 / 32    # E4M3 byte + its share of the block's scale byte
    return {
        "route": {"bytes": T * h * 2 + E * h * 4 + T * K * 8, "flops": 2.0 * T * h * E},
        # per-token quantisation of x (bf16 in, codes and scales out) and the layout
        "dispatch": {"bytes": T * h * 2 + T * h * q + 8 * T * K + 4 * R + 4 * E, "flops": 0.0},
        "ffn_gate_up": {"bytes": (2 * I * h * active + 2 * Is * h * n_sh + R * h + sh * h
                                  + R * I + sh * Is) * q,
                        "flops": 4.0 * R * h * I + 4.0 * sh * h * Is},
        "ffn_down": {"bytes": (I * h * active + Is * h * n_sh + R * I + sh * Is) * q
                     + (R * h + sh * h) * 2,
                     "flops": 2.0 * R * I * h + 2.0 * sh * Is * h},
        "combine": {"bytes": R * h * 2 + T * h * 2 + 8 * T * K + sh * h * 2, "flops": 0.0},
    }


def rate(work, ms, bound=None, mfma_peak=PEAK_BF16_TFLOPS):
    """Achieved GB/s and TFLOP/s of a stage, and its roofline fraction: against HBM when its
    arithmetic intensity is below the ridge of `mfma_peak`, else against that peak (the
    GEMMs: the dtype's dense MFMA peak; the router: route_bound's)."""
    sec = ms * 1e-3
    gbs = work["bytes"] / sec / 1e9
    tfs = work["flops"] / sec / 1e12
    if bound is None:
        ai = work["flops"] / max(work["bytes"], 1)
        bound = "mfma" if ai > mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "hbm":
        frac = gbs / PEAK_HBM_GBS
    else:
        frac = tfs / mfma_peak
    return {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "TFLOPs": round(tfs, 2),
            "bound": bound, "frac": round(frac, 4)}


# The router's logits are fp32-exact: with bf16 activations the fp32 weight enters as three
# bf16 planes, so one algorithmic multiply-add costs three bf16 MFMA ones; with fp32
# activations it runs on the fp32 vector units.
PEAK_ROUTER_MFMA_TFLOPS = PEAK_BF16_TFLOPS / 3


def route_bound(cfg):
    """(bound, peak TFLOP/s) of the router: its compute peak once its flops outweigh its
    bytes there, else HBM."""
    ai = 2.0 * cfg.T * cfg.h * cfg.E / (cfg.T * cfg.h * cfg.act_bytes + cfg.E * cfg.h * 4)
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_ROUTER_MFMA_TFLOPS
    if ai > peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        return ("f32" if cfg.dtype == "f32" else "mfma"), peak
    return "hbm", peak


def variant_suffix(args, workload_dtype):
    """Suffix of a workload's traffic summary: none for the default bf16 run (packed
    weights), _rows for row-major bf16 weights, _mxfp8 for MX-FP8."""
    if args.dtype == "mxfp8":
        return "_mxfp8"
    return "_rows" if workload_dtype == "bf16" and args.weights == "rows" else ""


def run_workload(name, args, moe, torch, np):
    from synth import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    mx = args.dtype == "mxfp8"
    pk = not mx and cfg.dtype == "bf16" and args.weights == "packed"
    inp = make_inputs(cfg, device="cuda")
    p = moe.problem_from_config(cfg)
    if mx:
        p.act_dtype = moe.DTYPE["mxfp8"]
    if pk:
        p.act_dtype = moe.DTYPE["bf16_packed"]
    b = moe.alloc_buffers(p, "cuda")
    t = dict(b)
    t.update(x=inp["x"], w_router=inp["w_router"], bias=inp["bias"], w13=inp["w13"],
             w2=inp["w2"], w13_sh=inp["w13_sh"], w2_sh=inp["w2_sh"])
    if mx:
        # the weights as E4M3 codes and block scales, quantised once before timing
        for k in ("w13", "w2", "w13_sh", "w2_sh"):
            w = inp[k]
            if w is None:
                t[k + "_scale"] = None
                continue
            c, sc = moe.quantize_mx(w.reshape(-1, w.shape[-1]))
            t[k] = c.reshape(w.shape)
            t[k + "_scale"] = sc.reshape(w.shape[:-1] + (w.shape[-1] // 32,))
        torch.cuda.synchronize()
    if pk:
        # the weights in the packed fragment order, once before timing
        for k in ("w13", "w2", "w13_sh", "w2_sh"):
            if inp[k] is not None:
                t[k] = moe.pack_weights(inp[k])
        torch.cuda.synchronize()
    gather = not args.materialize_xp
    if gather:
        t["xp"] = None
    pts = moe.TRACE_POINTS
    npts = len(pts)
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

    def stage_means():
        out = {n: 0.0 for n in pts[1:]}
        for i in range(args.steps):
            for j in range(1, npts):
                out[pts[j]] += ev.elapsed(i * npts + j - 1, i * npts + j) / args.steps
        return out

    # steady state: K back-to-back untraced steps (the headline rate)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        moe.moe_forward(p, t, b["ws"])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(stop) / args.steps

    # the same steps with HIP events between the stages (recorded by the library on its
    # launch stream); each event record itself occupies the GPU for a few microseconds
    for i in range(args.steps):
        moe.moe_forward_traced(p, t, b["ws"], ev.handles[i * npts:(i + 1) * npts])
    torch.cuda.synchronize()
    steady = stage_means()
    # cost of one event pair with nothing between: measured, then taken off each stage
    pairs = moe.HipEvents(2 * args.steps)
    for i in range(args.steps):
        pairs.record(2 * i)
        pairs.record(2 * i + 1)
    torch.cuda.synchronize()
    overhead = sorted(pairs.elapsed(2 * i, 2 * i + 1) for i in range(args.steps))[args.steps // 2]
    pairs.close()

    def net(st):
        return {k: max(v - overhead, 0.0) for k, v in st.items()}

    # flushed: each step starts with cold L2 and Infinity Cache
    flushed = None
    if not args.no_flush:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        for i in range(args.steps):
            flush.fill_(i & 0xff)
            moe.moe_forward_traced(p, t, b["ws"], ev.handles[i * npts:(i + 1) * npts])
        torch.cuda.synchronize()
        flushed = stage_means()
        del flush
    ev.close()

    # work actually done (the layout is deterministic, so any step's)
    offsets = b["offsets"].cpu().numpy()
    counts = b["counts"].cpu().numpy().astype(np.float64)
    R = int(offsets[-1])
    active = int((np.diff(offsets) > 0).sum())
    dropped = int(b["n_dropped"].item())
    work = stage_work(cfg, R, active, gather, mx)
    T, K = cfg.T, cfg.K
    gu = work["ffn_gate_up"]
    mfma_peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    gu_bound = "mfma" if gu["flops"] / gu["bytes"] > mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9) \
        else "hbm"
    traffic = load_traffic(name + variant_suffix(args, cfg.dtype))
    gu_ms = net(steady)["ffn_gate_up"]
    kname = ("ffn_gate_up_mxfp8 (grouped gate/up GEMM on scaled FP8 MFMA, fused silu*mul "
             "and MX quantisation)" if mx else
             "ffn_gate_up_pk (grouped gate/up GEMM on packed bf16 weights, fused silu*mul)"
             if pk else "ffn_gate_up_bf16 (grouped gate/up GEMM, fused silu*mul)")
    if gu_bound == "mfma":
        achieved = gu["flops"] / (gu_ms * 1e-3) / 1e12
        roof = {"kernel": kname, "bound": "mfma", "achieved": achieved, "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": achieved / mfma_peak}
    else:
        achieved = gu["bytes"] / (gu_ms * 1e-3) / 1e9
        roof = {"kernel": kname, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof.update({"traffic": (traffic["ffn_gate_up"]["fetch_bytes"]
                             + traffic["ffn_gate_up"]["write_bytes"]) if traffic else None,
                 "algorithmic_flops": gu["flops"], "algorithmic_bytes": gu["bytes"],
                 "avg_launch_ms": gu_ms})

    def stage_rates(st):
        r = {}
        rb, rpeak = route_bound(cfg)
        for sname in ("route", "dispatch", "ffn_gate_up", "ffn_down", "combine"):
            r[sname] = rate(work[sname], st[sname],
                            rb if sname == "route" else
                            ("hbm" if sname in ("dispatch", "combine") else None),
                            mfma_peak=rpeak if sname == "route" else mfma_peak)
        r["ffn_prep"] = {"us": round(st["ffn_prep"] * 1e3, 2)}   # 0: built by dispatch
        # route + dispatch + prep + combine against their summed roofline times
        rdc_t = st["route"] + st["dispatch"] + st["ffn_prep"] + st["combine"]
        roof_t = 0.0
        for sname in ("route", "dispatch", "combine"):
            wk = work[sname]
            peak_f = rpeak if sname == "route" else PEAK_BF16_TFLOPS
            roof_t += max(wk["bytes"] / (PEAK_HBM_GBS * 1e9), wk["flops"] / (peak_f * 1e12))
        r["route_dispatch_combine"] = {"us": round(rdc_t * 1e3, 2),
                                       "roofline_us": round(roof_t * 1e6, 2),
                                       "frac": round(roof_t * 1e3 / rdc_t, 4)}
        return r

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
        "dtype": "mxfp8" if mx else ("bf16" if cfg.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "h": cfg.h, "E": cfg.E, "K": K,
                   "inter": cfg.inter, "score": cfg.score, "n_groups": cfg.n_groups,
                   "topk_groups": cfg.topk_groups, "capacity_factor": cfg.capacity_factor,
                   "n_ep": cfg.n_ep, "n_shared": cfg.n_shared, "router": "fp32",
                   "xp": "gathered by the gate/up GEMM" if gather else "materialised",
                   "expert_weights": ("MX-FP8, quantised before timing" if mx else
                                      "packed fragment order, packed before timing" if pk
                                      else "row-major")},
        "roofline": roof,
        "routed_pairs_per_s": (T * K - dropped) / (ms * 1e-3),
        "layer_tflops": (gu["flops"] + work["ffn_down"]["flops"]) / (ms * 1e-3) / 1e12,
        "event_pair_us": round(overhead * 1e3, 2),
        "stages_traced_us": {k: round(v * 1e3, 2) for k, v in steady.items()},
        "stages_us": {k: round(v * 1e3, 2) for k, v in net(steady).items()},
        "stage_rates": stage_rates(net(steady)),
        "flushed": None if flushed is None else {
            "ms_per_step": sum(net(flushed).values()),
            "stages_traced_us": {k: round(v * 1e3, 2) for k, v in flushed.items()},
            "stages_us": {k: round(v * 1e3, 2) for k, v in net(flushed).items()},
            "stage_rates": stage_rates(net(flushed))},
        "layout": {"rows": R, "active_local_experts": active, "dropped": dropped,
                   "balancedness": float(counts.mean() / max(counts.max(), 1)),
                   "peak_to_mean": float(counts.max() / max(counts.mean(), 1e-30)),
                   "idle_experts": int((counts == 0).sum())},
        "wall_s_timed": round(wall, 4),
    }
    if cfg.bias == "zipf":
        # popularity law of the bias alone: E / H_{E,s}
        H = sum(r ** -cfg.zipf_s for r in range(1, cfg.E + 1))
        result["layout"]["zipf_popularity_peak_to_mean"] = cfg.E / H
    if cfg.T % cfg.n_ep == 0 and b["send_bytes"] is not None and cfg.n_ep > 1:
        sb = b["send_bytes"].cpu().numpy()
        result["layout"]["send_bytes_row_sum_mean"] = float(sb.sum(1).mean())
        result["layout"]["send_zero_pair_fraction"] = float((sb == 0).mean())
    if not args.no_cpu_baseline and not mx:
        ids = b["topk_ids"].cpu().numpy()
        result["cpu_baseline"], result["routing_check"] = cpu_baseline(cfg, inp, ids)
    else:
        result["cpu_baseline"] = None
    del b, t, inp
    torch.cuda.empty_cache()
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill",
                    help="a workload name, or 'all' for one line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cache-flushed repetition of the timed steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one device copy of a known size (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the practical-ceiling measurement added to a one-workload line")
    ap.add_argument("--measure-peaks", action="store_true",
                    help="print one JSON line of this GPU's practical ceilings (a hipBLASLt "
                         "bf16 GEMM, a device copy) and exit")
    ap.add_argument("--summarize-profile", nargs=3,
                    metavar=("KERNEL_TRACE_CSV", "BENCH_LOG", "SQ_CSV"))
    ap.add_argument("--dtype", choices=["bf16", "mxfp8"], default="bf16",
                    help="expert weights and GEMM operands: bf16 (the workloads' dtype), or "
                         "MX-FP8 (E4M3 with E8M0 block scales; activations stay bf16)")
    ap.add_argument("--weights", choices=["packed", "rows"], default="packed",
                    help="bf16 expert weights in the packed fragment order (packed once "
                         "before timing) or row-major")
    ap.add_argument("--materialize-xp", action="store_true",
                    help="pass xp, so dispatch copies rows into it (default: no xp; the "
                         "gate/up GEMM reads x through row_src)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic,
                          workload=args.workload + variant_suffix(args, "bf16"))
        return
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, workload=args.workload, dtype=args.dtype,
                          suffix=variant_suffix(args, "bf16"))
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

    torch.cuda.set_device(0)
    if args.measure_peaks:
        print(json.dumps(measure_peaks(torch)), flush=True)
        return
    if args.workload == "all":
        for name in ALL:
            print(json.dumps(run_workload(name, args, moe, torch, np)), flush=True)
        return
    line = run_workload(args.workload, args, moe, torch, np)
    if not args.no_peaks:
        # context measured after the timed steps, on the same GPU: what a plain hipBLASLt
        # GEMM and a device copy reach here (the fractions stay against the published peaks)
        line["practical_peaks"] = measure_peaks(torch)["practical_peaks"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
