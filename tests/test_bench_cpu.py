"""Host logic of bench.py, on the CPU: the kernel -> stage map, the rocprofv3 summaries
(traffic per layer call scaled by the calibration copy, the profile tables) on small
hand-made counter files, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# one layer call: a calibration copy first, then route, dispatch, table, GEMMs, combine
KERNELS = [
    ("void at::native::copyBuffer(char*)", None),
    ("void moe::(anonymous namespace)::router_small_e<true>(unsigned short const*)", "route"),
    ("void moe::(anonymous namespace)::disp_place(int const*)", "dispatch"),
    ("moe::(anonymous namespace)::ffn_split(moe::FfnPrepArgs)", "ffn_prep"),
    ("void moe::(anonymous namespace)::ffn_gate_up_pk<256, 256, 1, 4, false>(int)", "ffn_gate_up"),
    ("void moe::(anonymous namespace)::ffn_down_pk<256, 256, 1, 4, false>(int)", "ffn_down"),
    ("void moe::(anonymous namespace)::combine_kernel<true>(uint4 const*)", "combine"),
]


def test_stage_map():
    for name, stage in KERNELS:
        assert bench.stage_of(name) == stage, name
    assert bench.kernel_base_name(KERNELS[4][0]) == "ffn_gate_up_pk<256, 256, 1, 4, false>"
    assert bench.stage_of("void moe::(anonymous namespace)::select_topk<4>(float const*)") == "route"
    assert bench.stage_of("void moe::(anonymous namespace)::mx_quant_rows<true>(void const*)") \
        == "dispatch"


def _counter_csv(path, counter, values, calls=2):
    """rocprofv3 --pmc layout: one row per dispatch; values in KiB; the copy comes first."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        d = 1
        w.writerow({"Dispatch_Id": d, "Kernel_Name": KERNELS[0][0], "Counter_Name": counter,
                    "Counter_Value": values[None]})
        for _ in range(calls):
            for name, stage in KERNELS[1:]:
                d += 1
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": values[stage]})


def test_summarize_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kib = bench.CALIB_BYTES / 1024
    # FETCH_SIZE reads half the copy's bytes, WRITE_SIZE all of them: both scale back to bytes
    fetch = {None: kib / 2, "route": 100.0, "dispatch": 1.0, "ffn_prep": 0.5,
             "ffn_gate_up": 4000.0, "ffn_down": 2000.0, "combine": 300.0}
    write = {None: kib, "route": 0.0, "dispatch": 2.0, "ffn_prep": 0.0, "ffn_gate_up": 50.0,
             "ffn_down": 25.0, "combine": 100.0}
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl")
    t = json.load(open(tmp_path / "traffic_wl.json"))
    assert t["layer_calls_per_run"] == 2
    assert t["calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert t["calibration"]["write_scale"] == pytest.approx(1.0)
    for stage in ("route", "dispatch", "ffn_prep", "ffn_gate_up", "ffn_down", "combine"):
        assert t["stages"][stage]["fetch_bytes"] == pytest.approx(fetch[stage] * 1024 / 0.5)
        assert t["stages"][stage]["write_bytes"] == pytest.approx(write[stage] * 1024)
    # the summary counts only while the sources hash to what it was taken on
    assert bench.load_traffic("wl") == t["stages"]
    t["source_sha"] = "0" * 16
    json.dump(t, open(tmp_path / "traffic_wl.json", "w"))
    assert bench.load_traffic("wl") is None


def test_summarize_profile_tables(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    # kernel trace: the calibration copy, then two layer calls (ns timestamps)
    with open(tmp_path / "kt.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        d, t0 = 0, 1000
        for call in range(2):
            for name, stage in KERNELS if call == 0 else KERNELS[1:]:
                d += 1
                dur = 2000 if stage == "ffn_gate_up" else 1000 + 10 * d
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Start_Timestamp": t0,
                            "End_Timestamp": t0 + dur})
                t0 += dur
    line = {"event_pair_us": 5.0, "stages_us": {"route": 1.0}, "ms_per_step": 2.5,
            "value": 1.6e6, "roofline": {"kernel": "ffn_gate_up_pk (x)", "achieved": 1250.0,
                                         "unit": "TFLOP/s", "peak": 2500.0, "frac": 0.5}}
    (tmp_path / "kt.log").write_text("noise\n" + json.dumps(line) + "\n")
    # MFMA counters of the gate/up GEMM: GRBM over 8 XCDs, busy over 1024 SIMDs
    with open(tmp_path / "sq.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for c, v in (("GRBM_GUI_ACTIVE", 8 * 3200.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1600.0),
                     ("SQ_LDS_IDX_ACTIVE", 100.0), ("SQ_LDS_BANK_CONFLICT", 5.0)):
            w.writerow({"Kernel_Name": KERNELS[4][0], "Counter_Name": c, "Counter_Value": v})
    bench.summarize_profile(str(tmp_path / "kt.csv"), str(tmp_path / "kt.log"),
                            str(tmp_path / "sq.csv"), "wl", "bf16", "")
    md = (tmp_path / "wl_bf16.md").read_text()
    rows = [r for r in md.splitlines() if r.startswith("| ffn_gate_up_pk")]
    # trace: 2 calls of 2 us; counters: busy 0.5, conflicts 0.05, 3200 cycles / 2 us = 1.6 GHz
    assert rows[0] == "| ffn_gate_up_pk<256, 256, 1, 4, false> | 2 | 2.00 | 2.00 | 2.00 |"
    assert rows[1].endswith("| 0.500 | 0.050 | 1.60 |")
    assert "copyBuffer" not in md and "value 1.6e+06 tokens/s" in md


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
