"""bench.py's host-side arithmetic and contract, on the CPU: the algorithmic
FLOP count, the roofline bound and fraction for each kind of decode kernel,
the counter summary's calibration scaling, the traffic guard on the kernel
source, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys
from pathlib import Path
from types import SimpleNamespace

import pytest
import torch

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_visible_flops_closed_form():
    # q_len 1: every row sees all S positions; 2 (d_c + d_r + d_c) FLOP each
    assert bench.visible_flops(torch.tensor([4096] * 32), 1, 128, 512, 64) == 2.0 * 128 * 32 * 4096 * 1088
    # q_len 2: the first query token sees S - 1 positions, the second S; an
    # empty sequence and one shorter than the pair add (almost) nothing
    assert bench.visible_flops(torch.tensor([10, 0, 1]), 2, 4, 8, 2) == 2.0 * 4 * (9 + 10 + 1) * 18


def test_roofline_bounds_and_fractions():
    wl = SimpleNamespace()
    nbytes, ms = 150994944, 0.05
    flops = bench.visible_flops(torch.tensor([4096] * 32), 1, 128, 512, 64)
    r = bench.roofline(wl, bench.DECODE_KERNEL, ms, nbytes, flops, None)
    # 241.8 FLOP/B is below the bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312.5): HBM
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(nbytes / (ms * 1e-3) / 1e9, abs=0.1)
    assert r["frac"] == pytest.approx(nbytes / (ms * 1e-3) / 8e12, abs=1e-4)
    assert r["flop_per_byte"] == pytest.approx(241.8, abs=0.05)
    # the 8-bit kernel at 870 FLOP/B is past the fp8 ridge (625): MFMA
    r8 = bench.roofline(wl, bench.DECODE_KERNEL_FP8, 0.2, 193379200, 1.683e11, None)
    assert r8["bound"] == "mfma" and r8["peak"] == 5000.0 and r8["unit"] == "TFLOP/s"
    assert r8["frac"] == pytest.approx(1.683e11 / 0.2e-3 / 5e15, abs=1e-4)
    # the generic kernel is priced against the fp32 vector ALU
    rg = bench.roofline(wl, "decode_generic_kernel", 1.0, 1e6, 1e12, None)
    assert rg["bound"] == "alu" and rg["peak"] == 157.3


def test_decode_kernel_names():
    mk = lambda kv, qd="bf16", dc=512, dr=64: SimpleNamespace(kv_dtype=kv, q_dtype=qd, d_c=dc, d_r=dr)
    assert bench.decode_kernel_name(mk("bf16")) == "decode_mfma_kernel<mla::kv::Bf16>"
    assert bench.decode_kernel_name(mk("fp8_e4m3")) == "decode_f8w8_kernel"
    assert bench.decode_kernel_name(mk("bf16", dc=64)) == "decode_generic_kernel"
    assert bench.decode_kernel_name(mk("f32")) == "decode_generic_kernel"


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, kib in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy moves COPY_BYTES each way; FETCH_SIZE reads half of it (scale
    # 2), WRITE_SIZE all of it (scale 1); the decode's counters are averaged
    # over its dispatches and scaled the same way
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(bench.COPY_KERNEL, copy_kib / 2), (bench.DECODE_KERNEL + "(args)", 1000.0),
                                       (bench.DECODE_KERNEL + "(args)", 1200.0), ("other_kernel", 5e6)])
    _counter_csv(write, "WRITE_SIZE", [(bench.COPY_KERNEL, copy_kib), (bench.DECODE_KERNEL + "(args)", 300.0)])
    out_json = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out_json))
    bench.summarize_counters(str(fetch), str(write))
    t = json.load(open(out_json))
    assert t["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert t["read_bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2)
    assert t["write_bytes_per_launch"] == pytest.approx(300.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx(1100.0 * 2048 + 300.0 * 1024)
    assert t["kernel_source_sha"] == bench.kernel_sha()


def test_traffic_is_reported_only_for_the_summarised_source(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(p))
    w = "v2_decode_b32_s4096_bf16"
    json.dump({"kernel_source_sha": bench.kernel_sha(), "workload": w, "bytes_per_launch": 1234.4}, open(p, "w"))
    assert bench.traffic_for(bench.DECODE_KERNEL, w) == 1234
    assert bench.traffic_for(bench.DECODE_KERNEL, "other_workload") is None
    assert bench.traffic_for(bench.DECODE_KERNEL_FP8, w) is None
    json.dump({"kernel_source_sha": "0" * 16, "workload": w, "bytes_per_launch": 1.0}, open(p, "w"))
    assert bench.traffic_for(bench.DECODE_KERNEL, w) is None
    os.remove(p)
    assert bench.traffic_for(bench.DECODE_KERNEL, w) is None
