"""Benchmark of absorbed MLA decode on one MI355X.

One step = one mla_decode call (the split decode kernel, then the LSE
combine) over the measured batch: 32 sequences x 4096 cached tokens,
128 heads, a bf16 latent cache of 576-wide rows in 64-token paged blocks.
The split plan is built once per batch shape before timing (the pages build
this metadata once per batch, vLLM MLA page "MLA의 MQA 디코딩 경로").

Prints one JSON line: latent-cache GB/s over the whole step, plus
  roofline      the decode kernel's algorithmic cache bytes per launch over
                its average launch time (HIP events around back-to-back
                launches on the launch stream), against MI355X's 8 TB/s HBM
                peak; "traffic" is the measured HBM bytes per launch from the
                FETCH_SIZE / WRITE_SIZE counter summary, when that summary was
                taken on the current kernel source;
  cpu_baseline  the CPU oracle timed on the same batch on this host's cores.
Inputs are resident in HBM before timing; 4 replicas of the cache pool are
rotated so no step finds its pool in the 256 MB last-level (MALL) cache.

  --copy-calibration  also runs a plain 256 MiB device copy (for scaling the
                      HBM byte counters of a profiler run of this command);
  --summarize-counters FETCH_CSV WRITE_CSV
                      turns the counter CSVs of two `rocprofv3 --pmc` runs of
                      this command (FETCH_SIZE, then WRITE_SIZE) into
                      profiles/decode_bf16_traffic.json and exits.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
COPY_BYTES = 256 << 20          # calibration copy size
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "decode_bf16_traffic.json")
DECODE_KERNEL = "decode_bf16_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    return ap.parse_args()


def kernel_sha() -> str:
    import hashlib
    src = os.path.join(ROOT, "mla_latent_kv_07_amd", "csrc", "decode_bf16.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def summarize_counters(fetch_csv: str, write_csv: str) -> None:
    """Per-dispatch HBM bytes of the decode kernel from two counter runs.

    Each counter is scaled by what it reads for the 256 MiB calibration copy
    (which moves exactly COPY_BYTES in and COPY_BYTES out)."""
    import csv

    def per_kernel(path, counter):
        dec, cpy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0          # KiB -> bytes
            if DECODE_KERNEL in r["Kernel_Name"]:
                dec.append(v)
            elif r["Kernel_Name"].startswith(COPY_KERNEL) and v > COPY_BYTES / 8:
                cpy.append(v)
        assert dec and cpy, f"{path}: no {counter} rows for the decode kernel and the copy"
        return sum(dec) / len(dec), sum(cpy) / len(cpy), len(dec)

    f_dec, f_cpy, n_f = per_kernel(fetch_csv, "FETCH_SIZE")
    w_dec, w_cpy, n_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / f_cpy, COPY_BYTES / w_cpy
    read_b, write_b = f_dec * f_scale, w_dec * w_scale
    out = {
        "kernel": DECODE_KERNEL,
        "workload": "v2_decode_b32_s4096_bf16",
        "kernel_source_sha": kernel_sha(),
        "dispatches": {"fetch_run": n_f, "write_run": n_w},
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter_bytes": f_cpy,
                             "write_counter_bytes": w_cpy, "fetch_scale": f_scale,
                             "write_scale": w_scale},
        "raw_counter_bytes_per_launch": {"fetch": f_dec, "write": w_dec},
        "read_bytes_per_launch": read_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": read_b + write_b,
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(d, cache_bytes):
    """The oracle, as it stands, on the whole batch (all 32 sequences x 128
    heads x 4096 tokens, ~1-3 s on the host's cores), in latent-cache bytes
    per second."""
    import numpy as np
    import oracle as O

    B, n_h = d.wl.B, d.wl.n_h
    rows = np.arange(B * n_h, dtype=np.int64)
    O.decode(d.cache.pool, O.FMT_BF16, d.cache.block_table, d.cache.seq_lens, d.q_lat.double(),
             d.q_rope.double(), d.scale, rows=rows[:n_h // 8])   # warm up (load, page in)
    t0 = time.perf_counter()
    O.decode(d.cache.pool, O.FMT_BF16, d.cache.block_table, d.cache.seq_lens, d.q_lat.double(),
             d.q_rope.double(), d.scale, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(cache_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": O.threads(),
            "kind": "oracle",
            "sample": f"{B} of {B} sequences (all {n_h} heads x 4096 tokens), {dt:.2f} s"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_kv_07_amd import _lib as L
    from mla_latent_kv_07_amd import api
    from mla_latent_kv_07_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = I.C2
    d = I.make_decode_inputs(wl)
    cache_bytes = d.cache.cache_bytes                      # 150,994,944 B of valid rows
    S = int(d.cache.seq_lens[0])
    flops = 2 * wl.B * wl.n_h * S * (wl.d_c + wl.d_r + wl.d_c)   # score (576) + value (512) MACs

    pools = [api.DeviceCache.from_host(d.cache, dev) for _ in range(args.replicas)]
    bt = d.cache.block_table.to(dev)
    sl = d.cache.seq_lens.to(dev)
    ql, qr = d.q_lat.to(dev), d.q_rope.to(dev)
    dec = api.Decoder(d.cache.seq_lens, wl.q_len, wl.n_h, wl.d_c, wl.d_r, wl.kv_dtype, dev)
    o_lat = torch.empty((wl.B, wl.n_h, wl.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.B, wl.n_h), dtype=torch.float32, device=dev)

    # pre-marshalled arguments: the host must stay ahead of the GPU
    lib = L.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    descs = [p.desc() for p in pools]
    ws_bytes = dec.workspace.numel()
    call_args = [(P(ql.data_ptr()), P(qr.data_ptr()), L.DT_BF16, ctypes.byref(descs[r]),
                  P(bt.data_ptr()), bt.stride(0), P(sl.data_ptr()), wl.B, wl.q_len, wl.n_h,
                  ctypes.c_float(d.scale), ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()),
                  P(dec.workspace.data_ptr()), ws_bytes, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
                 for r in range(args.replicas)]
    fin_args = (ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()), P(dec.workspace.data_ptr()),
                ws_bytes, L.DT_BF16, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
    full, part, fin = lib.mla_decode, lib.mla_decode_partial, lib.mla_decode_finish
    R = args.replicas

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for i in range(args.warmup):
        L.check(full(*call_args[i % R]))
    torch.cuda.synchronize()

    # ---- timed steps: K whole decode calls, bracketed by synchronizations
    K = args.steps
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    bad = 0
    for i in range(K):
        bad |= full(*call_args[i % R])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    L.check(bad)
    ms_per_step = wall * 1e3 / K
    gpu_ms = e0.elapsed_time(e1) / K

    # ---- per-kernel launch durations: back-to-back launches of each phase
    def timed(fn, argsets, n):
        a, b = ev(), ev()
        a.record(stream)
        st = 0
        for i in range(n):
            st |= fn(*argsets[i % len(argsets)])
        b.record(stream)
        torch.cuda.synchronize()
        L.check(st)
        return a.elapsed_time(b) / n

    n_leg = max(K, 50)
    dec_ms = timed(part, call_args, n_leg)
    comb_ms = timed(fin, [fin_args], n_leg)

    # ---- per-call distribution of the whole call (events around each call)
    pairs = [(ev(), ev()) for _ in range(n_leg)]
    st = 0
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        st |= full(*call_args[i % R])
        b.record(stream)
    torch.cuda.synchronize()
    L.check(st)
    call_us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    pct = lambda q: round(call_us[min(len(call_us) - 1, int(q * len(call_us)))], 2)

    copy_gbs = None
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(5):
            dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        copy_gbs = round(2 * COPY_BYTES / (a.elapsed_time(b) / 5 * 1e-3) / 1e9, 1)
        del src, dst

    value = cache_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = cache_bytes / (dec_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_JSON):
        t = json.load(open(TRAFFIC_JSON))
        if t.get("kernel_source_sha") == kernel_sha():
            traffic = round(t["bytes_per_launch"])

    out = {
        "metric": "MLA decode latent-cache GB/s + TFLOP/s, B=32 S=4096 bf16, % of roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "seq_len": S, "q_len": wl.q_len, "n_h": wl.n_h,
                   "d_c": wl.d_c, "d_r": wl.d_r, "kv_dtype": wl.kv_dtype, "block_size": 64,
                   "cache_bytes": cache_bytes, "pool_replicas": R,
                   "work_items": dec.info.num_items, "splits_per_seq": dec.info.max_splits},
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "call_us": {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)},
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "combine_kernel_us": round(comb_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": DECODE_KERNEL,
                     "algorithmic_bytes": cache_bytes,
                     "mfma_tflops": round(flops / (dec_ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops / (dec_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if copy_gbs is not None:
        out["copy_calibration_gbs"] = copy_gbs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, cache_bytes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
