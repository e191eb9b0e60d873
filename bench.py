"""Benchmark of absorbed MLA decode on one MI355X.

One step = one mla_decode call (the split decode kernel, then the LSE
combine) over the measured batch: 32 sequences x 4096 cached tokens,
128 heads, a bf16 latent cache of 576-wide rows in 64-token paged blocks.
The split plan is built once per batch shape before timing (the pages build
this metadata once per batch, vLLM MLA page "MLA의 MQA 디코딩 경로").

Prints one JSON line: latent-cache GB/s over the whole step, plus
  roofline      the decode kernel's algorithmic cache bytes per launch over
                its average launch time (HIP events on the launch stream),
                against MI355X's 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle timed on the same batch on this host's cores.
Inputs are resident in HBM before timing; 4 replicas of the cache pool are
rotated so no step finds its pool in the 256 MB last-level (MALL) cache.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "profiles", "decode_bf16_traffic.json"))
    return ap.parse_args()


def cpu_baseline(d, cache_bytes):
    """The oracle, as it stands, on the whole batch (all 32 sequences x 128
    heads x 4096 tokens, ~1-3 s on the host's cores), in latent-cache bytes
    per second."""
    import numpy as np
    import oracle as O

    B, n_h = d.wl.B, d.wl.n_h
    n_seq = B
    rows = np.arange(n_seq * n_h, dtype=np.int64)
    O.decode(d.cache.pool, O.FMT_BF16, d.cache.block_table, d.cache.seq_lens, d.q_lat.double(),
             d.q_rope.double(), d.scale, rows=rows[:n_h // 8])   # warm up (load, page in)
    t0 = time.perf_counter()
    O.decode(d.cache.pool, O.FMT_BF16, d.cache.block_table, d.cache.seq_lens, d.q_lat.double(),
             d.q_rope.double(), d.scale, rows=rows)
    dt = time.perf_counter() - t0
    full = dt * B / n_seq
    return {"value": round(cache_bytes / full / 1e9, 4), "unit": "GB/s", "cores": O.threads(),
            "kind": "oracle",
            "sample": f"{n_seq} of {B} sequences (all {n_h} heads x 4096 tokens), {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path has no "
              "multi-GPU mode in this build", file=sys.stderr)
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

    # pre-marshalled arguments: the host must stay ahead of ~30 us steps
    lib = L.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    descs = [p.desc() for p in pools]
    ws_bytes = dec.workspace.numel()
    part_args = [(P(ql.data_ptr()), P(qr.data_ptr()), L.DT_BF16, ctypes.byref(descs[r]),
                  P(bt.data_ptr()), bt.stride(0), P(sl.data_ptr()), wl.B, wl.q_len, wl.n_h,
                  ctypes.c_float(d.scale), ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()),
                  P(dec.workspace.data_ptr()), ws_bytes, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
                 for r in range(args.replicas)]
    fin_args = (ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()), P(dec.workspace.data_ptr()),
                ws_bytes, L.DT_BF16, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
    part, fin = lib.mla_decode_partial, lib.mla_decode_finish

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = part(*part_args[i % args.replicas])
        if ev is not None:
            ev[1].record(stream)
        st |= fin(*fin_args)
        if ev is not None:
            ev[2].record(stream)
        return st

    for i in range(args.warmup):
        L.check(step(i))
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bad = 0
    for i in range(K):
        bad |= step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    L.check(bad)

    dec_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    comb_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    gpu_ms = evs[0][0].elapsed_time(evs[-1][2]) / K
    ms_per_step = wall * 1e3 / K
    value = cache_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = cache_bytes / (dec_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(args.traffic_json):
        t = json.load(open(args.traffic_json))
        if t.get("kernel_source_sha") == _kernel_sha():
            traffic = t.get("bytes_per_launch")

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
                   "cache_bytes": cache_bytes, "pool_replicas": args.replicas,
                   "work_items": dec.info.num_items, "splits_per_seq": dec.info.max_splits},
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "combine_kernel_us": round(comb_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "mfma_tflops": round(flops / (dec_ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops / (dec_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, cache_bytes)
    print(json.dumps(out), flush=True)


def _kernel_sha() -> str:
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_kv_07_amd", "csrc",
                       "decode_bf16.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
