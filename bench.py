"""Benchmark of absorbed MLA decode on one MI355X.

One step = one mla_decode call (the split decode kernel, then the LSE
combine) over the measured batch: 32 sequences x 4096 cached tokens,
128 heads, a bf16 latent cache of 576-wide rows in 64-token paged blocks.
The split plan is built once per batch shape before timing (the pages build
this metadata once per batch, vLLM MLA page "MLA의 MQA 디코딩 경로").

Prints one JSON line: latent-cache GB/s over the whole step, plus
  roofline      the decode kernel's algorithmic cache bytes per launch over
                its average launch time in the timed steps (start / stop
                events stamped from the kernel's own dispatch on the launch
                stream, mla_set_launch_events), against MI355X's 8 TB/s HBM
                peak; "traffic" is the measured HBM bytes per launch from the
                FETCH_SIZE / WRITE_SIZE counter summary, when that summary was
                taken on the current kernel source;
  cpu_baseline  the CPU oracle timed on the same batch on this host's cores.
Inputs are resident in HBM before timing; 4 replicas of the cache pool are
rotated so no step finds its pool in the 256 MB last-level (MALL) cache.

  --workload NAME     another workload of the same path: the long-context
                      batch, the fp8 cache with speculative query pairs, or
                      the whole absorbed layer (absorb_q -> decode ->
                      absorb_out); one JSON line of the same form;
  --copy-calibration  also runs a plain 256 MiB device copy (for scaling the
                      HBM byte counters of a profiler run of this command);
  --summarize-counters FETCH_CSV WRITE_CSV
                      turns the counter CSVs of two `rocprofv3 --pmc` runs of
                      this command (FETCH_SIZE, then WRITE_SIZE) into
                      profiles/decode_mfma_bf16_traffic.json and exits.
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
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA peak
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector peak
COPY_BYTES = 256 << 20          # calibration copy size
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "decode_mfma_bf16_traffic.json")
DECODE_KERNEL = "decode_mfma_kernel<mla::kv::Bf16>"       # bf16 cache
DECODE_KERNEL_FP8 = "decode_f8w8_kernel"    # e4m3 cache on the 8-bit MFMAs
MFMA_KERNELS = {"bf16": DECODE_KERNEL, "fp8_e4m3": DECODE_KERNEL_FP8,
                "f16": "decode_mfma_kernel<mla::kv::F16>",
                "fp8_e5m2": "decode_mfma_kernel<mla::kv::E5m2>",
                "fp8_e4m3_row": "decode_mfma_kernel<mla::kv::E4m3Row>"}
KV_DTYPE_LABEL = {"bf16": "bf16", "f32": "f32", "f16": "f16", "fp8_e4m3": "fp8_e4m3+bf16",
                  "fp8_e5m2": "fp8_e5m2+bf16", "fp8_e4m3_row": "fp8_e4m3"}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=0,
                    help="cache pool replicas rotated per call (default: enough for >= 512 MB)")
    ap.add_argument("--workload", default="v2_decode_b32_s4096_bf16",
                    choices=["v2_decode_b32_s4096_bf16", "long_ctx_b4_s64k_128k_bf16",
                             "fp8_cache_spec2_b64", "full_layer_b128_bf16", "decode_step_b128_bf16",
                             "f16_decode_b32_s4096", "fp8_e5m2_spec2_b64", "fp8_e4m3_row_spec2_b64"],
                    help="the measured batch (default) or one of the other parity workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    return ap.parse_args()


def kernel_sha() -> str:
    import hashlib
    src = os.path.join(ROOT, "mla_latent_kv_07_amd", "csrc", "decode_mfma.hip")
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


def cpu_baseline(d, cache_bytes, max_rows=4096):
    """The oracle, as it stands, on a bounded sample of the workload's query
    rows (all of them for the measured batch: 32 sequences x 128 heads x 4096
    tokens, ~1-3 s on the host's cores), scaled to latent-cache bytes per
    second of the whole batch."""
    import numpy as np
    import oracle as O

    wl = d.wl
    fmt = {"f32": O.FMT_F32, "bf16": O.FMT_BF16, "fp8_e4m3": O.FMT_FP8_E4M3, "f16": O.FMT_F16,
           "fp8_e5m2": O.FMT_FP8_E5M2, "fp8_e4m3_row": O.FMT_FP8_E4M3_ROW}[wl.kv_dtype]
    n_rows = wl.B * wl.q_len * wl.n_h
    rows = np.arange(n_rows, dtype=np.int64)
    if n_rows > max_rows:
        rows = np.sort(np.random.default_rng(0).choice(n_rows, size=max_rows, replace=False))

    def run(r):
        O.decode(d.cache.pool, fmt, d.cache.block_table, d.cache.seq_lens, d.q_lat.double(),
                 d.q_rope.double(), d.scale, q_len=wl.q_len, block_scales=d.cache.block_scales, rows=r)

    run(rows[:max(1, wl.n_h // 8)])   # warm up (load, page in)
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    full = dt * n_rows / rows.size
    out = {"value": round(cache_bytes / full / 1e9, 4), "unit": "GB/s", "cores": O.threads(),
           "kind": "oracle",
           "sample": f"{rows.size} of {n_rows} query rows ({dt:.2f} s), scaled to the whole batch",
           "cpu_model": cpu_model()}
    if wl.kv_dtype in ("bf16", "f16", "f32"):
        out["fast_cpu_context"] = torch_cpu_context(d, cache_bytes, O)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def torch_cpu_context(d, cache_bytes, O, max_seqs=8):
    """Context line, not a baseline: the same decode in plain torch fp32 on
    the host's cores (matmul, softmax, matmul per sequence over its gathered
    latent rows), on the first max_seqs sequences, scaled to the batch."""
    import numpy as np
    import torch as T
    wl = d.wl
    fmt = {"f32": O.FMT_F32, "bf16": O.FMT_BF16, "f16": O.FMT_F16}[wl.kv_dtype]
    nb = min(max_seqs, wl.B)
    S_max = int(d.cache.seq_lens[:nb].max())
    raw = O.gather(d.cache.pool, fmt, wl.d_c, wl.d_r, d.cache.block_table[:nb], d.cache.seq_lens[:nb], S_max)
    dt_np = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[wl.kv_dtype]
    rows = raw.view(dt_np).reshape(nb, S_max, wl.d_c + wl.d_r)
    if wl.kv_dtype == "bf16":
        kv = T.from_numpy(rows.astype(np.uint32) << 16).view(T.float32)
    else:
        kv = T.from_numpy(rows.astype(np.float32))
    T.set_num_threads(O.threads())
    q = T.cat([d.q_lat.float(), d.q_rope.float()], dim=-1).view(wl.B, wl.q_len * wl.n_h, -1)
    def run():
        for b in range(nb):
            S = int(d.cache.seq_lens[b])
            k = kv[b, :S]
            s = (q[b] @ k.T) * d.scale
            o = T.softmax(s, dim=-1) @ k[:, :wl.d_c]
        return o
    run()
    t0 = time.perf_counter()
    run()
    dt = time.perf_counter() - t0
    tokens = float(d.cache.seq_lens[:nb].sum())
    full = dt * float(d.cache.seq_lens.sum()) / tokens
    return {"value": round(cache_bytes / full / 1e9, 4), "unit": "GB/s", "kind": "torch fp32 matmul/softmax",
            "sample": f"{nb} of {wl.B} sequences ({dt:.2f} s), scaled to the whole batch (no causal mask)"}


def visible_flops(seq_lens, q_len, n_h, d_c, d_r) -> float:
    """Algorithmic decode FLOPs: 2 (d_c + d_R + d_c) per (query row, visible token)."""
    vis = sum(int(S) - q_len + t + 1 for S in seq_lens.tolist() for t in range(q_len)
              if int(S) - q_len + t + 1 > 0)
    return 2.0 * n_h * vis * (d_c + d_r + d_c)


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
    from mla_latent_kv_07_amd import inputs as I

    torch.cuda.set_device(torch.device("cuda:0"))
    if args.workload == "decode_step_b128_bf16":
        # the full-layer shapes, from hidden states: query production and the
        # cache append take the place of the drawn queries
        out = run_layer(args, I.C5, producers=True)
    elif args.workload in I.FORMAT_WORKLOADS:
        out = run_decode(args, I.FORMAT_WORKLOADS[args.workload])
    elif I.WORKLOADS[args.workload].d_model:
        out = run_layer(args, I.WORKLOADS[args.workload])
    else:
        out = run_decode(args, I.WORKLOADS[args.workload])
    print(json.dumps(out), flush=True)


class Timer:
    """HIP events on the launch stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def legs(self, fn, argsets, n, check):
        """Average time of n back-to-back launches (ms)."""
        a, b = self.ev(), self.ev()
        a.record(self.stream)
        st = 0
        for i in range(n):
            st |= fn(*argsets[i % len(argsets)])
        b.record(self.stream)
        self.torch.cuda.synchronize()
        check(st)
        return a.elapsed_time(b) / n

    def steps(self, step, K, check):
        """K steps between two synchronizations: (wall ms, event ms) per step."""
        e0, e1 = self.ev(), self.ev()
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        st = 0
        for i in range(K):
            st |= step(i)
        e1.record(self.stream)
        self.torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        check(st)
        return wall * 1e3 / K, e0.elapsed_time(e1) / K

    def kernel_steps(self, lib, step, n_k, K, check):
        """K steps between two events; before each step the next n_k kernel
        launches of the library are given start / stop events stamped from
        their own dispatch.  Returns (wall ms per step, event ms per step,
        [mean ms of launch j of a step])."""
        evs = [[self.ev() for _ in range(2 * n_k)] for _ in range(K)]
        for e in (x for row in evs for x in row):   # create the HIP events
            e.record(self.stream)
        handles = [(ctypes.c_void_p * (2 * n_k))(*[e.cuda_event for e in row]) for row in evs]
        e0, e1 = self.ev(), self.ev()
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        st = 0
        for i in range(K):
            st |= lib.mla_set_launch_events(handles[i], n_k)
            st |= step(i)
        e1.record(self.stream)
        self.torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        check(st)
        per = [sum(evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(K)) / K for j in range(n_k)]
        return wall * 1e3 / K, e0.elapsed_time(e1) / K, per

    def launch_means(self, lib, fn, argsets, K, check, n_max=16):
        """Per-launch mean duration (us) of the kernels one call of fn makes,
        stamped from their own dispatch, over K calls: [launch 0, launch 1, ...]."""
        evs = [[self.ev() for _ in range(2 * n_max)] for _ in range(K)]
        for e in (x for row in evs for x in row):
            e.record(self.stream)
        handles = [(ctypes.c_void_p * (2 * n_max))(*[e.cuda_event for e in row]) for row in evs]
        self.torch.cuda.synchronize()
        st, used = 0, None
        for i in range(K):
            st |= lib.mla_set_launch_events(handles[i], n_max)
            st |= fn(*argsets[i % len(argsets)])
            u = lib.mla_launch_events_used()
            assert used in (None, u), "a call's launch count changed between calls"
            used = u
        st |= lib.mla_set_launch_events(None, 0)
        self.torch.cuda.synchronize()
        check(st)
        return [round(sum(evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(K)) / K * 1e3, 2)
                for j in range(used)]

    def per_call(self, step, n, check):
        pairs = [(self.ev(), self.ev()) for _ in range(n)]
        st = 0
        for i, (a, b) in enumerate(pairs):
            a.record(self.stream)
            st |= step(i)
            b.record(self.stream)
        self.torch.cuda.synchronize()
        check(st)
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
        pct = lambda q: round(us[min(len(us) - 1, int(q * len(us)))], 2)
        return {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)}


def replicas_for(args, pool_bytes) -> int:
    """Enough rotated pool replicas that >= 512 MB separate two uses of one
    (so no call finds its cache in the 256 MB MALL)."""
    if args.replicas:
        return args.replicas
    return max(2, -(-(512 << 20) // pool_bytes))


def shader_clock_mhz(torch, timer, lib, step, n=8, iters=2000):
    """Shader clock under matrix-core load: a short MFMA-chain probe on every
    compute unit right after each of n steps of the workload (s_memtime
    cycles over s_memrealtime 100 MHz ticks, mla_clock_probe); the median over
    the probes, and their range."""
    from mla_latent_kv_07_amd import _lib as L
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros((n, wgs, 2), dtype=torch.int64, device="cuda:0")
    for i in range(n):
        L.check(step(i))
        L.check(lib.mla_clock_probe(ctypes.c_void_p(out[i].data_ptr()), wgs, iters,
                                    ctypes.c_void_p(timer.stream.cuda_stream)))
    torch.cuda.synchronize()
    o = out.cpu().double()
    mhz = sorted((o[i, :, 0].sum() / o[i, :, 1].sum() * 100.0).item() for i in range(n))
    return {"median": round(mhz[n // 2], 1), "min": round(mhz[0], 1), "max": round(mhz[-1], 1),
            "how": "s_memtime / s_memrealtime (100 MHz) over a bf16 MFMA chain on every CU, after each of "
                   f"{n} steps"}


def copy_calibration(torch, timer, dev):
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = timer.ev(), timer.ev()
    a.record(timer.stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(timer.stream)
    torch.cuda.synchronize()
    return round(2 * COPY_BYTES / (a.elapsed_time(b) / 5 * 1e-3) / 1e9, 1)


def decode_kernel_name(wl) -> str:
    """The decode kernel libmla launches for this shape."""
    if wl.q_dtype == "bf16" and wl.d_c == 512 and wl.d_r == 64 and wl.kv_dtype in MFMA_KERNELS:
        return MFMA_KERNELS[wl.kv_dtype]
    return "decode_generic_kernel"


def roofline(wl, kernel, dec_ms, cache_bytes, flops, traffic):
    """Roofline of the decode kernel.  Bound: HBM when the workload's FLOP per
    cache byte is below the ridge of the kernel's contraction (bf16 MFMA 2.5
    PFLOP/s, or fp32 vector ALU 157.3 TFLOP/s for the generic kernel, against
    8 TB/s), else the compute unit.  (fp16 caches run fp16 MFMAs, whose
    dense peak equals bf16's; the e4m3 kernel runs the latent score and the
    value sum, 94 % of its FLOPs, on 8-bit MFMAs and is priced at the fp8
    dense peak of 5.0 PFLOP/s.)"""
    gbs = cache_bytes / (dec_ms * 1e-3) / 1e9
    tfl = flops / (dec_ms * 1e-3) / 1e12
    if kernel == DECODE_KERNEL_FP8:
        cpeak, cbound = FP8_MFMA_PEAK_TFLOPS, "mfma"
    elif kernel in MFMA_KERNELS.values():
        cpeak, cbound = BF16_MFMA_PEAK_TFLOPS, "mfma"
    else:
        cpeak, cbound = FP32_VALU_PEAK_TFLOPS, "alu"
    intensity = flops / cache_bytes
    ridge = cpeak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        r = {"bound": cbound, "achieved": round(tfl, 1), "peak": cpeak, "unit": "TFLOP/s",
             "frac": round(tfl / cpeak, 4)}
    r.update({"traffic": traffic, "kernel": kernel, "algorithmic_bytes": cache_bytes,
              "algorithmic_flops": flops, "flop_per_byte": round(intensity, 1),
              "hbm_gbs": round(gbs, 1), "tflops": round(tfl, 1),
              "compute_frac": round(tfl / cpeak, 4)})
    return r


def mfma_util_at_clock(kernel, flops, dec_ms, mhz):
    """Algorithmic FLOPs per second over the dense peak of the kernel's MFMAs
    at the measured shader clock (the published peaks assume 2.4 GHz)."""
    if kernel not in MFMA_KERNELS.values():
        return None
    peak = FP8_MFMA_PEAK_TFLOPS if kernel == DECODE_KERNEL_FP8 else BF16_MFMA_PEAK_TFLOPS
    tfl = flops / (dec_ms * 1e-3) / 1e12
    return round(tfl / (peak * mhz / 2400.0), 4)


def traffic_for(kernel, workload):
    """Measured HBM bytes per launch, if the counter summary was taken for this
    kernel source on this workload."""
    if kernel != DECODE_KERNEL or not os.path.exists(TRAFFIC_JSON):
        return None
    t = json.load(open(TRAFFIC_JSON))
    ok = t.get("kernel_source_sha") == kernel_sha() and t.get("workload") == workload
    return round(t["bytes_per_launch"]) if ok else None


def run_decode(args, wl):
    import torch
    from mla_latent_kv_07_amd import _lib as L
    from mla_latent_kv_07_amd import api
    from mla_latent_kv_07_amd import inputs as I

    dev = torch.device("cuda:0")
    d = I.make_decode_inputs(wl)
    cache_bytes = d.cache.cache_bytes                      # valid rows only
    flops = visible_flops(d.cache.seq_lens, wl.q_len, wl.n_h, wl.d_c, wl.d_r)
    R = replicas_for(args, d.cache.pool.numel())

    pools = [api.DeviceCache.from_host(d.cache, dev) for _ in range(R)]
    bt = d.cache.block_table.to(dev)
    sl = d.cache.seq_lens.to(dev)
    ql, qr = d.q_lat.to(dev), d.q_rope.to(dev)
    dec = api.Decoder(d.cache.seq_lens, wl.q_len, wl.n_h, wl.d_c, wl.d_r, wl.kv_dtype, dev)
    T = wl.B * wl.q_len
    qdt = ql.dtype
    o_lat = torch.empty((T, wl.n_h, wl.d_c), dtype=qdt, device=dev)
    lse = torch.empty((T, wl.n_h), dtype=torch.float32, device=dev)

    # pre-marshalled arguments: the host must stay ahead of the GPU
    lib = L.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    descs = [p.desc() for p in pools]
    ws_bytes = dec.workspace.numel()
    qdt_c = L.DT_BF16 if qdt == torch.bfloat16 else L.DT_F32
    call_args = [(P(ql.data_ptr()), P(qr.data_ptr()), qdt_c, ctypes.byref(descs[r]),
                  P(bt.data_ptr()), bt.stride(0), P(sl.data_ptr()), wl.B, wl.q_len, wl.n_h,
                  ctypes.c_float(d.scale), ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()),
                  P(dec.workspace.data_ptr()), ws_bytes, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
                 for r in range(R)]
    fin_args = (ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()), P(dec.workspace.data_ptr()),
                ws_bytes, qdt_c, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
    full, part, fin = lib.mla_decode, lib.mla_decode_partial, lib.mla_decode_finish
    timer = Timer(torch, stream)

    def step(i):
        return full(*call_args[i % R])

    for i in range(args.warmup):
        L.check(step(i))
    torch.cuda.synchronize()
    K = args.steps
    # The headline: K plain mla_decode calls between two HIP events on the
    # launch stream (the kernels run back to back, no gap between them).
    # The decode kernel's average launch time: K back-to-back launches of the
    # decode kernel alone (mla_decode_partial) right after, between two HIP
    # events, in the same sustained-load state as the timed steps (the
    # kernel runs markedly faster after an idle gap, so a launch timed
    # alone would flatter it).  Then the same K steps again, each call's
    # kernels stamping their own start and stop (mla_set_launch_events,
    # from the dispatch itself) for the combine's share: the runtime follows
    # such a stamped launch with a cache flush, so those durations run on an
    # idler chip; the combine's figure is its stamped duration.
    n_k = 2 if dec.info.needs_combine else 1
    ms_per_step, gpu_ms = timer.steps(step, K, L.check)
    dec_ms = timer.legs(part, call_args, K, L.check)
    _, stamped_ms, per = timer.kernel_steps(lib, step, n_k, K, L.check)
    comb_ms = per[1] if n_k == 2 else 0.0
    n_leg = max(K, 50)
    call_us = timer.per_call(step, n_leg, L.check)
    clock = shader_clock_mhz(torch, timer, lib, step)
    copy_gbs = copy_calibration(torch, timer, dev) if args.copy_calibration else None

    kernel = decode_kernel_name(wl)
    S = d.cache.seq_lens.tolist()
    headline = wl.name == "v2_decode_b32_s4096_bf16"
    out = {
        "metric": ("MLA decode latent-cache GB/s + TFLOP/s, B=32 S=4096 bf16, % of roofline" if headline
                   else f"MLA decode latent-cache GB/s + TFLOP/s, {wl.name}, % of roofline"),
        "value": round(cache_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": KV_DTYPE_LABEL[wl.kv_dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "seq_len": S[0] if len(set(S)) == 1 else [min(S), max(S)],
                   "q_len": wl.q_len, "n_h": wl.n_h, "d_c": wl.d_c, "d_r": wl.d_r,
                   "kv_dtype": wl.kv_dtype, "block_size": 64, "cache_bytes": cache_bytes,
                   "pool_replicas": R, "work_items": dec.info.num_items,
                   "splits_per_seq": dec.info.max_splits},
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "call_us": call_us,
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "combine_kernel_us": round(comb_ms * 1e3, 2),
        "kernel_time_how": ("decode: K back-to-back mla_decode_partial launches right after the timed steps; "
                            "combine: its launches stamped from their own dispatch in a second pass"),
        "launches_per_step": n_k,
        "stamped_launch_us": [round(x * 1e3, 2) for x in per],
        "stamped_pass_us_per_step": round(stamped_ms * 1e3, 2),
        "shader_clock_mhz": clock,
        "roofline": roofline(wl, kernel, dec_ms, cache_bytes, flops, traffic_for(kernel, wl.name)),
        "cpu_baseline": None,
    }
    out["roofline"]["mfma_util_at_clock"] = mfma_util_at_clock(kernel, flops, dec_ms, clock["median"])
    if copy_gbs is not None:
        out["copy_calibration_gbs"] = copy_gbs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, cache_bytes)
    return out


def run_layer(args, wl, producers=False):
    """The whole absorbed layer at decode: absorb_q -> split decode + combine
    -> absorb_out, with q^C and q^R drawn N(0, 1) from the workload's
    generator after its cache.  With producers, one decode step from the
    hidden states instead: mla_project_step (h -> q~, q^R at position S_b - 1,
    and the new token's cache row written at S_b - 1, so the decode attends
    to it; the three down-projections of h as one weight) replaces the drawn
    queries and absorb_q.  The separate mla_project_q and mla_cache_append
    calls are timed beside it."""
    import torch
    from mla_latent_kv_07_amd import _lib as L
    from mla_latent_kv_07_amd import api
    from mla_latent_kv_07_amd import inputs as I

    dev = torch.device("cuda:0")
    Lw = I.make_layer_inputs(wl)
    cache = I.page_cache(wl, Lw["generator"], Lw["seq_lens"], Lw["cache_rows"])
    del Lw["cache_rows"]
    g = Lw["generator"]
    bf = torch.bfloat16
    T = wl.B * wl.q_len
    qn = torch.randn((T, wl.n_h, wl.d_nope), generator=g).to(bf).to(dev)
    qr = torch.randn((T, wl.n_h, wl.d_r), generator=g).to(bf).to(dev)
    keep = ("w_uk", "w_uv", "w_o") + (("w_dkv", "w_dq", "w_uq", "w_qr") if producers else ())
    w = {k: v.to(bf).to(dev) for k, v in Lw["weights"].items() if k in keep}
    sl_h = Lw["seq_lens"]
    cache_bytes = cache.cache_bytes
    weight_bytes = sum(v.numel() * 2 for v in w.values())
    flops_dec = visible_flops(sl_h, wl.q_len, wl.n_h, wl.d_c, wl.d_r)
    flops_q = 2.0 * T * wl.n_h * wl.d_nope * wl.d_c
    flops_o = 2.0 * T * wl.n_h * wl.d_c * wl.d_v + 2.0 * T * wl.n_h * wl.d_v * wl.d_model
    R = replicas_for(args, cache.pool.numel())
    pools = [api.DeviceCache.from_host(cache, dev) for _ in range(R)]
    bt, sl = cache.block_table.to(dev), sl_h.to(dev)
    dec = api.Decoder(sl_h, wl.q_len, wl.n_h, wl.d_c, wl.d_r, "bf16", dev)
    q_lat = torch.empty((T, wl.n_h, wl.d_c), dtype=bf, device=dev)
    o_lat = torch.empty((T, wl.n_h, wl.d_c), dtype=bf, device=dev)
    lse = torch.empty((T, wl.n_h), dtype=torch.float32, device=dev)
    u = torch.empty((T, wl.n_h, wl.d_v), dtype=bf, device=dev)
    out_t = torch.empty((T, wl.d_model), dtype=bf, device=dev)
    ws_o_bytes = api.absorb_out_workspace_bytes(T, wl.n_h, wl.d_v, wl.d_model, bf)
    ws_o = torch.empty(max(ws_o_bytes, 256), dtype=torch.uint8, device=dev)

    lib = L.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    descs = [p.desc() for p in pools]
    aq = (P(qn.data_ptr()), qn.stride(0), P(w["w_uk"].data_ptr()), P(q_lat.data_ptr()), T, wl.n_h,
          wl.d_nope, wl.d_c, L.DT_BF16, sp)
    dargs = [(P(q_lat.data_ptr()), P(qr.data_ptr()), L.DT_BF16, ctypes.byref(descs[r]), P(bt.data_ptr()),
              bt.stride(0), P(sl.data_ptr()), wl.B, wl.q_len, wl.n_h, ctypes.c_float(wl.scale),
              ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()), P(dec.workspace.data_ptr()),
              dec.workspace.numel(), P(o_lat.data_ptr()), P(lse.data_ptr()), sp) for r in range(R)]
    ao = (P(o_lat.data_ptr()), P(w["w_uv"].data_ptr()), P(w["w_o"].data_ptr()), P(u.data_ptr()),
          P(out_t.data_ptr()), P(ws_o.data_ptr()), ws_o_bytes, T, wl.n_h, wl.d_c, wl.d_v, wl.d_model,
          L.DT_BF16, sp)
    timer = Timer(torch, stream)

    if producers:
        h = Lw["hidden"].to(bf).to(dev)
        pos = (sl_h.to(torch.int32) - 1).to(dev)             # the new token of each sequence
        rope = api.rope()
        ws_a_bytes = api.cache_append_workspace_bytes(T, wl.d_model, wl.d_c, wl.d_r, bf)
        ws_a = torch.empty(max(ws_a_bytes, 256), dtype=torch.uint8, device=dev)
        ws_q_bytes = api.project_q_workspace_bytes(T, wl.d_model, wl.q_lora, wl.n_h, wl.d_nope, wl.d_c,
                                                   wl.d_r, bf)
        ws_q = torch.empty(max(ws_q_bytes, 256), dtype=torch.uint8, device=dev)
        qr_p = torch.empty((T, wl.n_h, wl.d_r), dtype=bf, device=dev)
        pq = (P(h.data_ptr()), P(w["w_dq"].data_ptr()), P(w["w_uq"].data_ptr()), P(w["w_qr"].data_ptr()),
              P(w["w_uk"].data_ptr()), L.DT_BF16, P(pos.data_ptr()), T, wl.d_model, wl.q_lora, wl.n_h,
              wl.d_nope, wl.d_c, wl.d_r, ctypes.byref(rope), P(q_lat.data_ptr()), P(qr_p.data_ptr()),
              P(ws_q.data_ptr()), ws_q.numel(), sp)
        cas = [(P(h.data_ptr()), P(w["w_dkv"].data_ptr()), L.DT_BF16, ctypes.byref(descs[r]), P(bt.data_ptr()),
                bt.stride(0), P(pos.data_ptr()), wl.B, wl.q_len, wl.d_model, ctypes.byref(rope),
                P(ws_a.data_ptr()), ws_a.numel(), sp) for r in range(R)]
        dargs = [(P(q_lat.data_ptr()), P(qr_p.data_ptr())) + a[2:] for a in dargs]
        # [W^DQ | W^DKV | W^KR]: the layout mla_project_step reads the three down-projections in
        w_dkvq = torch.cat([w["w_dq"], w["w_dkv"]], dim=1).contiguous()
        ws_s_bytes = api.project_step_workspace_bytes(wl.B, wl.q_len, wl.d_model, wl.q_lora, wl.n_h, wl.d_nope,
                                                      wl.d_c, wl.d_r, bf)
        assert ws_s_bytes > 0, "no fused producer path at this shape"
        ws_s = torch.empty(ws_s_bytes, dtype=torch.uint8, device=dev)
        pss = [(P(h.data_ptr()), P(w_dkvq.data_ptr()), P(w["w_uq"].data_ptr()), P(w["w_qr"].data_ptr()),
                P(w["w_uk"].data_ptr()), L.DT_BF16, ctypes.byref(descs[r]), P(bt.data_ptr()), bt.stride(0),
                P(pos.data_ptr()), wl.B, wl.q_len, wl.d_model, wl.q_lora, wl.n_h, wl.d_nope, ctypes.byref(rope),
                P(q_lat.data_ptr()), P(qr_p.data_ptr()), P(ws_s.data_ptr()), ws_s.numel(), sp) for r in range(R)]

        def step(i):
            return lib.mla_project_step(*pss[i % R]) | lib.mla_decode(*dargs[i % R]) | lib.mla_absorb_out(*ao)
    else:
        def step(i):
            return lib.mla_absorb_q(*aq) | lib.mla_decode(*dargs[i % R]) | lib.mla_absorb_out(*ao)

    for i in range(args.warmup):
        L.check(step(i))
    torch.cuda.synchronize()
    K = args.steps
    ms_per_step, gpu_ms = timer.steps(step, K, L.check)
    n_leg = max(K, 20)
    q_ms = timer.legs(lib.mla_absorb_q, [aq], n_leg, L.check)
    if producers:
        ps_ms = timer.legs(lib.mla_project_step, pss, n_leg, L.check)
        pq_ms = timer.legs(lib.mla_project_q, [pq], n_leg, L.check)
        ca_ms = timer.legs(lib.mla_cache_append, cas, n_leg, L.check)
    dec_ms = timer.legs(lib.mla_decode_partial, dargs, n_leg, L.check)
    fin = (ctypes.byref(dec.info), P(dec.plan_dev.data_ptr()), P(dec.workspace.data_ptr()),
           dec.workspace.numel(), L.DT_BF16, P(o_lat.data_ptr()), P(lse.data_ptr()), sp)
    comb_ms = timer.legs(lib.mla_decode_finish, [fin], n_leg, L.check)
    o_ms = timer.legs(lib.mla_absorb_out, [ao], n_leg, L.check)
    call_us = timer.per_call(step, n_leg, L.check)

    kernel = decode_kernel_name(wl)
    layer_bytes = cache_bytes + weight_bytes
    S = sl_h.tolist()
    out = {
        "metric": (f"MLA decode step from hidden states (project_step, decode, absorb_out) "
                   f"cache+weight GB/s, decode_step_b128_bf16" if producers else
                   f"MLA absorbed layer (absorb_q, decode, absorb_out) cache+weight GB/s, {wl.name}"),
        "value": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 2),
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
        "config": {"workload": "decode_step_b128_bf16" if producers else wl.name, "B": wl.B,
                   "seq_len": [min(S), max(S)], "q_len": wl.q_len,
                   "n_h": wl.n_h, "d_c": wl.d_c, "d_r": wl.d_r, "d_nope": wl.d_nope, "d_v": wl.d_v,
                   "d_model": wl.d_model, "cache_bytes": cache_bytes, "weight_bytes": weight_bytes,
                   "pool_replicas": R, "work_items": dec.info.num_items},
        "tflops": round((flops_dec + flops_q + flops_o) / (ms_per_step * 1e-3) / 1e12, 2),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "call_us": call_us,
        "absorb_q_us": round(q_ms * 1e3, 2),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "combine_kernel_us": round(comb_ms * 1e3, 2),
        "absorb_out_us": round(o_ms * 1e3, 2),
        "absorb_gemm_gbs": {
            "absorb_q": round((w["w_uk"].numel() * 2 + qn.numel() * 2 + q_lat.numel() * 2) / (q_ms * 1e-3) / 1e9, 1),
            "absorb_out": round((w["w_uv"].numel() * 2 + w["w_o"].numel() * 2 + o_lat.numel() * 2
                                 + out_t.numel() * 2) / (o_ms * 1e-3) / 1e9, 1)},
        "roofline": roofline(wl, kernel, dec_ms, cache_bytes, flops_dec, traffic_for(kernel, wl.name)),
        "cpu_baseline": None,
    }
    if producers:
        # weight-streaming rates of the producers (bytes: weights read +
        # activations read + outputs written, once each)
        b_pq = (sum(w[k].numel() for k in ("w_dq", "w_uq", "w_qr", "w_uk")) + h.numel()
                + q_lat.numel() + qr_p.numel()) * 2
        b_ca = (w["w_dkv"].numel() + h.numel() + T * (wl.d_c + wl.d_r)) * 2
        b_ps = b_pq + b_ca - h.numel() * 2   # h is read once
        out["producers"] = {
            # the step's producers in one call (queries and cache rows)
            "project_step_us": round(ps_ms * 1e3, 2), "project_step_gbs": round(b_ps / (ps_ms * 1e-3) / 1e9, 1),
            "project_step_bytes": b_ps,
            "project_step_launch_us": timer.launch_means(lib, lib.mla_project_step, pss, n_leg, L.check),
            # the same work as two separate calls
            "project_q_us": round(pq_ms * 1e3, 2), "project_q_gbs": round(b_pq / (pq_ms * 1e-3) / 1e9, 1),
            "project_q_bytes": b_pq,
            "cache_append_us": round(ca_ms * 1e3, 2), "cache_append_gbs": round(b_ca / (ca_ms * 1e-3) / 1e9, 1),
            "cache_append_bytes": b_ca,
            # each launch of one call, stamped from its own dispatch (us, in launch order)
            "project_q_launch_us": timer.launch_means(lib, lib.mla_project_q, [pq], n_leg, L.check),
            "cache_append_launch_us": timer.launch_means(lib, lib.mla_cache_append, cas, n_leg, L.check),
        }
        out["tflops"] = None
        del out["absorb_q_us"]
        out["absorb_gemm_gbs"].pop("absorb_q")
    if not args.no_cpu_baseline:
        d = I.DecodeInputs(wl=wl, cache=cache, q_lat=q_lat.cpu(), q_rope=(qr_p if producers else qr).cpu(),
                           scale=wl.scale)
        out["cpu_baseline"] = cpu_baseline(d, cache_bytes, max_rows=1024)
    return out


if __name__ == "__main__":
    main()
