"""Thin torch binding over libmla's C ABI (same names as the C entry points).

torch supplies device memory and the current HIP stream; every computation
runs in libmla's kernels.  Functions validate nothing beyond what is needed
to marshal arguments: the library's own host checks report errors, raised
here as MLAError.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L

_DT = {torch.float32: L.DT_F32, torch.bfloat16: L.DT_BF16}
_KV = {"f32": L.DT_F32, "bf16": L.DT_BF16, "fp8_e4m3": L.DT_FP8_E4M3, "f16": L.DT_F16,
       "fp8_e5m2": L.DT_FP8_E5M2, "fp8_e4m3_row": L.DT_FP8_E4M3_ROW}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def num_cus(device=None) -> int:
    return torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count


@dataclass
class DeviceCache:
    """A paged latent cache resident on the device (see mla_cache_desc_t)."""
    pool: torch.Tensor                 # uint8 [num_blocks, block_bytes]
    block_scales: torch.Tensor | None  # float32 [num_blocks] (fp8 only)
    kv_dtype: str
    d_c: int
    d_r: int
    # e4m3 latents: decode the codes exactly on 16-bit MFMAs instead of the
    # 8-bit MFMA path (mla_cache_desc_t.flags)
    fp8_exact: bool = False

    @property
    def num_blocks(self) -> int:
        return self.pool.shape[0]

    def desc(self) -> L.CacheDesc:
        return L.CacheDesc(self.pool.data_ptr(),
                           None if self.block_scales is None else self.block_scales.data_ptr(),
                           self.num_blocks, L.BLOCK_SIZE, self.d_c, self.d_r, _KV[self.kv_dtype],
                           L.CACHE_FP8_EXACT if self.fp8_exact else 0)

    @staticmethod
    def from_host(cache, device) -> "DeviceCache":
        return DeviceCache(cache.pool.to(device),
                           None if cache.block_scales is None else cache.block_scales.to(device),
                           cache.kv_dtype, cache.d_c, cache.d_r)


def decode_plan(seq_lens_host, q_len: int, n_h: int, d_c: int, d_r: int, kv_dtype: str,
                cus: int):
    """mla_decode_plan: returns (Plan, int32 host tensor of plan_ints entries)."""
    sl = torch.as_tensor(seq_lens_host, dtype=torch.int32).contiguous().cpu()
    B = sl.numel()
    lib = L.load()
    info = L.Plan()
    L.check(lib.mla_decode_plan(_p(sl), B, q_len, n_h, d_c, d_r, _KV[kv_dtype], cus, None, 0,
                                ctypes.byref(info)))
    plan = torch.empty(info.plan_ints, dtype=torch.int32)
    L.check(lib.mla_decode_plan(_p(sl), B, q_len, n_h, d_c, d_r, _KV[kv_dtype], cus, _p(plan),
                                plan.numel(), ctypes.byref(info)))
    return info, plan


class Decoder:
    """Holds the plan (host + device copy) and the partial-result workspace
    for repeated mla_decode calls over one batch shape."""

    def __init__(self, seq_lens_host, q_len, n_h, d_c, d_r, kv_dtype, device, cus=None):
        self.device = torch.device(device)
        self.info, self.plan_host = decode_plan(seq_lens_host, q_len, n_h, d_c, d_r, kv_dtype,
                                                cus or num_cus(self.device))
        self.plan_dev = self.plan_host.to(self.device)
        ws = max(256, self.info.workspace_bytes)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        self.q_len, self.n_h = q_len, n_h

    def __call__(self, q_lat, q_rope, cache: DeviceCache, block_table, seq_lens, scale,
                 o_lat=None, lse=None, stream=None, phase="all"):
        return decode(q_lat, q_rope, cache, block_table, seq_lens, self.q_len, self.n_h, scale,
                      self.info, self.plan_dev, self.workspace, o_lat=o_lat, lse=lse,
                      stream=stream, phase=phase)


def decode(q_lat, q_rope, cache: DeviceCache, block_table, seq_lens, q_len, n_h, scale, plan,
           plan_dev, workspace, o_lat=None, lse=None, stream=None, phase="all"):
    """mla_decode: returns (o_lat [T, n_h, d_c] in q's dtype, lse [T, n_h] fp32).
    phase="partial" / "finish" call mla_decode_partial / mla_decode_finish
    (the two launches of mla_decode) instead."""
    T = q_lat.shape[0]
    if o_lat is None:
        o_lat = torch.empty((T, n_h, cache.d_c), dtype=q_lat.dtype, device=q_lat.device)
    if lse is None:
        lse = torch.empty((T, n_h), dtype=torch.float32, device=q_lat.device)
    B = block_table.shape[0]
    desc = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = L.load()
    if phase == "finish":
        L.check(lib.mla_decode_finish(ctypes.byref(plan), _p(plan_dev), _p(workspace), ws_bytes,
                                      _DT[q_lat.dtype], _p(o_lat), _p(lse), _stream(stream)))
        return o_lat, lse
    fn = {"all": lib.mla_decode, "partial": lib.mla_decode_partial}[phase]
    L.check(fn(_p(q_lat), _p(q_rope), _DT[q_lat.dtype], ctypes.byref(desc), _p(block_table),
               block_table.stride(0), _p(seq_lens), B, q_len, n_h, float(scale), ctypes.byref(plan),
               _p(plan_dev), _p(workspace), ws_bytes, _p(o_lat), _p(lse), _stream(stream)))
    return o_lat, lse


def combine_lse(o_part, lse_part, split_off, B, rows, out_dtype=torch.float32, seq_flags=None,
                stream=None):
    """mla_combine_lse over partials o_part [P, rows, d_c] / lse_part [P, rows]."""
    d_c = o_part.shape[-1]
    o = torch.empty((B * rows, d_c), dtype=out_dtype, device=o_part.device)
    lse = torch.empty((B * rows,), dtype=torch.float32, device=o_part.device)
    L.check(L.load().mla_combine_lse(_p(o_part), _p(lse_part), _p(split_off), _p(seq_flags), B,
                                     rows, d_c, _p(o), _DT[out_dtype], _p(lse), _stream(stream)))
    return o, lse


def absorb_q(q_nope, w_uk, out=None, stream=None):
    """mla_absorb_q: q_nope [T, n_h, d_nope] (token stride may exceed n_h*d_nope),
    w_uk [n_h, d_c, d_nope] -> q_lat [T, n_h, d_c]."""
    T, n_h, d_nope = q_nope.shape
    d_c = w_uk.shape[1]
    assert q_nope.stride(2) == 1 and q_nope.stride(1) == d_nope
    if out is None:
        out = torch.empty((T, n_h, d_c), dtype=q_nope.dtype, device=q_nope.device)
    L.check(L.load().mla_absorb_q(_p(q_nope), q_nope.stride(0), _p(w_uk), _p(out), T, n_h, d_nope,
                                  d_c, _DT[q_nope.dtype], _stream(stream)))
    return out


def absorb_out_workspace_bytes(T, n_h, d_v, d_model, dtype) -> int:
    return int(L.load().mla_absorb_out_workspace(T, n_h, d_v, d_model, _DT[dtype]))


def absorb_out(o_lat, w_uv, w_o, u=None, out=None, ws=None, stream=None):
    """mla_absorb_out: o_lat [T, n_h, d_c], w_uv [n_h, d_c, d_v], w_o [n_h*d_v, d_model]
    -> (u [T, n_h, d_v], out [T, d_model])."""
    T, n_h, d_c = o_lat.shape
    d_v = w_uv.shape[2]
    d_model = w_o.shape[1]
    dev, dt = o_lat.device, o_lat.dtype
    if u is None:
        u = torch.empty((T, n_h, d_v), dtype=dt, device=dev)
    if out is None:
        out = torch.empty((T, d_model), dtype=dt, device=dev)
    need = absorb_out_workspace_bytes(T, n_h, d_v, d_model, dt)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    L.check(L.load().mla_absorb_out(_p(o_lat), _p(w_uv), _p(w_o), _p(u), _p(out), _p(ws), ws_bytes,
                                    T, n_h, d_c, d_v, d_model, _DT[dt], _stream(stream)))
    return u, out


def gather_paged(cache: DeviceCache, block_table, seq_lens, max_tokens, stream=None):
    """mla_gather_paged: [B, max_tokens, row_bytes] uint8 (rows past seq_len untouched: zero)."""
    B = block_table.shape[0]
    row_bytes = L.load().mla_cache_bytes(ctypes.byref(cache.desc())) // cache.num_blocks // L.BLOCK_SIZE
    out = torch.zeros((B, max_tokens, row_bytes), dtype=torch.uint8, device=cache.pool.device)
    desc = cache.desc()
    L.check(L.load().mla_gather_paged(ctypes.byref(desc), _p(block_table), block_table.stride(0),
                                      _p(seq_lens), B, max_tokens, _p(out), _stream(stream)))
    return out


def rope(base=10000.0, factor=1.0, orig_ctx=4096.0, beta_fast=32.0, beta_slow=1.0, mscale=1.0) -> L.Rope:
    """mla_rope_t (factor 1: plain RoPE; factor > 1: YaRN)."""
    return L.Rope(base, factor, orig_ctx, beta_fast, beta_slow, mscale)


def rope_freqs(cfg: L.Rope, d_r: int):
    """mla_rope_freqs (host): the d_r/2 angular frequencies as a list."""
    out = (ctypes.c_double * (d_r // 2))()
    L.check(L.load().mla_rope_freqs(ctypes.byref(cfg), d_r, ctypes.cast(out, ctypes.c_void_p)))
    return list(out)


def cache_append_workspace_bytes(T, d_model, d_c, d_r, dtype) -> int:
    return int(L.load().mla_cache_append_workspace(T, d_model, d_c, d_r, _DT[dtype]))


def cache_append(h, w_kv, cache: DeviceCache, block_table, pos0, q_len: int, rope_cfg: L.Rope,
                 ws=None, stream=None):
    """mla_cache_append: h [B*q_len, d_model], w_kv [d_model, d_c + d_r]; writes
    the rows of positions pos0[b] .. pos0[b] + q_len - 1 into `cache`."""
    T, d_model = h.shape
    B = T // q_len
    need = cache_append_workspace_bytes(T, d_model, cache.d_c, cache.d_r, h.dtype)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=h.device)
    desc = cache.desc()
    L.check(L.load().mla_cache_append(_p(h), _p(w_kv), _DT[h.dtype], ctypes.byref(desc), _p(block_table),
                                      block_table.stride(0), _p(pos0), B, q_len, d_model,
                                      ctypes.byref(rope_cfg), _p(ws), ws.numel(), _stream(stream)))


def project_q_workspace_bytes(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dtype) -> int:
    return int(L.load().mla_project_q_workspace(T, d_model, q_lora, n_h, d_nope, d_c, d_r, _DT[dtype]))


def project_q(h, w_dq, w_uq, w_qr, w_uk, pos, n_h: int, d_nope: int, d_r: int, rope_cfg: L.Rope,
              q_lat=None, q_rope=None, ws=None, stream=None):
    """mla_project_q: h [T, d_model] -> (q_lat [T, n_h, d_c], q_rope [T, n_h, d_r])."""
    T, d_model = h.shape
    q_lora = w_dq.shape[1]
    d_c = w_uk.shape[1]
    dev, dt = h.device, h.dtype
    if q_lat is None:
        q_lat = torch.empty((T, n_h, d_c), dtype=dt, device=dev)
    if q_rope is None:
        q_rope = torch.empty((T, n_h, d_r), dtype=dt, device=dev)
    need = project_q_workspace_bytes(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dt)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    L.check(L.load().mla_project_q(_p(h), _p(w_dq), _p(w_uq), _p(w_qr), _p(w_uk), _DT[dt], _p(pos), T, d_model,
                                   q_lora, n_h, d_nope, d_c, d_r, ctypes.byref(rope_cfg), _p(q_lat), _p(q_rope),
                                   _p(ws), ws.numel(), _stream(stream)))
    return q_lat, q_rope


def project_step_workspace_bytes(B, q_len, d_model, q_lora, n_h, d_nope, d_c, d_r, dtype) -> int:
    """0 when the shape or dtype has no fused path (use project_q and cache_append)."""
    return int(L.load().mla_project_step_workspace(B, q_len, d_model, q_lora, n_h, d_nope, d_c, d_r, _DT[dtype]))


def project_step(h, w_dkvq, w_uq, w_qr, w_uk, cache: DeviceCache, block_table, pos0, q_len: int, n_h: int,
                 d_nope: int, rope_cfg: L.Rope, q_lat=None, q_rope=None, ws=None, stream=None):
    """mla_project_step: h [B*q_len, d_model], w_dkvq [d_model, q_lora + d_c + d_r]
    (W^DQ | W^DKV | W^KR columns) -> (q_lat [T, n_h, d_c], q_rope [T, n_h, d_r]),
    and the new tokens' rows written into `cache` at pos0[b] .. pos0[b] + q_len - 1."""
    T, d_model = h.shape
    B = T // q_len
    d_c, d_r = cache.d_c, cache.d_r
    q_lora = w_dkvq.shape[1] - d_c - d_r
    dev, dt = h.device, h.dtype
    if q_lat is None:
        q_lat = torch.empty((T, n_h, d_c), dtype=dt, device=dev)
    if q_rope is None:
        q_rope = torch.empty((T, n_h, d_r), dtype=dt, device=dev)
    need = project_step_workspace_bytes(B, q_len, d_model, q_lora, n_h, d_nope, d_c, d_r, dt)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    desc = cache.desc()
    L.check(L.load().mla_project_step(_p(h), _p(w_dkvq), _p(w_uq), _p(w_qr), _p(w_uk), _DT[dt], ctypes.byref(desc),
                                      _p(block_table), block_table.stride(0), _p(pos0), B, q_len, d_model, q_lora,
                                      n_h, d_nope, ctypes.byref(rope_cfg), _p(q_lat), _p(q_rope), _p(ws), ws.numel(),
                                      _stream(stream)))
    return q_lat, q_rope
