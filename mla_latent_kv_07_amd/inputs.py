"""Seeded synthetic inputs for the absorbed-MLA decode path.

This module only draws random numbers, rounds them into the storage formats
with torch's casts, and lays rows out in the paged pool.  It holds none of
the method's arithmetic (no projection, RoPE, score, softmax or
absorption), so both the HIP path and the CPU oracle can take their inputs
from it.

Workloads follow the shapes the pages discuss: DeepSeek-V2 attention
(d_c = 512 latent, d_R = 64 shared RoPE key, 128 heads; donmain.dev "KV
Cache를 10분의 1로 줄인 MLA의 트릭"), a 4K context at batch 32 (blog.huny.dev
"DeepSeek MLA 해부" §1 and §4 table), 128K contexts (vLLM MLA page,
efficiency table), two-token speculative queries and an fp8 latent cache
(vLLM MLA page, "FlashMLAImpl" and "FP8 MLA 지원"; huny §6 FP8 item).

Draw order per workload (one torch CPU generator, seed fixed per workload):
  1 seq_lens, 2 weights, 3 hidden states, 4 queries, 5 cache rows,
  6 heavy-row mask, 7 pool permutation.
Values are N(0, 1) fp32 (weights N(0, 1/fan_in)), then rounded to the
workload's dtype.  Tail slots of each sequence's last block, spare blocks and
unused block-table entries hold NaN so that any read past the valid rows
shows in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

BLOCK = 64

__all__ = ["Workload", "C1", "C2", "C3", "C4", "C5", "WORKLOADS", "FORMAT_WORKLOADS", "PagedCache",
           "DecodeInputs", "draw_seq_lens", "draw_layer_weights", "draw_hidden",
           "draw_cache_rows", "draw_heavy_mask", "page_cache", "make_decode_inputs",
           "make_layer_inputs", "block_bytes"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kv_dtype: str            # "f32" | "bf16" | "fp8_e4m3"
    q_dtype: str             # "f32" | "bf16"
    B: int
    q_len: int
    n_h: int
    d_c: int
    d_r: int
    seq_lens: tuple = ()     # fixed lengths (used when seq_range is empty)
    seq_range: tuple = ()    # (lo, hi) inclusive, uniform per sequence
    heavy_frac: float = 0.0  # fraction of cached rows scaled by heavy_mult
    heavy_mult: float = 8.0
    d_nope: int = 128
    d_v: int = 128
    d_model: int = 0
    q_lora: int = 0
    spare_frac: float = 0.01

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d_nope + d_R) (the pages give none; this is
        the scale of the un-absorbed per-head dot product)."""
        return 1.0 / math.sqrt(self.d_nope + self.d_r)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny fp32 layer: the whole path, checked also against un-absorbed MHA.
C1 = Workload("tiny_fp32_layer", 1001, "f32", "f32", B=1, q_len=1, n_h=8, d_c=64, d_r=16,
              seq_lens=(256,), d_nope=32, d_v=32, d_model=256)
# DeepSeek-V2-shaped decode, 32 sequences of 4096 tokens (the measured workload).
C2 = Workload("v2_decode_b32_s4096_bf16", 1002, "bf16", "bf16", B=32, q_len=1, n_h=128,
              d_c=512, d_r=64, seq_lens=(4096,) * 32)
# Long-context split-KV stress.
C3 = Workload("long_ctx_b4_s64k_128k_bf16", 1003, "bf16", "bf16", B=4, q_len=1, n_h=128,
              d_c=512, d_r=64, seq_range=(65536, 131072), heavy_frac=0.01)
# fp8 latent cache, two-token speculative queries.
C4 = Workload("fp8_cache_spec2_b64", 1004, "fp8_e4m3", "bf16", B=64, q_len=2, n_h=128,
              d_c=512, d_r=64, seq_range=(1024, 8192))
# Full absorbed layer (absorb_q -> decode -> absorb_out), bf16.
C5 = Workload("full_layer_b128_bf16", 1005, "bf16", "bf16", B=128, q_len=1, n_h=128,
              d_c=512, d_r=64, seq_range=(1, 32768), d_nope=128, d_v=128, d_model=5120,
              q_lora=1536)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5)}

# The other cache formats at the measured shapes: fp16 rows at the
# 32 x 4096 batch, e5m2 latent codes and whole-row e4m3 at the speculative
# fp8 batch (own seeds).
FORMAT_WORKLOADS = {w.name: w for w in (
    C2.scaled(name="f16_decode_b32_s4096", seed=1012, kv_dtype="f16"),
    C4.scaled(name="fp8_e5m2_spec2_b64", seed=1014, kv_dtype="fp8_e5m2"),
    C4.scaled(name="fp8_e4m3_row_spec2_b64", seed=1024, kv_dtype="fp8_e4m3_row"),
)}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# fp8 cache formats: torch code type, largest finite value, whether k^R is coded too
_FP8 = {"fp8_e4m3": (torch.float8_e4m3fn, 448.0, False),
        "fp8_e5m2": (torch.float8_e5m2, 57344.0, False),
        "fp8_e4m3_row": (torch.float8_e4m3fn, 448.0, True)}


def block_bytes(kv_dtype: str, d_c: int, d_r: int) -> int:
    """Bytes of one 64-token block: [64][d_c + d_r] rows for f32/bf16/f16; for
    fp8_e4m3 / fp8_e5m2, 64 x d_c codes followed by 64 x d_r bf16 RoPE keys;
    for fp8_e4m3_row, 64 rows of d_c + d_r e4m3 codes."""
    if kv_dtype == "f32":
        return BLOCK * (d_c + d_r) * 4
    if kv_dtype in ("bf16", "f16"):
        return BLOCK * (d_c + d_r) * 2
    if kv_dtype in ("fp8_e4m3", "fp8_e5m2"):
        return BLOCK * d_c + BLOCK * d_r * 2
    if kv_dtype == "fp8_e4m3_row":
        return BLOCK * (d_c + d_r)
    raise ValueError(kv_dtype)


@dataclass
class PagedCache:
    pool: torch.Tensor          # uint8 [num_blocks, block_bytes]
    block_table: torch.Tensor   # int32 [B, max_blocks]
    seq_lens: torch.Tensor      # int32 [B]
    block_scales: torch.Tensor | None  # float32 [num_blocks] (fp8 only)
    kv_dtype: str
    d_c: int
    d_r: int
    perm: torch.Tensor = field(default=None)  # logical block k -> pool block

    @property
    def num_blocks(self) -> int:
        return self.pool.shape[0]

    @property
    def cache_bytes(self) -> int:
        """Bytes of valid cached rows (tail slots and spare blocks excluded)."""
        row = block_bytes(self.kv_dtype, self.d_c, self.d_r) // BLOCK
        return int(self.seq_lens.to(torch.int64).sum()) * row


@dataclass
class DecodeInputs:
    wl: Workload
    cache: PagedCache
    q_lat: torch.Tensor         # [B*q_len, n_h, d_c] (q dtype)
    q_rope: torch.Tensor        # [B*q_len, n_h, d_r]
    scale: float


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def draw_seq_lens(wl: Workload, g: torch.Generator) -> torch.Tensor:
    if wl.seq_range:
        lo, hi = wl.seq_range
        return torch.randint(lo, hi + 1, (wl.B,), generator=g, dtype=torch.int64).to(torch.int32)
    assert len(wl.seq_lens) == wl.B
    return torch.tensor(wl.seq_lens, dtype=torch.int32)


# Draws of more than this many values come from a NumPy PCG64 stream seeded
# with one 63-bit integer drawn from the workload's torch generator (one draw
# of the generator per tensor, as for small tensors, so the draw order is
# kept), filled sequentially: the multi-gigabyte caches of the long-context
# and full-layer workloads take seconds instead of minutes.
_BIG_DRAW = 1 << 20


def _normal(shape, g, std=1.0):
    n = math.prod(shape)
    if n <= _BIG_DRAW:
        return torch.randn(shape, generator=g, dtype=torch.float32) * std
    import numpy as np
    seed = int(torch.randint(0, 2 ** 63 - 1, (1,), generator=g, dtype=torch.int64))
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal(n, dtype=np.float32)
    t = torch.from_numpy(x).view(shape)
    return t * std if std != 1.0 else t


def draw_layer_weights(wl: Workload, g: torch.Generator) -> dict:
    """Weights N(0, 1/fan_in), fan_in = the input dimension of each matrix.
    Layouts: W_DKV [d_model][d_c + d_r] (first d_c columns the latent
    down-projection, the rest the RoPE-key projection); W_Q [d_model]
    [n_h (d_nope + d_r)] (head i = [q^C_i | q^R_i]) when there is no query
    low-rank path, else W_DQ [d_model][q_lora], W_UQ [q_lora][n_h d_nope],
    W_QR [d_model][n_h d_r]; W_UK [n_h][d_c][d_nope]; W_UV [n_h][d_c][d_v];
    W_O [n_h d_v][d_model]."""
    dm, n_h = wl.d_model, wl.n_h
    w = {}
    w["w_dkv"] = _normal((dm, wl.d_c + wl.d_r), g, 1 / math.sqrt(dm))
    if wl.q_lora:
        w["w_dq"] = _normal((dm, wl.q_lora), g, 1 / math.sqrt(dm))
        w["w_uq"] = _normal((wl.q_lora, n_h * wl.d_nope), g, 1 / math.sqrt(wl.q_lora))
        w["w_qr"] = _normal((dm, n_h * wl.d_r), g, 1 / math.sqrt(dm))
    else:
        w["w_q"] = _normal((dm, n_h * (wl.d_nope + wl.d_r)), g, 1 / math.sqrt(dm))
    w["w_uk"] = _normal((n_h, wl.d_c, wl.d_nope), g, 1 / math.sqrt(wl.d_c))
    w["w_uv"] = _normal((n_h, wl.d_c, wl.d_v), g, 1 / math.sqrt(wl.d_c))
    w["w_o"] = _normal((n_h * wl.d_v, dm), g, 1 / math.sqrt(n_h * wl.d_v))
    return w


def draw_hidden(wl: Workload, g: torch.Generator, n_tokens: int) -> torch.Tensor:
    return _normal((n_tokens, wl.d_model), g)


def draw_cache_rows(wl: Workload, g: torch.Generator, seq_lens: torch.Tensor) -> torch.Tensor:
    """Logical cache rows [sum(seq_lens)][d_c + d_r], N(0, 1), in (b, p) order."""
    n = int(seq_lens.to(torch.int64).sum())
    return _normal((n, wl.d_c + wl.d_r), g)


def draw_heavy_mask(wl: Workload, g: torch.Generator, n_rows: int) -> torch.Tensor:
    """Bernoulli(heavy_frac) per cached row."""
    if wl.heavy_frac <= 0:
        return torch.zeros(n_rows, dtype=torch.bool)
    return torch.rand(n_rows, generator=g) < wl.heavy_frac


def page_cache(wl: Workload, g: torch.Generator, seq_lens: torch.Tensor,
               rows: torch.Tensor) -> PagedCache:
    """Round logical rows into the storage format and scatter their 64-token
    blocks over a pool in a random order (draws the pool permutation)."""
    d_c, d_r = wl.d_c, wl.d_r
    sl = seq_lens.to(torch.int64)
    nblk = (sl + BLOCK - 1) // BLOCK
    total = int(nblk.sum())
    spare = max(1, math.ceil(wl.spare_frac * total))
    num_blocks = total + spare
    max_blocks = max(1, int(nblk.max()) if len(nblk) else 1)
    perm = torch.randperm(num_blocks, generator=g)

    # logical [total][64][d_c + d_r], NaN past each sequence's end; staged in
    # the storage dtype for f32/bf16 (rounding each value once, as a cast of
    # the whole block would), in fp32 for fp8 (the block scale needs it)
    stage_dt = _TORCH_DT.get(wl.kv_dtype, torch.float32)
    logical = torch.full((total, BLOCK, d_c + d_r), float("nan"), dtype=stage_dt)
    flat = logical.view(total * BLOCK, d_c + d_r)
    src = 0
    dst_blk = 0
    for b in range(wl.B):
        n = int(sl[b])
        if n:
            flat[dst_blk * BLOCK: dst_blk * BLOCK + n] = rows[src:src + n]
        src += n
        dst_blk += int(nblk[b])

    bt = torch.empty((wl.B, max_blocks), dtype=torch.int32)
    spare_ids = perm[total:]
    bt[:] = int(spare_ids[0])  # unused entries point at a NaN-filled spare block
    k = 0
    for b in range(wl.B):
        n = int(nblk[b])
        bt[b, :n] = perm[k:k + n].to(torch.int32)
        k += n

    bb = block_bytes(wl.kv_dtype, d_c, d_r)
    pool = torch.empty((num_blocks, bb), dtype=torch.uint8)
    scales = None
    if wl.kv_dtype in ("f32", "bf16", "f16"):
        dt = _TORCH_DT[wl.kv_dtype]
        typed = pool.view(dt).view(num_blocks, BLOCK, d_c + d_r)
        typed[:] = float("nan")
        typed[perm[:total]] = logical
    else:
        # fp8: one scale per block = absmax of its valid coded values / the
        # format's largest finite value (448 e4m3, 57344 e5m2); an all-zero
        # block takes scale 1.  The coded values are the latent, or the whole
        # row for fp8_e4m3_row.
        code_dt, top, full = _FP8[wl.kv_dtype]
        c = logical if full else logical[:, :, :d_c]
        finite = torch.nan_to_num(c, nan=0.0).abs()
        amax = finite.amax(dim=(1, 2))
        sc = torch.where(amax > 0, amax / top, torch.ones_like(amax))
        scaled = (c / sc[:, None, None]).clamp(-top, top)   # NaN stays NaN
        codes = scaled.to(code_dt).view(torch.uint8)
        pool[:] = 0
        if full:
            blk = codes.reshape(total, -1)
            pool[:] = 0x7F                      # spare blocks: NaN codes
        else:
            kr = logical[:, :, d_c:].to(torch.bfloat16).view(torch.uint8).reshape(total, -1)
            blk = torch.cat([codes.reshape(total, -1), kr], dim=1)
            # spare blocks: NaN codes and NaN RoPE keys
            pool[:, :BLOCK * d_c] = 0x7F
            pool[:, BLOCK * d_c:].view(torch.bfloat16)[:] = float("nan")
        pool[perm[:total]] = blk
        scales = torch.full((num_blocks,), float("nan"), dtype=torch.float32)
        scales[perm[:total]] = sc
    return PagedCache(pool=pool, block_table=bt, seq_lens=seq_lens.to(torch.int32),
                      block_scales=scales, kv_dtype=wl.kv_dtype, d_c=d_c, d_r=d_r, perm=perm)


def make_decode_inputs(wl: Workload) -> DecodeInputs:
    """Decode-only workload: q~ and q^R drawn directly, cache rows N(0, 1)."""
    g = _gen(wl.seed)
    seq_lens = draw_seq_lens(wl, g)
    T = wl.B * wl.q_len
    qdt = _TORCH_DT[wl.q_dtype]
    q_lat = _normal((T, wl.n_h, wl.d_c), g).to(qdt)
    q_rope = _normal((T, wl.n_h, wl.d_r), g).to(qdt)
    rows = draw_cache_rows(wl, g, seq_lens)
    heavy = draw_heavy_mask(wl, g, rows.shape[0])
    if heavy.any():
        rows[heavy] *= wl.heavy_mult
    cache = page_cache(wl, g, seq_lens, rows)
    return DecodeInputs(wl=wl, cache=cache, q_lat=q_lat, q_rope=q_rope, scale=wl.scale)


def make_layer_inputs(wl: Workload) -> dict:
    """Full-layer workload: seq_lens, weights, hidden states of the query
    tokens (one per sequence position S_b - q_len + t), and for workloads
    without a hidden-state cache (d_model > 1024) i.i.d. N(0, 1) cache rows.
    The caller derives cached rows / queries from h where the workload says so."""
    g = _gen(wl.seed)
    seq_lens = draw_seq_lens(wl, g)
    w = draw_layer_weights(wl, g)
    out = {"seq_lens": seq_lens, "weights": w}
    if wl.d_model <= 1024:
        # small layers: hidden states of every cached token (the last q_len
        # of each sequence are also the query tokens)
        out["hidden"] = draw_hidden(wl, g, int(seq_lens.to(torch.int64).sum()))
    else:
        out["hidden"] = draw_hidden(wl, g, wl.B * wl.q_len)
        out["cache_rows"] = draw_cache_rows(wl, g, seq_lens)
    out["generator"] = g
    return out
