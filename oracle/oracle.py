"""Plain fp64 CPU oracle for absorbed MLA decode (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  It never calls the HIP library and the HIP library never calls
it.  Every function states the passage of the pages it follows:

  [huny]    blog.huny.dev, "DeepSeek Multi-Head Latent Attention(MLA) 해부:
            저차원 KV 압축과 Decoupled RoPE를 통한 VRAM 98% 절감 및 행렬 흡수 ..."
  [donmain] donmain.dev/llm/attention-variants, "KV Cache를 10분의 1로 줄인
            MLA의 트릭"
  [vllm]    blog.secrett2633.cloud/opensource/vllm/mla, "[vLLM] Multi-head
            Latent Attention: KV 캐시를 압축하는 DeepSeek의 어텐션"
  [thaki]   thakicloud.com/.../transformer-attention-kv-cache-math

Parity pins (what each function is checked against, other than itself) are
recorded in PIN_STATUS below and exercised by tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from pathlib import Path

import numpy as np

__all__ = [
    "PIN_STATUS", "FMT_F32", "FMT_BF16", "FMT_FP8_E4M3", "FMT_F16", "FMT_FP8_E5M2", "FMT_FP8_E4M3_ROW",
    "FP8_SPLIT", "SCALED", "FP8_MAX", "BLOCK", "f16_bits_to_f64", "e5m2_to_f64", "f64_to_e5m2", "f64_to_f16",
    "fp8_decode", "fp8_encode",
    "lib", "build_oracle", "threads",
    "kv_bytes_per_token_layer", "kv_cache_bytes", "floats_per_token_all_layers",
    "bf16_bits_to_f64", "e4m3_to_f64", "f64_to_e4m3", "f64_to_bf16", "block_bytes",
    "gather", "decode", "combine", "decode_splits",
    "rope", "rope_inv_freq", "project_kv", "project_queries_direct", "project_queries_lowrank",
    "cache_append", "project_queries_absorbed", "E4M3_MAX",
    "absorb_q", "absorb_out", "fused_out_weights", "absorb_out_fused",
    "score_split", "unabsorbed_mha",
]

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "mla_oracle.c"
_SO = _HERE / "liboracle.so"

FMT_F32, FMT_BF16, FMT_FP8_E4M3, FMT_F16, FMT_FP8_E5M2, FMT_FP8_E4M3_ROW = 0, 1, 2, 3, 4, 5
FP8_SPLIT = (FMT_FP8_E4M3, FMT_FP8_E5M2)        # 8-bit latent codes + bf16 k^R
SCALED = (FMT_FP8_E4M3, FMT_FP8_E5M2, FMT_FP8_E4M3_ROW)
FP8_MAX = {FMT_FP8_E4M3: 448.0, FMT_FP8_E4M3_ROW: 448.0, FMT_FP8_E5M2: 57344.0}
BLOCK = 64  # tokens per paged block ([vllm] "FlashMLABackend: 하드웨어 요구사항")

# How each oracle function is pinned to something other than itself.
PIN_STATUS = {
    "kv_bytes_per_token_layer": "pinned: every cache size printed on the pages (tests/golden/cache_sizes.json)",
    "bf16_bits_to_f64": "pinned: torch bf16->fp64 cast over all 65536 codes",
    "e4m3_to_f64": "pinned: OCP E4M3 landmark values + torch float8_e4m3fn->fp64 over all 256 codes",
    "f64_to_e4m3": "pinned: torch float8_e4m3fn cast (RNE, ties, subnormals, saturation)",
    "gather": "pinned: contiguous logical rows scattered through a random block table come back bit-exact",
    "decode": "pinned: torch SDPA fp64 (MQA, one KV head); S=1 and q=0 closed forms; "
              "un-absorbed MHA equivalence; block-table permutation invariance; "
              "causal q_len=2 == q_len=1 on the truncated sequence",
    "combine": "pinned: split invariance against the unsplit decode for random partitions",
    "rope": "pinned: norm preservation, relative-position property, complex-multiply form",
    "rope_inv_freq": "pinned: factor 1 is plain RoPE; YaRN's two limits (position interpolation p/s "
                     "below beta_slow, plain RoPE above beta_fast) in closed form; relative-position "
                     "property and the mscale norm factor with the scaled frequencies",
    "f16_bits_to_f64": "pinned: numpy's fp16 decode over all 65536 codes",
    "f64_to_f16": "pinned: torch's fp32->fp16 cast on fp32 values (numpy's correctly rounded cast is the step)",
    "e5m2_to_f64": "pinned: OCP E5M2 landmarks + torch float8_e5m2->fp64 over all 256 codes",
    "f64_to_e5m2": "pinned: torch float8_e5m2 cast below the saturation point (RNE, ties, subnormals); "
                   "saturation to +-57344",
    "decode (f16, fp8_e5m2, fp8_e4m3_row caches)": "pinned: torch SDPA fp64 on the f16-rounded rows; fp8 "
                   "variants equal the fp32 cache of torch-decoded codes times the block scale",
    "f64_to_bf16": "pinned: torch's fp32->bf16 cast on fp32-exact values incl. ties and subnormals; "
                   "nearest of the two neighbours (independently pinned decoder) on fp64 values",
    "cache_append": "pinned: appended rows gather back as the single rounding of project_kv's rows "
                    "(bf16, f32) over ragged call sizes; bytes outside written slots unchanged; fp8 "
                    "whole-block scale = amax/448 with codes within half an e4m3 step; scale growth "
                    "re-encodes earlier rows within two roundings; all-zero block takes scale 1",
    "project_kv": "pinned: one-hot hidden states select weight rows exactly (c = first d_c columns, "
                  "k^R = the rest, unrotated at position 0) and each rotary pair equals an explicit 2x2 "
                  "rotation by p * 10000^(-2j/d_R) at the token's own position; linear in h",
    "project_queries_direct": "pinned: one-hot hidden states select head blocks [q^C_i | q^R_i] of W_Q "
                              "exactly, q^R turned by an explicit 2x2 rotation at each token's position",
    "project_queries_lowrank": "pinned: equals the one-matrix projection with merged per-head weights; "
                               "with W^DQ = I one-hot rows select W^UQ / W^QR head columns, q^R turned "
                               "by an explicit 2x2 rotation",
    "project_queries_absorbed": "pinned: absorbed scores equal scores against explicitly reconstructed keys",
    "absorb_q": "pinned: absorbed score equals score against explicitly reconstructed keys",
    "absorb_out": "pinned: equals explicit per-head value reconstruction followed by W^O",
    "absorb_out_fused": "pinned: W^UV W^O fusion equals the unfused path",
    "unabsorbed_mha": "pinned: torch SDPA fp64 per head (textbook multi-head attention)",
    "paper_case_values": "parity unpinned: the -22.3809850107 and -6.073908192658 values of the "
                         "pages' five-case script have no seed or shapes",
}


# ----------------------------------------------------------------------------
# Build / load the C part
# ----------------------------------------------------------------------------

def build_oracle(force: bool = False) -> Path:
    """Compile mla_oracle.c with gcc (fp64, OpenMP over output rows)."""
    if force or not _SO.exists() or _SO.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _SO.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-o", str(tmp), str(_SRC), "-lm"],
            check=True,
        )
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # MLA_ORACLE_LIB names another build of mla_oracle.c (the
        # host-sanitizer build the CPU tests make)
        so = os.environ.get("MLA_ORACLE_LIB") or build_oracle()
        L = ctypes.CDLL(str(so))
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = dbl
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = dbl
        L.oracle_f64_to_e4m3.argtypes = [dbl]
        L.oracle_f64_to_e4m3.restype = ctypes.c_uint8
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e5m2_to_f64.restype = dbl
        L.oracle_f64_to_e5m2.argtypes = [dbl]
        L.oracle_f64_to_e5m2.restype = ctypes.c_uint8
        L.oracle_block_bytes.argtypes = [i32, i32, i32]
        L.oracle_block_bytes.restype = i64
        L.oracle_gather.argtypes = [P, i32, i32, i32, P, i32, P, i32, i32, P]
        L.oracle_gather.restype = i32
        L.oracle_decode.argtypes = [P, i32, P, P, i32, P, i32, i32, i32, i32, i32,
                                    P, P, dbl, P, P, P, i64, P, P]
        L.oracle_decode.restype = i32
        L.oracle_combine.argtypes = [P, P, i32, i64, i32, P, P]
        L.oracle_combine.restype = i32
        L.oracle_threads.restype = i32
        _lib = L
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(lib().oracle_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _np(x, dtype=None):
    """Host array view of a numpy array or CPU torch tensor (no arithmetic)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if dtype is not None and str(x.dtype) in ("torch.bfloat16", "torch.float8_e4m3fn"):
            raise TypeError("pass raw bits for reduced formats")
        x = x.numpy()
    x = np.ascontiguousarray(x)
    if dtype is not None:
        x = np.ascontiguousarray(x, dtype=dtype)
    return x


# ----------------------------------------------------------------------------
# Closed-form cache sizes
# ----------------------------------------------------------------------------

def kv_bytes_per_token_layer(kind: str, *, n_h: int = 0, d_h: int = 0, groups: int = 0,
                             d_c: int = 0, d_r: int = 0, bytes_per: int = 2) -> int:
    """Cache bytes one token occupies in one layer.

    MHA keeps a key and a value per head: 2 * n_h * d_h * P ([huny] §1 memory
    formula).  GQA keeps one pair per group: 2 * g * d_h * P ([huny] §1, §4
    table; [thaki] "논문 공식을 코드로 옮기기").  MQA is GQA with g = 1
    ([donmain] "공유의 한계": 2 * d_h floor).  MLA keeps the latent and the
    shared RoPE key: (d_c + d_R) * P ([donmain] "MLA, 압축이라는 다른 길" 576
    = 512 + 64; [huny] §4 table).
    """
    if kind == "mha":
        return 2 * n_h * d_h * bytes_per
    if kind == "gqa":
        return 2 * groups * d_h * bytes_per
    if kind == "mqa":
        return 2 * d_h * bytes_per
    if kind == "mla":
        return (d_c + d_r) * bytes_per
    raise ValueError(kind)


def kv_cache_bytes(kind: str, *, layers: int, tokens: int, **kw) -> int:
    """Whole-request cache: per-token-per-layer bytes x layers x tokens
    ([huny] §1 memory formula, factors L and S)."""
    return kv_bytes_per_token_layer(kind, **kw) * layers * tokens


def floats_per_token_all_layers(kind: str, *, layers: int, kv_heads: int = 0,
                                d_head: int = 0, d_latent: int = 0) -> int:
    """Cache floats per token summed over layers as [thaki] counts them
    ("논문 공식을 코드로 옮기기"): layers * kv_heads * 2 * d_head for MHA/GQA,
    layers * d_L for the latent (one shared vector per token and layer)."""
    if kind == "mla":
        return layers * d_latent
    return layers * kv_heads * 2 * d_head


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (upper half of binary32), exact."""
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([L.oracle_bf16_to_f64(int(b)) for b in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes -> float64, from the format definition."""
    L = lib()
    table = np.array([L.oracle_e4m3_to_f64(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 codes, round-to-nearest-even, saturating at +-448."""
    L = lib()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([L.oracle_f64_to_e4m3(float(v)) for v in flat], dtype=np.uint8)
    return out.reshape(np.shape(x))


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, rounded once to nearest-even from
    the fp64 value (8 significant bits, binary32's exponent range with
    subnormals; overflow -> inf; NaN -> quiet NaN)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    a = np.abs(np.where(fin, x, 0.0))
    m, e = np.frexp(a)                          # a = m 2^e, m in [0.5, 1)
    e = np.maximum(e, -125)                     # below 2^-126 the spacing stays 2^-133
    q = np.ldexp(np.rint(np.ldexp(a, 8 - e)), e - 8)   # rint: half to even
    q = np.where(q > 3.3895313892515355e38, np.inf, q)  # past the largest finite bf16
    out[...] = np.where(fin, np.copysign(q, x), x)
    bits = (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE fp16 bit patterns -> float64, from the format definition."""
    L = lib()
    table = np.array([L.oracle_f16_to_f64(c) for c in range(65536)], dtype=np.float64)
    return table[np.asarray(bits, dtype=np.uint16)]


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE fp16 bit patterns, one round-to-nearest-even step
    (numpy's double -> half conversion; overflow -> inf)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def e5m2_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E5M2 codes -> float64, from the format definition."""
    L = lib()
    table = np.array([L.oracle_e5m2_to_f64(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def f64_to_e5m2(x: np.ndarray) -> np.ndarray:
    """float64 -> E5M2 codes, round-to-nearest-even, saturating at +-57344."""
    L = lib()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([L.oracle_f64_to_e5m2(float(v)) for v in flat], dtype=np.uint8)
    return out.reshape(np.shape(x))


def fp8_decode(fmt: int, codes: np.ndarray) -> np.ndarray:
    return e5m2_to_f64(codes) if fmt == FMT_FP8_E5M2 else e4m3_to_f64(codes)


def fp8_encode(fmt: int, x: np.ndarray) -> np.ndarray:
    return f64_to_e5m2(x) if fmt == FMT_FP8_E5M2 else f64_to_e4m3(x)


def block_bytes(fmt: int, d_c: int, d_r: int) -> int:
    return int(lib().oracle_block_bytes(fmt, d_c, d_r))


# ----------------------------------------------------------------------------
# Paged cache and decode (C part)
# ----------------------------------------------------------------------------

def gather(pool, fmt, d_c, d_r, block_table, seq_lens, max_tokens) -> np.ndarray:
    """Bytes of each sequence's logical rows, out[b][p] for p < seq_lens[b]
    (paged block table, [huny] §6; [vllm] "MLA의 MQA 디코딩 경로").
    Rows past seq_lens[b] are zero."""
    pool = _np(pool)
    bt = _np(block_table, np.int32)
    sl = _np(seq_lens, np.int32)
    B, stride = bt.shape
    row_bytes = block_bytes(fmt, d_c, d_r) // BLOCK
    out = np.zeros((B, max_tokens, row_bytes), dtype=np.uint8)
    rc = lib().oracle_gather(_ptr(pool), fmt, d_c, d_r, _ptr(bt), stride, _ptr(sl),
                             B, max_tokens, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_gather failed ({rc})")
    return out


def decode(pool, fmt, block_table, seq_lens, q_lat, q_rope, scale, *, q_len=1,
           block_scales=None, win_lo=None, win_hi=None, rows=None):
    """Absorbed decode in fp64: see oracle_decode in mla_oracle.c.

    q_lat: [B*q_len, n_h, d_c] and q_rope: [B*q_len, n_h, d_r], any real dtype
    (converted to float64 exactly).  Returns (o_lat, lse) as float64 with shapes
    [B*q_len, n_h, d_c] / [B*q_len, n_h], or [n_rows, d_c] / [n_rows] when
    `rows` lists flat row indices.
    """
    pool = _np(pool)
    bt = _np(block_table, np.int32)
    sl = _np(seq_lens, np.int32)
    ql = _np(q_lat, np.float64)
    qr = _np(q_rope, np.float64)
    T, n_h, d_c = ql.shape
    d_r = qr.shape[2]
    B = bt.shape[0]
    assert T == B * q_len and qr.shape[:2] == (T, n_h)
    bs = None if block_scales is None else _np(block_scales, np.float32)
    lo = None if win_lo is None else _np(win_lo, np.int32)
    hi = None if win_hi is None else _np(win_hi, np.int32)
    rws = None if rows is None else _np(rows, np.int64)
    n_out = T * n_h if rws is None else rws.size
    o = np.empty((n_out, d_c), dtype=np.float64)
    lse = np.empty((n_out,), dtype=np.float64)
    rc = lib().oracle_decode(_ptr(pool), fmt, _ptr(bs), _ptr(bt), bt.shape[1], _ptr(sl),
                             B, q_len, n_h, d_c, d_r, _ptr(ql), _ptr(qr), float(scale),
                             _ptr(lo), _ptr(hi), _ptr(rws), 0 if rws is None else rws.size,
                             _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    if rws is None:
        return o.reshape(T, n_h, d_c), lse.reshape(T, n_h)
    return o, lse


def combine(o_part, lse_part):
    """Merge per-split results: o_part [S][rows][d_c], lse_part [S][rows]."""
    op = _np(o_part, np.float64)
    lp = _np(lse_part, np.float64)
    S, rows, d_c = op.shape
    o = np.empty((rows, d_c), dtype=np.float64)
    lse = np.empty((rows,), dtype=np.float64)
    lib().oracle_combine(_ptr(op), _ptr(lp), S, rows, d_c, _ptr(o), _ptr(lse))
    return o, lse


def decode_splits(pool, fmt, block_table, seq_lens, q_lat, q_rope, scale, bounds, *,
                  q_len=1, block_scales=None):
    """Per-split partials: bounds is a list of (win_lo[B], win_hi[B]) arrays.
    Returns o_part [S][T*n_h][d_c], lse_part [S][T*n_h]."""
    os_, ls_ = [], []
    for lo, hi in bounds:
        o, l = decode(pool, fmt, block_table, seq_lens, q_lat, q_rope, scale, q_len=q_len,
                      block_scales=block_scales, win_lo=lo, win_hi=hi)
        os_.append(o.reshape(-1, o.shape[-1]))
        ls_.append(l.reshape(-1))
    return np.stack(os_), np.stack(ls_)


# ----------------------------------------------------------------------------
# Projections, RoPE and the un-absorbed reference (numpy, fp64)
# ----------------------------------------------------------------------------

def rope_inv_freq(d: int, base: float = 10000.0, factor: float = 1.0, orig_ctx: float = 4096.0,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Angular frequency theta_j of rotary pair j (j < d/2), in fp64.

    Plain RoPE (factor == 1): theta_j = base^(-2j/d) ([huny] §2-3 decoupled
    RoPE; [donmain] "위치 정보와 압축의 충돌").  The pages name YaRN for
    128K+ contexts and say only that its base frequency and scaling factor
    must match the model ([huny] §6, the YaRN item); they give no formula.
    This follows the published YaRN method (Peng et al., 2023, "NTK-by-parts"
    interpolation): pair j turns r_j = orig_ctx * theta_j / (2 pi) times over
    the original context; pairs with r_j <= beta_slow are interpolated
    (theta_j / factor), pairs with r_j >= beta_fast keep theta_j, and a
    linear ramp gamma = (r_j - beta_slow) / (beta_fast - beta_slow) blends
    the two in between: theta'_j = (1 - gamma) theta_j / factor + gamma theta_j."""
    assert d % 2 == 0 and factor > 0
    j = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / d)
    if factor == 1.0:
        return theta
    r = orig_ctx * theta / (2.0 * math.pi)
    if beta_fast > beta_slow:
        gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    else:
        gamma = (r >= beta_fast).astype(np.float64)
    return (1.0 - gamma) * theta / factor + gamma * theta


def rope(x: np.ndarray, positions: np.ndarray, base: float = 10000.0, *,
         inv_freq: np.ndarray | None = None, mscale: float = 1.0) -> np.ndarray:
    """Rotary position embedding of the last axis (decoupled RoPE input,
    [huny] §2-3; [donmain] "위치 정보와 압축의 충돌").  The pages do not fix
    the pairing: adjacent pairs (2j, 2j+1) are rotated by angle p * theta_j
    with theta_j = base^(-2j/d), or the given inv_freq (rope_inv_freq's YaRN
    frequencies); the result is multiplied by mscale (YaRN's magnitude
    factor, 1 for plain RoPE).  positions broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    if inv_freq is None:
        j = np.arange(d // 2, dtype=np.float64)
        theta = base ** (-2.0 * j / d)
    else:
        theta = np.asarray(inv_freq, dtype=np.float64)
        assert theta.shape == (d // 2,)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out * mscale if mscale != 1.0 else out


def project_kv(h: np.ndarray, w_dkv: np.ndarray, d_c: int, positions: np.ndarray, *,
               inv_freq: np.ndarray | None = None, mscale: float = 1.0):
    """Cached row of each token: c = h W^DKV ([huny] §2-1 compression equation)
    and k^R = RoPE(h W^KR) ([huny] §2-3 shared rotary key).  W^DKV and W^KR
    are read as the first d_c and the remaining columns of one matrix."""
    z = np.asarray(h, np.float64) @ np.asarray(w_dkv, np.float64)
    c = z[:, :d_c]
    kr = rope(z[:, d_c:], positions, inv_freq=inv_freq, mscale=mscale)
    return c, kr


def project_queries_direct(h: np.ndarray, w_q: np.ndarray, n_h: int, d_nope: int,
                           d_r: int, positions: np.ndarray):
    """Per-head query [q^C_i ; q^R_i] from one projection of h; q^R is rotated
    at the query's position ([huny] §2-3 rotary query and concatenation)."""
    z = (np.asarray(h, np.float64) @ np.asarray(w_q, np.float64)).reshape(-1, n_h, d_nope + d_r)
    q_nope = z[:, :, :d_nope]
    q_rope = rope(z[:, :, d_nope:], np.asarray(positions)[:, None])
    return q_nope, q_rope


def project_queries_lowrank(h, w_dq, w_uq, w_qr, n_h, d_nope, d_r, positions, *,
                            inv_freq=None, mscale=1.0):
    """Low-rank query path: c^Q = h W^DQ, q^C_i = c^Q W^UQ_i ([huny] §2-2), and
    q^R_i = RoPE(h W^QR_i) ([huny] §2-3, read literally from h)."""
    h = np.asarray(h, np.float64)
    cq = h @ np.asarray(w_dq, np.float64)
    q_nope = (cq @ np.asarray(w_uq, np.float64)).reshape(-1, n_h, d_nope)
    q_rope = rope((h @ np.asarray(w_qr, np.float64)).reshape(-1, n_h, d_r),
                  np.asarray(positions)[:, None], inv_freq=inv_freq, mscale=mscale)
    return q_nope, q_rope


def project_queries_absorbed(h, w_dq, w_uq, w_qr, w_uk, n_h, d_nope, d_r, positions, *,
                             inv_freq=None, mscale=1.0):
    """The decode's query inputs straight from the hidden state: the low-rank
    query path ([huny] §2-2, §2-3) followed by the W^UK absorption ([huny]
    §3-1).  Returns (q_lat [T][n_h][d_c], q_rope [T][n_h][d_r])."""
    q_nope, q_rope = project_queries_lowrank(h, w_dq, w_uq, w_qr, n_h, d_nope, d_r, positions,
                                             inv_freq=inv_freq, mscale=mscale)
    return absorb_q(q_nope, w_uk), q_rope


E4M3_MAX = 448.0   # largest finite OCP E4M3 value


def cache_append(pool, block_scales, fmt: int, d_c: int, d_r: int, block_table, pos0,
                 q_len: int, h, w_kv, *, inv_freq=None, mscale: float = 1.0) -> None:
    """Write the cache rows of q_len new tokens per sequence, in place.

    Token t = b q_len + i of sequence b sits at position p = pos0[b] + i.  Its
    row [c | k^R] = project_kv(h_t) at p ([huny] §2-1 compression equation,
    §2-3 shared rotary key) goes to slot p % 64 of block block_table[b][p // 64]
    (paged cache of 64-token blocks, [vllm] "FlashMLABackend" and
    "FlashMLAImpl").  The exact fp64 row is rounded once into the storage
    format: f32 / bf16 rows to nearest-even.

    fp16 rows round to nearest-even once too.

    fp8 (e4m3 or e5m2 latent with bf16 k^R, or the whole row in e4m3; one
    scale per block: [huny] §6 FP8 item) — the pages ask for a dynamic
    per-block scale and give no update rule for a block that fills over
    several calls.  Reading used here (M = 448 for e4m3, 57344 for e5m2; the
    amax covers the coded values: c, or c and k^R for the whole-row format):
      - a block whose slot 0 is written by this call starts fresh: its scale
        is amax over the tokens written into it / M (1 if that is 0), as for
        a block written whole;
      - otherwise scale' = max(scale, amax / M); when it grows, the codes of
        the slots before the first one written are re-encoded,
        code' = fp8(value(code) * scale / scale');
      - the new codes are fp8(value / scale').
    Scales are kept as float32; the codes use the stored float32 value.
    A token whose position has no table entry (p < 0 or p >= 64 * table
    width), or whose entry is not a pool block id (an unallocated slot such as
    -1), is not written: the pages leave such tokens undefined, and skipping
    them keeps every other block intact.
    pool: uint8 [num_blocks][block_bytes]; block_scales: float32 [num_blocks]
    (fp8 only).  Both are modified."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    pos0 = np.asarray(pos0)
    B = bt.shape[0]
    T = B * q_len
    pos = (pos0[:, None].astype(np.int64) + np.arange(q_len)[None, :]).reshape(T)
    c, kr = project_kv(h, w_kv, d_c, pos, inv_freq=inv_freq, mscale=mscale)
    nblk_pool = pool.shape[0]
    if fmt in (FMT_F32, FMT_BF16, FMT_F16):
        rows = np.concatenate([c, kr], axis=1)
        if fmt == FMT_BF16:
            enc = f64_to_bf16(rows).view(np.uint8).reshape(T, -1)
        elif fmt == FMT_F16:
            enc = f64_to_f16(rows).view(np.uint8).reshape(T, -1)
        else:
            enc = rows.astype(np.float32).view(np.uint8).reshape(T, -1)
        rb = enc.shape[1]
        for t in range(T):
            b, p = t // q_len, int(pos[t])
            if p < 0 or p // BLOCK >= bt.shape[1]:
                continue                     # no table entry: not written
            blk = int(bt[b, p // BLOCK])
            if not 0 <= blk < nblk_pool:
                continue                     # unallocated table slot: not written
            pool[blk, (p % BLOCK) * rb:(p % BLOCK + 1) * rb] = enc[t]
        return
    assert fmt in SCALED
    full = fmt == FMT_FP8_E4M3_ROW
    W = d_c + d_r if full else d_c                  # code bytes per token
    vals = np.concatenate([c, kr], axis=1) if full else c
    top = FP8_MAX[fmt]
    scales = np.asarray(block_scales)
    kr_bits = f64_to_bf16(kr).view(np.uint8).reshape(T, -1)
    for b in range(B):
        # the sequence's tokens, grouped by the block they land in (in order)
        groups: dict[int, list[int]] = {}
        for i in range(q_len):
            p = int(pos[b * q_len + i])
            if p < 0 or p // BLOCK >= bt.shape[1]:
                continue                     # no table entry: not written
            groups.setdefault(p // BLOCK, []).append(i)
        for lb, idx in groups.items():
            blk = int(bt[b, lb])
            if not 0 <= blk < nblk_pool:
                continue                     # unallocated table slot: not written
            toks = [b * q_len + i for i in idx]
            slots = [int(pos[t]) % BLOCK for t in toks]
            amax = float(np.max(np.abs(vals[toks])))
            fresh = min(slots) == 0
            new = amax / top
            if fresh:
                sc = float(np.float32(new if amax > 0 else 1.0))
            else:
                old = float(scales[blk])
                sc = float(np.float32(max(old, new)))
                if sc > old:
                    s0 = min(slots)
                    codes = pool[blk, :s0 * W]
                    pool[blk, :s0 * W] = fp8_encode(fmt, fp8_decode(fmt, codes) * (old / sc))
            scales[blk] = np.float32(sc)
            for t, sl in zip(toks, slots):
                pool[blk, sl * W:(sl + 1) * W] = fp8_encode(fmt, vals[t] / sc)
                if not full:
                    off = BLOCK * d_c + sl * 2 * d_r
                    pool[blk, off:off + 2 * d_r] = kr_bits[t]


def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q~_{t,i} = q^C_{t,i} (W^UK_i)^T, one d_c-wide vector per head
    ([huny] §3-1 absorption equation; [donmain] column form W^UK^T q).
    q_nope [T][n_h][d_nope], w_uk [n_h][d_c][d_nope] -> [T][n_h][d_c]."""
    q = np.asarray(q_nope, np.float64)
    w = np.asarray(w_uk, np.float64)
    out = np.empty((q.shape[0], q.shape[1], w.shape[1]), dtype=np.float64)
    for i in range(q.shape[1]):
        out[:, i, :] = q[:, i, :] @ w[i].T
    return out


def absorb_out(o_lat: np.ndarray, w_uv: np.ndarray, w_o: np.ndarray):
    """u_{t,i} = (sum_j A c_j) W^UV_i ([huny] §3-2 value equation), then
    Output_t = sum_i u_{t,i} W^O_i with W^O_i the i-th d_v-row block of W^O
    ([huny] §3-2 output equation).  o_lat [T][n_h][d_c], w_uv [n_h][d_c][d_v],
    w_o [n_h*d_v][d_model].  Returns (u [T][n_h][d_v], out [T][d_model])."""
    o = np.asarray(o_lat, np.float64)
    wv = np.asarray(w_uv, np.float64)
    wo = np.asarray(w_o, np.float64)
    T, n_h, _ = o.shape
    d_v = wv.shape[2]
    u = np.empty((T, n_h, d_v), dtype=np.float64)
    for i in range(n_h):
        u[:, i, :] = o[:, i, :] @ wv[i]
    out = np.zeros((T, wo.shape[1]), dtype=np.float64)
    for i in range(n_h):
        out += u[:, i, :] @ wo[i * d_v:(i + 1) * d_v, :]
    return u, out


def fused_out_weights(w_uv: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """W^combined_i = W^UV_i W^O_i in R^{d_c x d} ([huny] §3-2 output equation)."""
    wv = np.asarray(w_uv, np.float64)
    wo = np.asarray(w_o, np.float64)
    d_v = wv.shape[2]
    return np.stack([wv[i] @ wo[i * d_v:(i + 1) * d_v, :] for i in range(wv.shape[0])])


def absorb_out_fused(o_lat: np.ndarray, w_comb: np.ndarray) -> np.ndarray:
    """Output_t = sum_i o_{t,i} W^combined_i ([huny] §3-2)."""
    o = np.asarray(o_lat, np.float64)
    out = np.zeros((o.shape[0], w_comb.shape[2]), dtype=np.float64)
    for i in range(o.shape[1]):
        out += o[:, i, :] @ w_comb[i]
    return out


def score_split(q_c, q_r, k_c, k_r):
    """Concatenated-vector score and its content + position parts
    ([huny] §2-3 decomposition equation).  Returns (full, content, position)."""
    q = np.concatenate([q_c, q_r])
    k = np.concatenate([k_c, k_r])
    return float(q @ k), float(q_c @ k_c), float(q_r @ k_r)


def unabsorbed_mha(c, kr, q_nope, q_rope, w_uk, w_uv, w_o, scale, query_pos):
    """Textbook multi-head attention with explicitly reconstructed keys and
    values, the path absorption removes ([huny] §2-1 up-projections,
    §2-3 concatenated q/k; [huny] §6 'naive fallback').

    c [S][d_c], kr [S][d_r] (already rotated), q_nope [T][n_h][d_nope],
    q_rope [T][n_h][d_r] (rotated), query_pos [T]: query t sees positions
    <= query_pos[t].  Returns (o_lat_equiv [T][n_h][d_c] = sum_j A c_j,
    u [T][n_h][d_v], out [T][d_model], lse [T][n_h])."""
    c = np.asarray(c, np.float64)
    kr = np.asarray(kr, np.float64)
    wk = np.asarray(w_uk, np.float64)
    wv = np.asarray(w_uv, np.float64)
    wo = np.asarray(w_o, np.float64)
    T, n_h, _ = np.shape(q_nope)
    d_v = wv.shape[2]
    o_lat = np.zeros((T, n_h, c.shape[1]))
    u = np.zeros((T, n_h, d_v))
    lse = np.zeros((T, n_h))
    for i in range(n_h):
        k_full = np.concatenate([c @ wk[i], kr], axis=1)   # [S][d_nope + d_r]
        v_full = c @ wv[i]                                 # [S][d_v]
        for t in range(T):
            n = int(query_pos[t]) + 1
            qf = np.concatenate([np.asarray(q_nope[t, i], np.float64),
                                 np.asarray(q_rope[t, i], np.float64)])
            s = scale * (k_full[:n] @ qf)
            m = s.max()
            e = np.exp(s - m)
            a = e / e.sum()
            u[t, i] = a @ v_full[:n]
            o_lat[t, i] = a @ c[:n]
            lse[t, i] = m + math.log(e.sum())
    out = np.zeros((T, wo.shape[1]))
    for i in range(n_h):
        out += u[:, i, :] @ wo[i * d_v:(i + 1) * d_v, :]
    return o_lat, u, out, lse
