"""ctypes declarations of libmla.so (the C ABI in include/mla.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind these entry points.  Loading fails loudly if the library has
not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

# MLA_LIB names another build of the same library (the host-sanitizer build
# the CPU tests make); by default the in-tree one
LIB_PATH = Path(os.environ.get("MLA_LIB") or Path(__file__).resolve().parent / "libmla.so")

(MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_HIP,
 MLA_ERR_DEVICE_CHECK) = range(7)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "ALIGN", 4: "WORKSPACE", 5: "HIP",
                6: "DEVICE_CHECK"}
DT_F32, DT_BF16, DT_FP8_E4M3, DT_F16, DT_FP8_E5M2, DT_FP8_E4M3_ROW = 0, 1, 2, 3, 4, 5
BLOCK_SIZE = 64
CACHE_FP8_EXACT = 1   # mla_cache_desc_t.flags: exact fp8 decode on 16-bit MFMAs
NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES

c_int32, c_int64, c_void_p, c_float = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("base", c_void_p),
        ("block_scales", c_void_p),
        ("num_blocks", c_int64),
        ("block_size", c_int32),
        ("d_c", c_int32),
        ("d_r", c_int32),
        ("kv_dtype", c_int32),
        ("flags", c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("q_len", c_int32), ("n_h", c_int32), ("d_c", c_int32),
        ("num_items", c_int32), ("row_chunks", c_int32), ("num_partials", c_int32),
        ("needs_combine", c_int32), ("max_splits", c_int32), ("blocks_per_item", c_int32),
        ("partial_dtype", c_int32), ("plan_ints", c_int64), ("workspace_bytes", c_int64),
        ("grid_wgs", c_int32), ("kv_dtype", c_int32), ("d_r", c_int32), ("max_seq_blocks", c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Rope(ctypes.Structure):
    """mla_rope_t: plain RoPE (factor 1) or YaRN-scaled frequencies."""
    _fields_ = [
        ("base", ctypes.c_double), ("factor", ctypes.c_double), ("orig_ctx", ctypes.c_double),
        ("beta_fast", ctypes.c_double), ("beta_slow", ctypes.c_double), ("mscale", ctypes.c_double),
    ]


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmla.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is not built; run python -m mla_latent_kv_07_amd.build")
    L = ctypes.CDLL(str(LIB_PATH))
    P = c_void_p
    L.mla_decode_plan.argtypes = [P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  P, c_int64, ctypes.POINTER(Plan)]
    L.mla_decode.argtypes = [P, P, c_int32, ctypes.POINTER(CacheDesc), P, c_int32, P, c_int32,
                             c_int32, c_int32, c_float, ctypes.POINTER(Plan), P, P, c_int64, P,
                             P, P]
    L.mla_decode_partial.argtypes = L.mla_decode.argtypes
    L.mla_decode_noalloc.argtypes = [P, P, c_int32, ctypes.POINTER(CacheDesc), P, c_int32, P, c_int32,
                                     c_int32, c_int32, c_float, ctypes.POINTER(Plan), P, P, P, P]
    L.mla_decode_noalloc.restype = c_int32
    L.mla_decode_finish.argtypes = [ctypes.POINTER(Plan), P, P, c_int64, c_int32, P, P, P]
    L.mla_combine_lse.argtypes = [P, P, P, P, c_int32, c_int32, c_int32, P, c_int32, P, P]
    L.mla_absorb_q.argtypes = [P, c_int64, P, P, c_int32, c_int32, c_int32, c_int32, c_int32, P]
    L.mla_absorb_out_workspace.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32]
    L.mla_absorb_out_workspace.restype = c_int64
    L.mla_absorb_out.argtypes = [P, P, P, P, P, P, c_int64, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, P]
    L.mla_gather_paged.argtypes = [ctypes.POINTER(CacheDesc), P, c_int32, P, c_int32, c_int32, P, P]
    L.mla_cache_bytes.argtypes = [ctypes.POINTER(CacheDesc)]
    L.mla_cache_bytes.restype = c_int64
    L.mla_rope_freqs.argtypes = [ctypes.POINTER(Rope), c_int32, P]
    L.mla_cache_append_workspace.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32]
    L.mla_cache_append_workspace.restype = c_int64
    L.mla_cache_append.argtypes = [P, P, c_int32, ctypes.POINTER(CacheDesc), P, c_int32, P, c_int32,
                                   c_int32, c_int32, ctypes.POINTER(Rope), P, c_int64, P]
    L.mla_project_q_workspace.argtypes = [c_int32] * 8
    L.mla_project_q_workspace.restype = c_int64
    L.mla_project_q.argtypes = [P, P, P, P, P, c_int32, P, c_int32, c_int32, c_int32, c_int32,
                                c_int32, c_int32, c_int32, ctypes.POINTER(Rope), P, P, P, c_int64, P]
    L.mla_project_step_workspace.argtypes = [c_int32] * 9
    L.mla_project_step_workspace.restype = c_int64
    L.mla_project_step.argtypes = [P, P, P, P, P, c_int32, ctypes.POINTER(CacheDesc), P, c_int32, P, c_int32,
                                   c_int32, c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(Rope), P, P, P,
                                   c_int64, P]
    L.mla_set_launch_events.argtypes = [P, c_int32]
    L.mla_set_launch_events.restype = c_int32
    L.mla_launch_events_used.argtypes = []
    L.mla_launch_events_used.restype = c_int32
    L.mla_set_debug.argtypes = [c_int32]
    L.mla_set_debug.restype = c_int32
    L.mla_debug.argtypes = []
    L.mla_debug.restype = c_int32
    L.mla_clock_probe.argtypes = [P, c_int32, c_int32, P]
    L.mla_clock_probe.restype = c_int32
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_version.restype = ctypes.c_char_p
    for name in ("mla_decode_plan", "mla_decode", "mla_decode_partial", "mla_decode_finish",
                 "mla_combine_lse", "mla_absorb_q",
                 "mla_absorb_out", "mla_gather_paged", "mla_rope_freqs", "mla_cache_append",
                 "mla_project_q", "mla_project_step"):
        getattr(L, name).restype = c_int32
    _lib = L
    return L


def check(status: int) -> None:
    if status != MLA_OK:
        raise MLAError(status, load().mla_last_error().decode())
