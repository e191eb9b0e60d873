"""mla_decode_noalloc (the decode entry point that allocates nothing) against
mla_decode with a caller workspace, through the C ABI: two calls in a row on
one GPU, the second with a smaller batch, each bit-identical to mla_decode
(both run the same kernels) and within the bf16 bound of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from mla_latent_kv_07_amd import _lib as L
from mla_latent_kv_07_amd import api
from mla_latent_kv_07_amd import inputs as I

from parity import DEV, compare_decode, say, to_device

pytestmark = pytest.mark.gpu


def _noalloc(d, cache, bt, sl, ql, qr, dec):
    wl = d.wl
    T = wl.B * wl.q_len
    o = torch.empty((T, wl.n_h, wl.d_c), dtype=ql.dtype, device=DEV)
    lse = torch.empty((T, wl.n_h), dtype=torch.float32, device=DEV)
    desc = cache.desc()
    P = ctypes.c_void_p
    st = L.load().mla_decode_noalloc(P(ql.data_ptr()), P(qr.data_ptr()), L.DT_BF16, ctypes.byref(desc),
                                     P(bt.data_ptr()), bt.stride(0), P(sl.data_ptr()), wl.B, wl.q_len,
                                     wl.n_h, ctypes.c_float(d.scale), ctypes.byref(dec.info),
                                     P(dec.plan_dev.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()),
                                     P(torch.cuda.current_stream().cuda_stream))
    L.check(st)
    return o, lse


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_noalloc_matches_workspace_decode_twice(kv):
    cases = [((3000, 700, 4096, 1, 0, 2500), 1, 8), ((640, 65), 2 if kv == "fp8_e4m3" else 1, 4)]
    for seq, q_len, seed in cases:
        d = I.make_decode_inputs(I.Workload(f"noalloc_{kv}_{len(seq)}", seed, kv, "bf16", B=len(seq),
                                            q_len=q_len, n_h=128, d_c=512, d_r=64, seq_lens=seq,
                                            heavy_frac=0.01))
        cache, bt, sl, ql, qr = to_device(d)
        # few compute units: several splits per sequence, so the partials
        # (in the scratch array) and the combine are used
        dec = api.Decoder(d.cache.seq_lens, q_len, 128, 512, 64, kv, DEV, cus=16)
        assert dec.info.num_partials > 0
        assert dec.info.workspace_bytes <= L.NOALLOC_SCRATCH_BYTES
        o_ref, l_ref = dec(ql, qr, cache, bt, sl, d.scale)
        o, lse = _noalloc(d, cache, bt, sl, ql, qr, dec)
        torch.cuda.synchronize()
        say(f"  {kv} B={len(seq)} q_len={q_len}: workspace {dec.info.workspace_bytes} B")
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        compare_decode(d, o, lse)


def test_noalloc_rejects_plans_beyond_the_scratch():
    # a plan whose partials exceed the scratch maximum is refused before any
    # HIP call (a host-side struct copy with a large workspace figure)
    info, _ = api.decode_plan([100, 200], 1, 128, 512, 64, "bf16", 4)
    info.workspace_bytes = L.NOALLOC_SCRATCH_BYTES + 256
    A = ctypes.c_void_p(1 << 20)
    desc = L.CacheDesc(1 << 20, None, 10, 64, 512, 64, L.DT_BF16, 0)
    st = L.load().mla_decode_noalloc(A, A, L.DT_BF16, ctypes.byref(desc), A, 64, A, 2, 1, 128,
                                     ctypes.c_float(0.07), ctypes.byref(info), A, A, A, None)
    assert st == L.MLA_ERR_WORKSPACE
    assert b"scratch" in L.load().mla_last_error()
