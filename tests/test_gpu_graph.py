"""Decode calls captured in a HIP graph (through torch.cuda.CUDAGraph): mla_decode
with a caller workspace and mla_decode_noalloc, each replayed three times with
an eager decode of other inputs in between (which overwrites the workspace or
the scratch array and the plan's partial slots), every replay bit-identical to
the eager call on the same inputs.  The batch is split over few compute units
so that the partials and the combine are part of the captured work; a bf16
cache runs the 16-bit MFMA decode, an e4m3 one the 8-bit decode."""
import ctypes

import pytest
import torch

from mla_latent_kv_07_amd import _lib as L
from mla_latent_kv_07_amd import api
from mla_latent_kv_07_amd import inputs as I

from parity import DEV, to_device

pytestmark = pytest.mark.gpu

SEQ = (3000, 700, 1, 0, 2500)


def _inputs(seed, kv):
    d = I.make_decode_inputs(I.Workload(f"graph_{seed}", seed, kv, "bf16", B=len(SEQ), q_len=1, n_h=128,
                                        d_c=512, d_r=64, seq_lens=SEQ))
    return d, to_device(d)


def _call(entry, d, dev_in, dec, o, lse, stream):
    cache, bt, sl, ql, qr = dev_in
    desc = cache.desc()
    P = ctypes.c_void_p
    lib = L.load()
    common = (P(ql.data_ptr()), P(qr.data_ptr()), L.DT_BF16, ctypes.byref(desc), P(bt.data_ptr()), bt.stride(0),
              P(sl.data_ptr()), d.wl.B, 1, 128, ctypes.c_float(d.scale), ctypes.byref(dec.info),
              P(dec.plan_dev.data_ptr()))
    if entry == "noalloc":
        L.check(lib.mla_decode_noalloc(*common, P(o.data_ptr()), P(lse.data_ptr()), P(stream.cuda_stream)))
    else:
        L.check(lib.mla_decode(*common, P(dec.workspace.data_ptr()), dec.workspace.numel(), P(o.data_ptr()),
                               P(lse.data_ptr()), P(stream.cuda_stream)))


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_graph_replays_match_eager(entry, kv):
    d, dev_in = _inputs(41, kv)
    d2, dev_in2 = _inputs(42, kv)                 # same lengths, other values
    dec = api.Decoder(d.cache.seq_lens, 1, 128, 512, 64, kv, DEV, cus=16)
    assert dec.info.num_partials > 0 and dec.info.needs_combine
    T = d.wl.B
    new = lambda: (torch.empty((T, 128, 512), dtype=torch.bfloat16, device=DEV),
                   torch.empty((T, 128), dtype=torch.float32, device=DEV))
    o_ref, l_ref = new()
    o2, l2 = new()
    s0 = torch.cuda.current_stream()
    _call(entry, d, dev_in, dec, o_ref, l_ref, s0)       # eager reference (and the scratch lookup)
    torch.cuda.synchronize()

    o_g, l_g = new()
    side = torch.cuda.Stream()
    side.wait_stream(s0)
    with torch.cuda.stream(side):                        # warm-up off the capture, as torch asks
        _call(entry, d, dev_in, dec, o_g, l_g, side)
    s0.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(entry, d, dev_in, dec, o_g, l_g, torch.cuda.current_stream())
    torch.cuda.synchronize()

    for _ in range(3):
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        _call(entry, d2, dev_in2, dec, o2, l2, s0)       # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(l_g, l_ref)
    assert not torch.equal(o2, o_ref)
