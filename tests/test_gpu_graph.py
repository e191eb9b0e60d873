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


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_project_step_graph_replays_match_eager(kv):
    """mla_project_step captured in a HIP graph (its three launches): each of
    three replays, from the same starting cache, writes the same q_lat,
    q_rope, cache rows and block scales as the eager call, with an eager
    call on other inputs (same workspace, another cache) between replays."""
    B, q_len, dm, ql, n_h, dn, dc, dr = 5, 3, 256, 128, 4, 128, 512, 64
    T = B * q_len
    g = torch.Generator().manual_seed(43)
    bf = torch.bfloat16
    rnd = lambda *shape, std=1.0: (torch.randn(*shape, generator=g) * std).to(bf).to(DEV)
    h, h2 = rnd(T, dm), rnd(T, dm)
    w_dkvq = rnd(dm, ql + dc + dr, std=dm ** -0.5)
    w_uq, w_qr, w_uk = rnd(ql, n_h * dn, std=ql ** -0.5), rnd(dm, n_h * dr, std=dm ** -0.5), rnd(n_h, dc, dn, std=dc ** -0.5)
    nblk = 4
    bt = torch.randperm(B * nblk + 3, generator=g)[:B * nblk].view(B, nblk).to(torch.int32).to(DEV)
    pos0 = torch.randint(0, 190, (B,), generator=g, dtype=torch.int32).to(DEV)
    bb = 64 * (dc + dr) * 2 if kv == "bf16" else 64 * dc + 64 * dr * 2   # bytes of one paged block
    pool0 = torch.randint(0, 256, (B * nblk + 3, bb), generator=g, dtype=torch.uint8).to(DEV)
    scales0 = (torch.rand(B * nblk + 3, generator=g) + 0.5).to(DEV) if kv != "bf16" else None
    mk = lambda: api.DeviceCache(pool0.clone(), None if scales0 is None else scales0.clone(), kv, dc, dr)
    cfg = api.rope()
    need = api.project_step_workspace_bytes(B, q_len, dm, ql, n_h, dn, dc, dr, bf)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = lambda: (torch.empty((T, n_h, dc), dtype=bf, device=DEV), torch.empty((T, n_h, dr), dtype=bf, device=DEV))

    ref_cache, (ql_ref, qr_ref) = mk(), out()
    api.project_step(h, w_dkvq, w_uq, w_qr, w_uk, ref_cache, bt, pos0, q_len, n_h, dn, cfg, ql_ref, qr_ref, ws)
    torch.cuda.synchronize()

    cache, (ql_g, qr_g) = mk(), out()
    other, (ql_o, qr_o) = mk(), out()
    s0 = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(s0)
    with torch.cuda.stream(side):                        # warm-up off the capture
        api.project_step(h, w_dkvq, w_uq, w_qr, w_uk, cache, bt, pos0, q_len, n_h, dn, cfg, ql_g, qr_g, ws,
                         stream=side)
    s0.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.project_step(h, w_dkvq, w_uq, w_qr, w_uk, cache, bt, pos0, q_len, n_h, dn, cfg, ql_g, qr_g, ws,
                         stream=torch.cuda.current_stream())
    torch.cuda.synchronize()

    for _ in range(3):
        cache.pool.copy_(pool0)
        if scales0 is not None:
            cache.block_scales.copy_(scales0)
        ql_g.fill_(float("nan"))
        qr_g.fill_(float("nan"))
        api.project_step(h2, w_dkvq, w_uq, w_qr, w_uk, other, bt, pos0, q_len, n_h, dn, cfg, ql_o, qr_o, ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ql_g, ql_ref) and torch.equal(qr_g, qr_ref)
        assert torch.equal(cache.pool, ref_cache.pool)
        if scales0 is not None:
            assert torch.equal(cache.block_scales, ref_cache.block_scales)
