"""Oracle checks (b)-(d) and the decode/combine/gather pins.

Each oracle function is checked against something other than itself: torch's
scaled_dot_product_attention in fp64 (textbook attention), closed forms of
degenerate cases, the un-absorbed multi-head attention the pages start from,
and invariances the definition implies (block-table permutation, causal
truncation, split merging)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from mla_latent_kv_07_amd import inputs as I


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _paged(wl, rows, seed, seq_lens):
    return I.page_cache(wl, _gen(seed), torch.tensor(seq_lens, dtype=torch.int32), rows)


def _fmt(kv):
    return {"f32": O.FMT_F32, "bf16": O.FMT_BF16, "fp8_e4m3": O.FMT_FP8_E4M3, "f16": O.FMT_F16,
            "fp8_e5m2": O.FMT_FP8_E5M2, "fp8_e4m3_row": O.FMT_FP8_E4M3_ROW}[kv]


def _small(kv="bf16", n_h=16, d_c=64, d_r=16, q_len=1, seq=(1, 70, 200)):
    return I.Workload("t", 5, kv, "f32" if kv == "f32" else "bf16", B=len(seq), q_len=q_len,
                      n_h=n_h, d_c=d_c, d_r=d_r, seq_lens=tuple(seq), d_nope=32)


def _rounded_rows(wl, rows):
    """Logical rows as the cache stores them (exact values)."""
    if wl.kv_dtype == "bf16":
        return rows.to(torch.bfloat16).to(torch.float64)
    if wl.kv_dtype == "f16":
        return rows.to(torch.float16).to(torch.float64)
    return rows.to(torch.float64)


@pytest.mark.parametrize("kv,d_c,d_r", [("f32", 64, 16), ("bf16", 64, 16), ("f16", 64, 16),
                                        ("bf16", 512, 64)])
def test_decode_matches_sdpa_fp64(kv, d_c, d_r):
    # one KV head of width D_qk = d_c + d_r with D_v = d_c: small dims, and
    # the DeepSeek-V2 dims (576 / 512)
    wl = _small(kv, d_c=d_c, d_r=d_r)
    g = _gen(11)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    T = wl.B
    q_lat = torch.randn(T, wl.n_h, wl.d_c, generator=g).to(I._TORCH_DT[wl.q_dtype])
    q_rope = torch.randn(T, wl.n_h, wl.d_r, generator=g).to(I._TORCH_DT[wl.q_dtype])
    cache = _paged(wl, rows, 3, wl.seq_lens)
    o, lse = O.decode(cache.pool, _fmt(kv), cache.block_table, cache.seq_lens,
                      q_lat.double(), q_rope.double(), wl.scale)
    logical = _rounded_rows(wl, rows)
    start = 0
    for b, S in enumerate(wl.seq_lens):
        K = logical[start:start + S]                       # [S][d_c + d_r]
        start += S
        V = K[:, :wl.d_c]
        q = torch.cat([q_lat[b], q_rope[b]], dim=-1).double()   # [n_h][d_c + d_r]
        ref = F.scaled_dot_product_attention(
            q[None, :, None, :], K[None, None].expand(1, wl.n_h, S, -1),
            V[None, None].expand(1, wl.n_h, S, -1), scale=wl.scale)[0, :, 0]
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-12)
        ref_lse = torch.logsumexp(wl.scale * (q @ K.T), dim=-1)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_decode_single_token_is_exact():
    wl = _small("bf16", seq=(1, 1))
    g = _gen(12)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    q_lat = torch.randn(2, wl.n_h, wl.d_c, generator=g).to(torch.bfloat16)
    q_rope = torch.randn(2, wl.n_h, wl.d_r, generator=g).to(torch.bfloat16)
    cache = _paged(wl, rows, 4, wl.seq_lens)
    o, lse = O.decode(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens,
                      q_lat.double(), q_rope.double(), wl.scale)
    logical = _rounded_rows(wl, rows).numpy()
    for b in range(2):
        assert np.array_equal(o[b], np.broadcast_to(logical[b, :wl.d_c], o[b].shape))
        s0 = wl.scale * (q_lat[b].double().numpy() @ logical[b, :wl.d_c]
                         + q_rope[b].double().numpy() @ logical[b, wl.d_c:])
        np.testing.assert_allclose(lse[b], s0, rtol=1e-14, atol=1e-14)


def test_decode_zero_query_is_mean():
    wl = _small("bf16", seq=(5, 64, 130))
    rows = I.draw_cache_rows(wl, _gen(13), torch.tensor(wl.seq_lens))
    cache = _paged(wl, rows, 5, wl.seq_lens)
    z1 = torch.zeros(wl.B, wl.n_h, wl.d_c, dtype=torch.float64)
    z2 = torch.zeros(wl.B, wl.n_h, wl.d_r, dtype=torch.float64)
    o, lse = O.decode(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens, z1, z2, wl.scale)
    logical = _rounded_rows(wl, rows).numpy()
    start = 0
    for b, S in enumerate(wl.seq_lens):
        mean = logical[start:start + S, :wl.d_c].mean(axis=0)
        start += S
        np.testing.assert_allclose(o[b], np.broadcast_to(mean, o[b].shape), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(S), rtol=1e-14)


def test_decode_block_table_permutation_invariant():
    wl = _small("bf16", seq=(65, 190, 7))
    g = _gen(14)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    ql = torch.randn(wl.B, wl.n_h, wl.d_c, generator=g).double()
    qr = torch.randn(wl.B, wl.n_h, wl.d_r, generator=g).double()
    a = _paged(wl, rows, 100, wl.seq_lens)
    b = _paged(wl, rows, 200, wl.seq_lens)
    assert not torch.equal(a.block_table, b.block_table)
    oa, la = O.decode(a.pool, O.FMT_BF16, a.block_table, a.seq_lens, ql, qr, wl.scale)
    ob, lb = O.decode(b.pool, O.FMT_BF16, b.block_table, b.seq_lens, ql, qr, wl.scale)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_gather_returns_logical_rows():
    for kv in ("f32", "bf16", "fp8_e4m3", "f16", "fp8_e5m2", "fp8_e4m3_row"):
        wl = _small(kv, seq=(3, 64, 129))
        rows = I.draw_cache_rows(wl, _gen(15), torch.tensor(wl.seq_lens))
        cache = _paged(wl, rows, 6, wl.seq_lens)
        out = O.gather(cache.pool, _fmt(kv), wl.d_c, wl.d_r, cache.block_table, cache.seq_lens, 130)
        start = 0
        for b, S in enumerate(wl.seq_lens):
            got = out[b, :S]
            if kv == "f32":
                want = rows[start:start + S].numpy().view(np.uint8).reshape(S, -1)
            elif kv == "bf16":
                want = rows[start:start + S].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8).reshape(S, -1)
            elif kv == "f16":
                want = rows[start:start + S].to(torch.float16).view(torch.int16).numpy().view(np.uint8).reshape(S, -1)
            elif kv == "fp8_e4m3_row":
                # the whole row's codes, straight from the pool block the table names
                W = wl.d_c + wl.d_r
                want = np.stack([cache.pool[int(cache.block_table[b, p // 64])].numpy()[(p % 64) * W:(p % 64 + 1) * W]
                                 for p in range(S)])
            else:
                # rebuild the row bytes from the pool block the table names:
                # codes of the latent, then the bf16 RoPE key
                want = []
                for p in range(S):
                    blk = cache.pool[int(cache.block_table[b, p // 64])].numpy()
                    slot = p % 64
                    want.append(np.concatenate([blk[slot * wl.d_c:(slot + 1) * wl.d_c],
                                                blk[64 * wl.d_c + slot * 2 * wl.d_r:
                                                    64 * wl.d_c + (slot + 1) * 2 * wl.d_r]]))
                want = np.stack(want)
                kr = rows[start:start + S, wl.d_c:].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
                assert np.array_equal(want[:, wl.d_c:], kr.reshape(S, -1))
            start += S
            assert np.array_equal(got, want), (kv, b)
            assert not out[b, S:].any()


def test_decode_causal_pair_equals_truncated_single():
    # q_len = 2: query t of a sequence of length S sees positions <= S - 2 + t,
    # i.e. it is a one-token decode of the sequence cut to S - 1 + t tokens.
    wl2 = _small("bf16", q_len=2, seq=(2, 65, 129))
    g = _gen(16)
    rows = I.draw_cache_rows(wl2, g, torch.tensor(wl2.seq_lens))
    ql = torch.randn(wl2.B * 2, wl2.n_h, wl2.d_c, generator=g).double()
    qr = torch.randn(wl2.B * 2, wl2.n_h, wl2.d_r, generator=g).double()
    cache = _paged(wl2, rows, 7, wl2.seq_lens)
    o2, l2 = O.decode(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens, ql, qr,
                      wl2.scale, q_len=2)
    for t in range(2):
        sl = cache.seq_lens - 1 + t
        o1, l1 = O.decode(cache.pool, O.FMT_BF16, cache.block_table, sl, ql[t::2], qr[t::2],
                          wl2.scale, q_len=1)
        assert np.array_equal(o2[t::2], o1) and np.array_equal(l2[t::2], l1)


def test_decode_empty_rows():
    # q_len larger than the sequence: the first query sees nothing.
    wl = _small("bf16", q_len=2, seq=(1, 0))
    rows = I.draw_cache_rows(wl, _gen(17), torch.tensor(wl.seq_lens))
    cache = _paged(wl, rows, 8, wl.seq_lens)
    ql = torch.ones(4, wl.n_h, wl.d_c, dtype=torch.float64)
    qr = torch.ones(4, wl.n_h, wl.d_r, dtype=torch.float64)
    o, l = O.decode(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens, ql, qr, wl.scale, q_len=2)
    assert np.all(l[0] == -np.inf) and not o[0].any()
    assert np.all(np.isfinite(l[1]))
    assert np.all(l[2:] == -np.inf) and not o[2:].any()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_combine_split_invariance(seed):
    wl = _small("bf16", seq=(1, 77, 300, 64))
    g = _gen(20 + seed)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    ql = torch.randn(wl.B, wl.n_h, wl.d_c, generator=g).double()
    qr = torch.randn(wl.B, wl.n_h, wl.d_r, generator=g).double()
    cache = _paged(wl, rows, 9, wl.seq_lens)
    full_o, full_l = O.decode(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens, ql, qr, wl.scale)
    rng = np.random.default_rng(seed)
    n_split = 4
    cuts = []
    for S in wl.seq_lens:
        c = np.sort(rng.integers(0, S + 1, size=n_split - 1))
        cuts.append(np.concatenate([[0], c, [S]]))
    bounds = [(np.array([c[k] for c in cuts], np.int32), np.array([c[k + 1] for c in cuts], np.int32))
              for k in range(n_split)]
    op, lp = O.decode_splits(cache.pool, O.FMT_BF16, cache.block_table, cache.seq_lens, ql, qr,
                             wl.scale, bounds)
    o, l = O.combine(op, lp)
    np.testing.assert_allclose(o, full_o.reshape(-1, wl.d_c), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, full_l.reshape(-1), rtol=1e-13, atol=1e-13)


def test_fp8_cache_reads_codes_times_block_scale():
    wl = _small("fp8_e4m3", q_len=2, seq=(3, 100, 200))
    g = _gen(30)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    ql = torch.randn(wl.B * 2, wl.n_h, wl.d_c, generator=g).double()
    qr = torch.randn(wl.B * 2, wl.n_h, wl.d_r, generator=g).double()
    cache = _paged(wl, rows, 10, wl.seq_lens)
    o8, l8 = O.decode(cache.pool, O.FMT_FP8_E4M3, cache.block_table, cache.seq_lens, ql, qr,
                      wl.scale, q_len=2, block_scales=cache.block_scales)
    # same values through torch's fp8 decode, stored as an fp32 cache
    nb = cache.num_blocks
    codes = cache.pool[:, :64 * wl.d_c].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
    c = codes.view(nb, 64, wl.d_c) * cache.block_scales[:, None, None]
    kr = cache.pool[:, 64 * wl.d_c:].contiguous().view(torch.bfloat16).to(torch.float32).view(nb, 64, wl.d_r)
    pool32 = torch.cat([c, kr], dim=2).contiguous().view(torch.uint8).view(nb, -1)
    o32, l32 = O.decode(pool32, O.FMT_F32, cache.block_table, cache.seq_lens, ql, qr, wl.scale, q_len=2)
    # fp32 rounding of code * scale is the only difference
    np.testing.assert_allclose(o8, o32, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(l8, l32, rtol=1e-6, atol=1e-6)
    assert np.all(np.isfinite(o8))


@pytest.mark.parametrize("kv,code_dt", [("fp8_e5m2", torch.float8_e5m2), ("fp8_e4m3_row", torch.float8_e4m3fn)])
def test_other_fp8_caches_read_codes_times_block_scale(kv, code_dt):
    """e5m2 latent codes (+ bf16 k^R), and the whole row in e4m3 under one
    block scale, decoded by torch's fp8 casts and stored as an fp32 cache."""
    wl = _small(kv, q_len=2, seq=(3, 100, 200))
    g = _gen(31)
    rows = I.draw_cache_rows(wl, g, torch.tensor(wl.seq_lens))
    ql = torch.randn(wl.B * 2, wl.n_h, wl.d_c, generator=g).double()
    qr = torch.randn(wl.B * 2, wl.n_h, wl.d_r, generator=g).double()
    cache = _paged(wl, rows, 10, wl.seq_lens)
    fmt = _fmt(kv)
    o8, l8 = O.decode(cache.pool, fmt, cache.block_table, cache.seq_lens, ql, qr,
                      wl.scale, q_len=2, block_scales=cache.block_scales)
    nb, W = cache.num_blocks, wl.d_c + wl.d_r
    sc = cache.block_scales[:, None, None]
    if kv == "fp8_e4m3_row":
        full = cache.pool.contiguous().view(code_dt).to(torch.float32).view(nb, 64, W) * sc
    else:
        c = cache.pool[:, :64 * wl.d_c].contiguous().view(code_dt).to(torch.float32).view(nb, 64, wl.d_c) * sc
        kr = cache.pool[:, 64 * wl.d_c:].contiguous().view(torch.bfloat16).to(torch.float32).view(nb, 64, wl.d_r)
        full = torch.cat([c, kr], dim=2)
    pool32 = full.contiguous().view(torch.uint8).view(nb, -1)
    o32, l32 = O.decode(pool32, O.FMT_F32, cache.block_table, cache.seq_lens, ql, qr, wl.scale, q_len=2)
    np.testing.assert_allclose(o8, o32, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(l8, l32, rtol=1e-6, atol=1e-6)
    assert np.all(np.isfinite(o8))
