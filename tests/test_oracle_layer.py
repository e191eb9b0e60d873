"""Oracle layer pins: RoPE, the score decomposition (check b), W^UK absorption
(check c), W^UV W^O fusion (check d) and the absorbed path against brute-force
un-absorbed multi-head attention on the tiny fp32 layer."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from mla_latent_kv_07_amd import inputs as I


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(0)
    q = rng.normal(size=64)
    k = rng.normal(size=64)
    for p in (0, 1, 17, 4095):
        assert np.linalg.norm(O.rope(q, np.array(p))) == pytest.approx(np.linalg.norm(q), rel=1e-14)
    # rotated dot product depends only on the position difference
    d1 = O.rope(q, np.array(100)) @ O.rope(k, np.array(90))
    d2 = O.rope(q, np.array(1010)) @ O.rope(k, np.array(1000))
    assert d1 == pytest.approx(d2, rel=1e-11)
    assert O.rope(q, np.array(0)) == pytest.approx(q)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.normal(size=16)
    p = 37
    z = x[0::2] + 1j * x[1::2]
    theta = 10000.0 ** (-np.arange(8) * 2 / 16)
    w = z * np.exp(1j * p * theta)
    r = O.rope(x, np.array(p))
    np.testing.assert_allclose(r[0::2], w.real, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r[1::2], w.imag, rtol=1e-13, atol=1e-14)


def test_score_decomposition():
    # check (b): concatenated score = content part + position part
    rng = np.random.default_rng(2)
    for _ in range(5):
        qc, qr, kc, kr = rng.normal(size=128), rng.normal(size=64), rng.normal(size=128), rng.normal(size=64)
        full, content, pos = O.score_split(qc, qr, kc, kr)
        assert full == pytest.approx(content + pos, rel=1e-13, abs=1e-13)


def test_absorption_equivalence():
    # check (c): q^C . (c W^UK_i) == (q^C W^UK_i^T) . c, for every head
    rng = np.random.default_rng(3)
    n_h, d_c, d_nope = 4, 64, 32
    w_uk = rng.normal(size=(n_h, d_c, d_nope))
    q = rng.normal(size=(3, n_h, d_nope))
    c = rng.normal(size=(10, d_c))
    qt = O.absorb_q(q, w_uk)
    for i in range(n_h):
        k_explicit = c @ w_uk[i]                       # reconstructed content keys
        np.testing.assert_allclose(q[:, i] @ k_explicit.T, qt[:, i] @ c.T, rtol=1e-12, atol=1e-12)


def test_fusion_equivalence():
    # check (d): sum_i o_i (W^UV_i W^O_i) == sum_i (o_i W^UV_i) W^O_i
    rng = np.random.default_rng(4)
    n_h, d_c, d_v, d = 4, 64, 32, 96
    w_uv = rng.normal(size=(n_h, d_c, d_v))
    w_o = rng.normal(size=(n_h * d_v, d))
    o = rng.normal(size=(5, n_h, d_c))
    _, out = O.absorb_out(o, w_uv, w_o)
    fused = O.absorb_out_fused(o, O.fused_out_weights(w_uv, w_o))
    np.testing.assert_allclose(fused, out, rtol=1e-11, atol=1e-11)
    # and the unfused path equals concat(u) @ W^O done as one matrix product
    u = np.einsum("thc,hcv->thv", o, w_uv)
    np.testing.assert_allclose(out, u.reshape(5, -1) @ w_o, rtol=1e-11, atol=1e-11)


def test_unabsorbed_mha_matches_sdpa():
    rng = np.random.default_rng(5)
    S, n_h, d_c, d_r, d_nope, d_v, d = 40, 3, 16, 8, 8, 8, 12
    c = rng.normal(size=(S, d_c))
    kr = rng.normal(size=(S, d_r))
    q_nope = rng.normal(size=(1, n_h, d_nope))
    q_rope = rng.normal(size=(1, n_h, d_r))
    w_uk = rng.normal(size=(n_h, d_c, d_nope))
    w_uv = rng.normal(size=(n_h, d_c, d_v))
    w_o = rng.normal(size=(n_h * d_v, d))
    scale = 0.3
    _, u, out, lse = O.unabsorbed_mha(c, kr, q_nope, q_rope, w_uk, w_uv, w_o, scale, [S - 1])
    for i in range(n_h):
        K = torch.from_numpy(np.concatenate([c @ w_uk[i], kr], 1))
        V = torch.from_numpy(c @ w_uv[i])
        q = torch.from_numpy(np.concatenate([q_nope[0, i], q_rope[0, i]]))
        ref = F.scaled_dot_product_attention(q[None, None, None], K[None, None], V[None, None], scale=scale)
        np.testing.assert_allclose(u[0, i], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[0], u[0].reshape(-1) @ w_o, rtol=1e-12)


def build_tiny_layer():
    """The tiny fp32 layer: cache and queries from hidden states through the
    oracle's projections and RoPE, positions 0..S-1, query = last token."""
    wl = I.C1
    L = I.make_layer_inputs(wl)
    w = {k: v.numpy().astype(np.float64) for k, v in L["weights"].items()}
    h = L["hidden"].numpy().astype(np.float64)
    S = int(L["seq_lens"][0])
    c, kr = O.project_kv(h, w["w_dkv"], wl.d_c, np.arange(S))
    q_nope, q_rope = O.project_queries_direct(h[S - 1:S], w["w_q"], wl.n_h, wl.d_nope, wl.d_r,
                                              np.array([S - 1]))
    return wl, L, w, c, kr, q_nope, q_rope


def test_tiny_layer_absorbed_equals_unabsorbed():
    wl, L, w, c, kr, q_nope, q_rope = build_tiny_layer()
    S = c.shape[0]
    rows = torch.from_numpy(np.concatenate([c, kr], 1)).to(torch.float32)
    cache = I.page_cache(wl, L["generator"], L["seq_lens"], rows)
    # absorbed path in the oracle, on the fp32-stored cache and fp64 queries
    q_lat = O.absorb_q(q_nope, w["w_uk"])
    o_lat, lse = O.decode(cache.pool, O.FMT_F32, cache.block_table, cache.seq_lens,
                          q_lat, q_rope, wl.scale)
    _, out = O.absorb_out(o_lat, w["w_uv"], w["w_o"])
    # brute-force multi-head attention with reconstructed K and V, on the same
    # stored (fp32-rounded) rows
    c32 = rows[:, :wl.d_c].double().numpy()
    kr32 = rows[:, wl.d_c:].double().numpy()
    o_ref, u_ref, out_ref, lse_ref = O.unabsorbed_mha(c32, kr32, q_nope, q_rope, w["w_uk"], w["w_uv"],
                                                      w["w_o"], wl.scale, [S - 1])
    np.testing.assert_allclose(o_lat, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, out_ref, rtol=1e-10, atol=1e-11)
    # and the offline-fused output weights give the same layer output
    fused = O.absorb_out_fused(o_lat, O.fused_out_weights(w["w_uv"], w["w_o"]))
    np.testing.assert_allclose(fused, out_ref, rtol=1e-10, atol=1e-11)


def test_latent_equals_lowrank_mha_without_rope():
    # Without the RoPE part, attention over the latent cache is exactly MHA
    # whose keys are the low-rank products c W^UK (thakicloud page, section
    # on RoPE breaking latent equivalence): set d_R terms to zero.
    wl, L, w, c, kr, q_nope, q_rope = build_tiny_layer()
    z_r = np.zeros_like(q_rope)
    q_lat = O.absorb_q(q_nope, w["w_uk"])
    rows = torch.from_numpy(np.concatenate([c, np.zeros_like(kr)], 1)).to(torch.float32)
    cache = I.page_cache(wl, L["generator"], L["seq_lens"], rows)
    o_lat, _ = O.decode(cache.pool, O.FMT_F32, cache.block_table, cache.seq_lens, q_lat, z_r, wl.scale)
    c32 = rows[:, :wl.d_c].double().numpy()
    o_ref, _, _, _ = O.unabsorbed_mha(c32, np.zeros_like(kr), q_nope, z_r, w["w_uk"], w["w_uv"],
                                      w["w_o"], wl.scale, [c.shape[0] - 1])
    np.testing.assert_allclose(o_lat, o_ref, rtol=1e-11, atol=1e-12)
