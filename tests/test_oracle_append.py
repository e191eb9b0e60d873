"""Oracle pins for the cache append, the query production and YaRN-scaled
RoPE: each checked against a format definition, a library cast, a limit the
method reduces to in closed form, or an independently written path."""
import math

import numpy as np
import pytest
import torch

import oracle as O

BLK = O.BLOCK


# ---------------------------------------------------------------- bf16 rounding

def test_f64_to_bf16_matches_torch_on_fp32_values():
    # for values that are exact in fp32, one rounding from fp64 equals
    # torch's fp32 -> bf16 cast (round to nearest even)
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000) * 1e-39,                  # subnormal range
        [0.0, -0.0, 3.38e38, -3.39e38, 1e38, np.inf, -np.inf],
    ]).astype(np.float32)
    # exact ties: 8 significant bits + a half ulp
    m = rng.integers(128, 256, 4000).astype(np.float64)
    e = rng.integers(-100, 100, 4000)
    ties = np.ldexp(m + 0.5, e).astype(np.float32)
    v = np.concatenate([v, ties, -ties])
    ours = O.f64_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_is_nearest_for_fp64_values():
    # values with more than fp32's precision: the result is one of the two
    # neighbouring bf16 values (decoded by the independently pinned decoder)
    # and no farther than the other one
    rng = np.random.default_rng(12)
    x = rng.standard_normal(5000) * 10.0 ** rng.integers(-20, 20, 5000)
    bits = O.f64_to_bf16(x)
    got = O.bf16_bits_to_f64(bits)
    up = O.bf16_bits_to_f64((bits.astype(np.int32) + np.where(np.abs(got) < np.abs(x), 1, -1)).astype(np.uint16))
    assert np.all(np.abs(got - x) <= np.abs(up - x))
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0 ** -8)


# ---------------------------------------------------------------- YaRN RoPE

def test_yarn_factor_one_is_plain_rope():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((7, 64))
    pos = rng.integers(0, 200000, 7)
    inv = O.rope_inv_freq(64, 10000.0, factor=1.0)
    assert np.array_equal(O.rope(x, pos, inv_freq=inv), O.rope(x, pos))


def test_yarn_limits_are_interpolation_and_identity():
    # pairs that turn less than beta_slow times over the original context are
    # position-interpolated (plain RoPE at p / s); pairs that turn more than
    # beta_fast times keep plain RoPE at p
    d, base, s, L, bf, bs = 64, 10000.0, 40.0, 4096.0, 32.0, 1.0
    inv = O.rope_inv_freq(d, base, s, L, bf, bs)
    theta = O.rope_inv_freq(d, base)
    r = L * theta / (2 * math.pi)
    lo, hi = r <= bs, r >= bf
    assert lo.any() and hi.any() and (~lo & ~hi).any()
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, d))
    pos = rng.integers(0, 160000, 5).astype(np.float64)
    got = O.rope(x, pos, inv_freq=inv)
    interp = O.rope(x, pos / s)
    plain = O.rope(x, pos)
    for j in range(d // 2):
        sl = slice(2 * j, 2 * j + 2)
        if lo[j]:
            np.testing.assert_allclose(got[:, sl], interp[:, sl], rtol=0, atol=1e-9)
        if hi[j]:
            np.testing.assert_allclose(got[:, sl], plain[:, sl], rtol=0, atol=1e-9)
    # in between: strictly between the two limits, and decreasing in j
    mid = ~lo & ~hi
    assert np.all(inv[mid] < theta[mid]) and np.all(inv[mid] > theta[mid] / s)
    assert np.all(np.diff(inv) < 0)


def test_yarn_rope_is_relative_and_scales_norm():
    inv = O.rope_inv_freq(64, 10000.0, 40.0, 4096.0, 32.0, 1.0)
    rng = np.random.default_rng(15)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    ms = 1.0 + 0.1 * math.log(40.0)
    dots = []
    for m, n in [(100, 40), (130060, 130000), (60, 0)]:
        dots.append(O.rope(q, m, inv_freq=inv, mscale=ms) @ O.rope(k, n, inv_freq=inv, mscale=ms))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(O.rope(q, 777, inv_freq=inv, mscale=ms)),
                               ms * np.linalg.norm(q), rtol=1e-12)


# ---------------------------------------------------------------- cache append

def _empty_cache(fmt, d_c, d_r, num_blocks, rng):
    bb = O.block_bytes(fmt, d_c, d_r)
    pool = rng.integers(0, 256, (num_blocks, bb), dtype=np.uint8)   # arbitrary old bytes
    scales = rng.random(num_blocks).astype(np.float32) + 0.5
    return pool, scales


def _append_all(fmt, lens, q_lens, d_c=32, d_r=16, d_model=48, seed=0, yarn=None):
    """Append every position of each sequence over calls of the given q_len
    values; returns what a test needs."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    nblk = [(L + BLK - 1) // BLK for L in lens]
    num_blocks = sum(nblk) + 3
    perm = rng.permutation(num_blocks)
    bt = np.full((B, max(nblk)), -1, np.int32)
    k = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    pool, scales = _empty_cache(fmt, d_c, d_r, num_blocks, rng)
    pool0 = pool.copy()
    w = rng.standard_normal((d_model, d_c + d_r)) / math.sqrt(d_model)
    inv, ms = (None, 1.0) if yarn is None else yarn
    H = rng.standard_normal((B, max(lens), d_model))
    pos = np.zeros(B, np.int64)
    # the given call sizes, then single tokens until every sequence is full;
    # a call appends the same count to every sequence it covers (sequences
    # without room sit the call out)
    calls = list(q_lens) + [1] * max(lens)
    for ql in calls:
        live = [b for b in range(B) if pos[b] + ql <= lens[b]]
        if not live:
            continue
        h = np.stack([H[b, pos[b]:pos[b] + ql] for b in live]).reshape(-1, d_model)
        O.cache_append(pool, scales, fmt, d_c, d_r, bt[live], pos[live], ql, h, w,
                       inv_freq=inv, mscale=ms)
        pos[live] += ql
    assert np.array_equal(pos, lens), (pos, lens)
    return dict(pool=pool, pool0=pool0, scales=scales, bt=bt, w=w, H=H, lens=np.array(lens),
                d_c=d_c, d_r=d_r, inv=inv, ms=ms)


def _touched(d, fmt):
    """Mask of pool bytes that belong to written slots (and, for fp8, the codes
    of every written block)."""
    pool = d["pool"]
    m = np.zeros(pool.shape, bool)
    rb = O.block_bytes(fmt, d["d_c"], d["d_r"]) // BLK
    for b, L in enumerate(d["lens"]):
        for p in range(L):
            blk, sl = d["bt"][b, p // BLK], p % BLK
            if fmt == O.FMT_FP8_E4M3_ROW:
                W = d["d_c"] + d["d_r"]
                m[blk, sl * W:(sl + 1) * W] = True
            elif fmt in O.FP8_SPLIT:
                m[blk, sl * d["d_c"]:(sl + 1) * d["d_c"]] = True
                off = BLK * d["d_c"] + sl * 2 * d["d_r"]
                m[blk, off:off + 2 * d["d_r"]] = True
            else:
                m[blk, sl * rb:(sl + 1) * rb] = True
    return m


@pytest.mark.parametrize("fmt", [O.FMT_BF16, O.FMT_F32, O.FMT_F16])
def test_append_writes_rounded_projected_rows(fmt):
    lens = [1, 64, 65, 130, 7]
    d = _append_all(fmt, lens, [1, 2, 3, 64, 1, 1, 5, 64, 64, 64, 1, 1, 1, 1, 1, 1, 1, 1], seed=1)
    # every written row is the single rounding of project_kv's exact row
    rows = O.gather(d["pool"], fmt, d["d_c"], d["d_r"], d["bt"], d["lens"], max(lens))
    for b, L in enumerate(lens):
        c, kr = O.project_kv(d["H"][b, :L], d["w"], d["d_c"], np.arange(L))
        exact = np.concatenate([c, kr], axis=1)
        if fmt == O.FMT_BF16:
            want = O.f64_to_bf16(exact).view(np.uint8).reshape(L, -1)
        elif fmt == O.FMT_F16:
            want = O.f64_to_f16(exact).view(np.uint8).reshape(L, -1)
        else:
            want = exact.astype(np.float32).view(np.uint8).reshape(L, -1)
        assert np.array_equal(rows[b, :L], want)
    # nothing else in the pool changed
    m = _touched(d, fmt)
    assert np.array_equal(d["pool"][~m], d["pool0"][~m])


def test_append_yarn_rows_use_the_scaled_frequencies():
    inv = O.rope_inv_freq(16, 10000.0, 8.0, 64.0, 8.0, 1.0)
    ms = 1.0 + 0.1 * math.log(8.0)
    d = _append_all(O.FMT_BF16, [70, 3], [2] * 40, seed=2, yarn=(inv, ms))
    rows = O.gather(d["pool"], O.FMT_BF16, 32, 16, d["bt"], d["lens"], 70)
    z = d["H"][0, :70] @ d["w"]
    kr = O.rope(z[:, 32:], np.arange(70), inv_freq=inv) * ms
    want = O.f64_to_bf16(kr)
    got = rows[0, :70, 64:].copy().view(np.uint16)
    assert np.array_equal(got, want)


def test_append_fp8_whole_block_scale_and_codes():
    # one call fills whole blocks: scale = amax / 448 of the block, codes are
    # the e4m3 rounding of c / scale, k^R is bf16
    d = _append_all(O.FMT_FP8_E4M3, [64, 128], [64, 64], seed=3)
    for b, L in enumerate([64, 128]):
        c, kr = O.project_kv(d["H"][b, :L], d["w"], 32, np.arange(L))
        for lb in range(L // BLK):
            blk = d["bt"][b, lb]
            cb = c[lb * BLK:(lb + 1) * BLK]
            sc = np.float32(np.abs(cb).max() / 448.0)
            assert d["scales"][blk] == sc
            codes = d["pool"][blk, :BLK * 32].reshape(BLK, 32)
            assert np.array_equal(codes, O.f64_to_e4m3(cb / float(sc)))
            val = O.e4m3_to_f64(codes) * float(sc)
            # within half an e4m3 step (3 mantissa bits) or the subnormal step
            bound = np.maximum(np.abs(cb) * 2.0 ** -4, 2.0 ** -10 * float(sc)) * 1.0000001
            assert np.all(np.abs(val - cb) <= bound)
            krb = d["pool"][blk, BLK * 32:].copy().view(np.uint16).reshape(BLK, 16)
            assert np.array_equal(krb, O.f64_to_bf16(kr[lb * BLK:(lb + 1) * BLK]))


def test_append_fp8_scale_grows_and_reencodes():
    rng = np.random.default_rng(4)
    d_c, d_r, dm = 32, 16, 48
    bt = np.array([[2]], np.int32)
    pool, scales = _empty_cache(O.FMT_FP8_E4M3, d_c, d_r, 4, rng)
    w = rng.standard_normal((dm, d_c + d_r)) / math.sqrt(dm)
    h_small = rng.standard_normal((3, dm)) * 0.01
    h_big = rng.standard_normal((1, dm)) * 5.0
    O.cache_append(pool, scales, O.FMT_FP8_E4M3, d_c, d_r, bt, np.array([0]), 3, h_small, w)
    s1 = float(scales[2])
    codes1 = pool[2, :3 * d_c].copy()
    # an append that does not raise the amax leaves earlier codes alone
    O.cache_append(pool, scales, O.FMT_FP8_E4M3, d_c, d_r, bt, np.array([3]), 1, h_small[:1] * 0.5, w)
    assert float(scales[2]) == s1 and np.array_equal(pool[2, :3 * d_c], codes1)
    # a large token raises the scale; the four earlier rows are re-encoded
    O.cache_append(pool, scales, O.FMT_FP8_E4M3, d_c, d_r, bt, np.array([4]), 1, h_big, w)
    s2 = float(scales[2])
    c_big = (h_big @ w)[:, :d_c]
    assert s2 == float(np.float32(np.abs(c_big).max() / 448.0)) and s2 > s1
    exact_old = np.concatenate([(h_small @ w)[:, :d_c], (h_small[:1] * 0.5 @ w)[:, :d_c]])
    val = O.e4m3_to_f64(pool[2, :4 * d_c].reshape(4, d_c)) * s2
    # two roundings: the first at scale s1, the re-encoding at s2
    bound = (np.abs(exact_old) * 2.0 ** -4 + 2.0 ** -10 * s1) + (np.abs(exact_old) * 2.0 ** -3 + 2.0 ** -10 * s2)
    assert np.all(np.abs(val - exact_old) <= bound)
    # untouched: other blocks, and slots past the written ones
    assert np.array_equal(pool[2, 5 * d_c:BLK * d_c], _empty_cache(O.FMT_FP8_E4M3, d_c, d_r, 4,
                                                                     np.random.default_rng(4))[0][2, 5 * d_c:BLK * d_c])


def test_append_fp8_all_zero_block_takes_scale_one():
    rng = np.random.default_rng(5)
    pool, scales = _empty_cache(O.FMT_FP8_E4M3, 32, 16, 2, rng)
    O.cache_append(pool, scales, O.FMT_FP8_E4M3, 32, 16, np.array([[1]], np.int32), np.array([0]), 2,
                   np.zeros((2, 8)), rng.standard_normal((8, 48)))
    assert scales[1] == 1.0 and not pool[1, :64].any()


# ---------------------------------------------------------------- query production

def test_lowrank_queries_equal_direct_with_merged_weights():
    # c^Q W^UQ_i with W^DQ applied first equals one projection by the merged
    # per-head matrix [W^DQ W^UQ_i | W^QR_i]
    rng = np.random.default_rng(6)
    T, dm, ql, n_h, dn, dr = 3, 40, 24, 4, 8, 6
    h = rng.standard_normal((T, dm))
    w_dq = rng.standard_normal((dm, ql))
    w_uq = rng.standard_normal((ql, n_h * dn))
    w_qr = rng.standard_normal((dm, n_h * dr))
    pos = np.array([5, 900, 70000])
    w_q = np.concatenate([(w_dq @ w_uq).reshape(dm, n_h, dn), w_qr.reshape(dm, n_h, dr)], axis=2)
    a_n, a_r = O.project_queries_lowrank(h, w_dq, w_uq, w_qr, n_h, dn, dr, pos)
    b_n, b_r = O.project_queries_direct(h, w_q.reshape(dm, -1), n_h, dn, dr, pos)
    np.testing.assert_allclose(a_n, b_n, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(a_r, b_r, rtol=1e-12, atol=1e-12)


def test_absorbed_queries_give_the_unabsorbed_scores():
    # q~ . c + q^R . k^R == [q^C ; q^R] . [c W^UK_i ; k^R] for every head
    rng = np.random.default_rng(7)
    T, dm, ql, n_h, dn, dr, dc = 2, 32, 16, 3, 8, 4, 12
    h = rng.standard_normal((T, dm))
    w_dq, w_uq = rng.standard_normal((dm, ql)), rng.standard_normal((ql, n_h * dn))
    w_qr, w_uk = rng.standard_normal((dm, n_h * dr)), rng.standard_normal((n_h, dc, dn))
    pos = np.array([3, 11])
    q_lat, q_rope = O.project_queries_absorbed(h, w_dq, w_uq, w_qr, w_uk, n_h, dn, dr, pos)
    q_nope, q_rope2 = O.project_queries_lowrank(h, w_dq, w_uq, w_qr, n_h, dn, dr, pos)
    c, kr = rng.standard_normal((5, dc)), rng.standard_normal((5, dr))
    for t in range(T):
        for i in range(n_h):
            full = np.concatenate([q_nope[t, i], q_rope2[t, i]]) @ np.concatenate([c @ w_uk[i], kr], axis=1).T
            np.testing.assert_allclose(q_lat[t, i] @ c.T + q_rope[t, i] @ kr.T, full, rtol=1e-10)


@pytest.mark.parametrize("fmt", [O.FMT_FP8_E5M2, O.FMT_FP8_E4M3_ROW])
def test_append_other_fp8_whole_block(fmt):
    # e5m2 latent: scale = amax|c| / 57344; whole-row e4m3: one scale from the
    # amax over c and k^R, every row value coded; within half a code step
    d = _append_all(fmt, [64, 128], [64, 64], seed=8)
    full = fmt == O.FMT_FP8_E4M3_ROW
    W = 48 if full else 32
    top = O.FP8_MAX[fmt]
    half_step = 2.0 ** -4 if fmt != O.FMT_FP8_E5M2 else 2.0 ** -3
    sub = 2.0 ** -10 if fmt != O.FMT_FP8_E5M2 else 2.0 ** -17
    for b, L in enumerate([64, 128]):
        c, kr = O.project_kv(d["H"][b, :L], d["w"], 32, np.arange(L))
        vals = np.concatenate([c, kr], axis=1) if full else c
        for lb in range(L // BLK):
            blk = d["bt"][b, lb]
            vb = vals[lb * BLK:(lb + 1) * BLK]
            sc = np.float32(np.abs(vb).max() / top)
            assert d["scales"][blk] == sc
            codes = d["pool"][blk, :BLK * W].reshape(BLK, W)
            val = O.fp8_decode(fmt, codes) * float(sc)
            bound = np.maximum(np.abs(vb) * half_step, sub * float(sc)) * 1.0000001
            assert np.all(np.abs(val - vb) <= bound)
            if not full:
                krb = d["pool"][blk, BLK * 32:].copy().view(np.uint16).reshape(BLK, 16)
                assert np.array_equal(krb, O.f64_to_bf16(kr[lb * BLK:(lb + 1) * BLK]))
    m = _touched(d, fmt)
    assert np.array_equal(d["pool"][~m], d["pool0"][~m])
