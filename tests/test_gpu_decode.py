"""GPU parity of mla_decode / mla_combine_lse / mla_gather_paged against the
CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
from mla_latent_kv_07_amd import _lib as L
from mla_latent_kv_07_amd import api
from mla_latent_kv_07_amd import inputs as I

from parity import DEV, FMT, TOL, compare_decode, oracle_decode, run_decode, say, to_device

pytestmark = pytest.mark.gpu


def small(kv="bf16", seq=(1, 100, 333), q_len=1, n_h=128, d_c=512, d_r=64, seed=7, heavy=0.0, heavy_mult=8.0):
    return I.make_decode_inputs(I.Workload(
        f"small_{kv}_q{q_len}_h{n_h}", seed, kv, "f32" if kv == "f32" else "bf16", B=len(seq),
        q_len=q_len, n_h=n_h, d_c=d_c, d_r=d_r, seq_lens=tuple(seq), heavy_frac=heavy, heavy_mult=heavy_mult))


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8_e4m3", "f16", "fp8_e5m2", "fp8_e4m3_row"])
def test_gather_bit_exact(kv):
    d = small(kv, seq=(3, 64, 129, 0), d_c=512 if kv != "f32" else 64, d_r=64 if kv != "f32" else 16, n_h=8)
    cache, bt, sl, _, _ = to_device(d)
    got = api.gather_paged(cache, bt, sl, 130).cpu().numpy()
    ref = O.gather(d.cache.pool, FMT[kv], d.wl.d_c, d.wl.d_r, d.cache.block_table, d.cache.seq_lens, 130)
    assert np.array_equal(got, ref)


def test_decode_bf16_mfma_ragged():
    # several tiles and ragged tails; one split per sequence (one "CU")
    d = small("bf16", seq=(1, 100, 333, 64, 65))
    o, lse, dec = run_decode(d, cus=1)
    assert dec.info.num_partials == 0
    compare_decode(d, o, lse)


def test_decode_bf16_mfma_splits_and_combine():
    # a tiny CU count forces several splits per sequence and the LSE combine
    d = small("bf16", seq=(1, 700, 1500, 64, 0, 129), seed=8)
    o, lse, dec = run_decode(d, cus=8)
    assert dec.info.num_partials > 0 and dec.info.max_splits > 1
    compare_decode(d, o, lse)


@pytest.mark.parametrize("seq,cus,min_splits", [((6000, 70, 0), 96, 16),
                                               ((16384, 70, 0), 256, 96)])
def test_decode_bf16_many_splits_wide_combine(seq, cus, min_splits):
    # a long sequence split over many CUs: more than 16 partial slots per
    # segment take the workgroup-per-row merge (more than 96: several rounds
    # of partial rows per wave); a short and an empty sequence ride along
    d = small("bf16", seq=seq, seed=12)
    o, lse, dec = run_decode(d, cus=cus)
    assert dec.info.max_splits > min_splits, dec.info.max_splits
    compare_decode(d, o, lse)


def test_decode_bf16_heavy_rows_and_nan_tails():
    # 5 % of rows scaled x8 (large softmax range, exercises the running-max
    # raise); NaN tails and spare blocks must not leak
    d = small("bf16", seq=(2000, 37, 640), seed=9, heavy=0.05)
    o, lse, _ = run_decode(d, cus=16)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8_e4m3", "fp8_e5m2", "fp8_e4m3_row"])
def test_decode_reference_raise_every_format(kv):
    # rows scaled x8 in later stages lift a row's stage max far above the
    # reference taken from its first stage: the kernel recomputes those
    # stages' scores and rescales the value sum (the rare path of the lazy
    # max); few CUs give long items with many stages each
    d = small(kv, seq=(900, 1300, 40), seed=21, heavy=0.03)
    o, lse, _ = run_decode(d, cus=4)
    compare_decode(d, o, lse)


def test_decode_bf16_reference_raise_large_jumps():
    # rows scaled x32 push scores 100+ log2 units above a row's first-stage
    # max: every row raises its reference several times, by large steps
    d = small("bf16", seq=(900, 1300, 40), seed=22, heavy=0.03, heavy_mult=32.0)
    o, lse, _ = run_decode(d, cus=4)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("exp2", [40, -60])
def test_decode_bf16_value_range_with_outlier_keys(exp2):
    # The bf16 decode lets p reach 2^40 before it raises a row's reference max,
    # and a raise leaves 2^24 of headroom.  Latent values scaled by 2^40 (fp32
    # sums near 2^100) or by 2^-60 (products p v near 2^-84), with x8 outlier
    # keys raising the reference, must still match the oracle.  The latent
    # queries take the inverse power, so every score is unchanged.
    d = small("bf16", seq=(900, 1300, 40), seed=23, heavy=0.03)
    rows = d.cache.pool.view(torch.bfloat16).view(d.cache.pool.shape[0], 64, d.wl.d_c + d.wl.d_r)
    rows[:, :, :d.wl.d_c] = (rows[:, :, :d.wl.d_c].float() * 2.0 ** exp2).to(torch.bfloat16)
    d.q_lat.copy_((d.q_lat.float() * 2.0 ** -exp2).to(d.q_lat.dtype))
    o, lse, _ = run_decode(d, cus=4)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_decode_many_ragged_sequences_dispatch_table(kv):
    # 300 sequences of 1-700 tokens with q_len 2 (two row chunks each): the
    # plan holds far more items than compute units, mixes split and whole
    # (sequence, row chunk) segments, and the dispatch table gives every XCD
    # a long queue; empty sequences and one-token ones included
    import numpy as np
    rng = np.random.default_rng(31)
    seq = rng.integers(1, 701, size=300)
    seq[[5, 77, 200]] = 0
    seq[[6, 78]] = 1
    d = small(kv, seq=tuple(int(x) for x in seq), q_len=2, seed=32)
    o, lse, dec = run_decode(d)
    assert dec.info.num_items > 256 and dec.info.grid_wgs > 256 and dec.info.row_chunks == 2
    say(f"  items {dec.info.num_items}, grid {dec.info.grid_wgs}, partial slots {dec.info.num_partials}")
    rows = np.sort(np.random.default_rng(33).choice(300 * 256, size=3000, replace=False))
    compare_decode(d, o, lse, rows=rows)


def test_decode_bf16_spec_pair_causal():
    # q_len = 2: 256 rows per sequence -> two row chunks per work item
    d = small("bf16", seq=(2, 3, 64, 65, 500), q_len=2, seed=10)
    o, lse, dec = run_decode(d, cus=16)
    assert dec.info.row_chunks == 2
    compare_decode(d, o, lse)


def test_decode_bf16_few_heads():
    # n_h = 16 (e.g. one tensor-parallel shard): rows < one chunk, partly idle waves
    d = small("bf16", seq=(77, 300), n_h=16, seed=11)
    o, lse, _ = run_decode(d)
    compare_decode(d, o, lse)


def test_decode_query_longer_than_sequence():
    d = small("bf16", seq=(1, 0, 2), q_len=2, seed=12)
    o, lse, _ = run_decode(d)
    compare_decode(d, o, lse)
    lse_c = lse.cpu()
    assert torch.isinf(lse_c[0]).all() and torch.isinf(lse_c[2:4]).all()


def test_decode_generic_paths():
    # f32 cache (tiny dims) and bf16 with f32 queries go through the generic kernel
    d = small("f32", seq=(1, 70, 200), n_h=8, d_c=64, d_r=16, seed=13)
    o, lse, _ = run_decode(d, cus=4)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("exact", [False, True], ids=["fp8_mfma", "exact_bf16"])
def test_decode_fp8_cache(exact):
    d = small("fp8_e4m3", seq=(2, 150, 300), q_len=2, seed=14)
    o, lse, _ = run_decode(d, cus=8, fp8_exact=exact)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("exact", [False, True], ids=["fp8_mfma", "exact_bf16"])
def test_decode_fp8_long_items(exact):
    # a 30,000-token sequence over two compute units: items of ~230 blocks,
    # hundreds of stages per workgroup (block ids, stage buffers and the lazy
    # reference max over a long loop), next to one-block and empty sequences
    d = small("fp8_e4m3", seq=(30000, 5, 0, 64), q_len=1, seed=45, heavy=0.01)
    o, lse, dec = run_decode(d, cus=2, fp8_exact=exact)
    assert dec.info.blocks_per_item > 200
    compare_decode(d, o, lse)


def test_decode_fp8_mfma_path_tracks_exact_path():
    # the two arithmetics over one e4m3 cache: the 8-bit MFMA path (two-term
    # e4m3 query and probabilities) against the exact decode, row by row, and
    # both against the oracle.  The rows scaled x8 here carry 8x larger
    # logits, so the query's residual rounding (~2^-8) moves their weights
    # most: the paths differ by up to ~2 % (a few 1e-3 on N(0,1) rows)
    d = small("fp8_e4m3", seq=(700, 1, 64, 65, 1300), q_len=2, seed=41, heavy=0.02)
    o8, l8, _ = run_decode(d, cus=6)
    ox, lx, _ = run_decode(d, cus=6, fp8_exact=True)
    a8 = o8.float().cpu().numpy().reshape(-1, 512)
    ax = ox.float().cpu().numpy().reshape(-1, 512)
    nz = np.linalg.norm(ax, axis=1) > 0
    rel = np.linalg.norm(a8 - ax, axis=1)[nz] / np.linalg.norm(ax, axis=1)[nz]
    say(f"  8-bit vs exact path: max row rel diff {rel.max():.3e}")
    assert rel.max() < 3e-2
    assert np.array_equal(np.isinf(l8.cpu().numpy()), np.isinf(lx.cpu().numpy()))
    compare_decode(d, o8, l8)
    compare_decode(d, ox, lx)


@pytest.mark.parametrize("exact", [False, True], ids=["fp8_mfma", "exact_bf16"])
def test_decode_fp8_ragged_row_chunks(exact):
    # q_len 3 x 48 heads = 144 rows per sequence: a full 128-row chunk and one
    # of 16 rows, with the causal limit moving inside each chunk
    d = small("fp8_e4m3", seq=(5, 400, 129), q_len=3, n_h=48, seed=46)
    o, lse, dec = run_decode(d, cus=6, fp8_exact=exact)
    assert dec.info.row_chunks == 2
    compare_decode(d, o, lse)


@pytest.mark.parametrize("exact", [False, True], ids=["fp8_mfma", "exact_bf16"])
def test_decode_fp8_few_heads_and_empty_rows(exact):
    # n_h = 16 with a query pair: 32 rows per sequence, so three of the four
    # waves hold only rows past the end; sequences shorter than the pair and
    # empty ones leave rows with no visible position (o = 0, lse = -inf)
    d = small("fp8_e4m3", seq=(1, 0, 2, 77, 300), q_len=2, n_h=16, seed=45)
    o, lse, _ = run_decode(d, cus=4, fp8_exact=exact)
    compare_decode(d, o, lse)
    lse_c = lse.cpu().reshape(5, 2, 16)
    assert torch.isinf(lse_c[0, 0]).all() and torch.isinf(lse_c[1]).all()
    assert torch.isfinite(lse_c[0, 1]).all() and torch.isfinite(lse_c[3]).all()


@pytest.mark.parametrize("kv,exact", [("fp8_e4m3", False), ("fp8_e4m3", True), ("fp8_e5m2", False),
                                      ("fp8_e4m3_row", False)],
                         ids=["e4m3_fp8_mfma", "e4m3_exact_bf16", "e5m2", "e4m3_row"])
def test_decode_fp8_block_scale_edges(kv, exact):
    # block scales at the edges of both fp8 arithmetics: zero (the block's
    # latent term vanishes; the whole row for e4m3_row), a tiny scale
    # (2^-126: the 8-bit path clamps the E8M0 exponent and shrinks the
    # mantissa, the exact path raises the magnitude to 2^-64), an odd
    # mantissa (x 1.37) and a negative scale (the codes change sign); the
    # oracle decodes code * scale exactly.  (A scale far above the data's
    # absmax / 448 inflates that block's logits, and with them the score
    # error of the two-term query: the exact path serves such caches.)
    d = small(kv, seq=(640, 300), seed=43)
    sc = d.cache.block_scales
    blocks = d.cache.block_table[0, :10].tolist()
    sc[blocks[1]] = 0.0
    sc[blocks[2]] = 2.0 ** -126
    sc[blocks[3]] = sc[blocks[3]] * 1.37
    sc[blocks[5]] = -sc[blocks[5]]
    o, lse, _ = run_decode(d, cus=4, fp8_exact=exact)
    compare_decode(d, o, lse)


def test_block_table_permutation_gives_identical_bits():
    d = small("bf16", seq=(190, 64, 7), seed=15)
    o1, l1, _ = run_decode(d, cus=8)
    # same logical rows through another pool permutation
    g = torch.Generator()
    g.manual_seed(99)
    rows = []
    for b, S in enumerate(d.cache.seq_lens.tolist()):
        for p in range(S):
            blk = int(d.cache.block_table[b, p // 64])
            rows.append(d.cache.pool[blk].view(torch.bfloat16).view(64, -1)[p % 64].float())
    rows = torch.stack(rows)
    cache2 = I.page_cache(d.wl, g, d.cache.seq_lens, rows)
    assert not torch.equal(cache2.block_table, d.cache.block_table)
    d2 = I.DecodeInputs(d.wl, cache2, d.q_lat, d.q_rope, d.scale)
    o2, l2, _ = run_decode(d2, cus=8)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_is_deterministic():
    d = small("bf16", seq=(900, 31), seed=16)
    cache, bt, sl, ql, qr = to_device(d)
    dec = api.Decoder(d.cache.seq_lens, 1, 128, 512, 64, "bf16", DEV, cus=8)
    o1, l1 = dec(ql, qr, cache, bt, sl, d.scale)
    o2, l2 = dec(ql, qr, cache, bt, sl, d.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_combine_lse_standalone():
    rng = np.random.default_rng(3)
    P, rows, d_c = 7, 16, 512
    o_part = rng.normal(size=(P, rows, d_c))
    lse_part = rng.normal(size=(P, rows)) * 3
    lse_part[2, :5] = -np.inf
    lse_part[3:5, 7] = -np.inf
    split_off = np.array([0, 3, 3, 7], np.int32)      # sequence 1 has no slots
    seq_flags = np.array([0, 0, 0], np.int32)
    o32 = torch.from_numpy(o_part).float()
    l32 = torch.from_numpy(lse_part).float()
    o, l = api.combine_lse(o32.to(DEV), l32.to(DEV), torch.from_numpy(split_off).to(DEV), 3, rows,
                           out_dtype=torch.float32, seq_flags=torch.from_numpy(seq_flags).to(DEV))
    o, l = o.cpu().numpy().reshape(3, rows, d_c), l.cpu().numpy().reshape(3, rows)
    for b in range(3):
        k0, k1 = split_off[b], split_off[b + 1]
        if k1 == k0:
            assert not o[b].any() and np.all(np.isneginf(l[b]))
            continue
        ro, rl = O.combine(o32.double().numpy()[k0:k1], l32.double().numpy()[k0:k1])
        assert np.abs(o[b] - ro).max() < 1e-5 and np.abs(l[b] - rl).max() < 1e-5


@pytest.mark.timeout(600)
def test_decode_measured_batch_full_size():
    """The measured batch (32 x 4096, bf16, 128 heads), in the launch
    configuration the benchmark times, against the oracle on all 4,096 rows."""
    d = I.make_decode_inputs(I.C2)
    o, lse, dec = run_decode(d)
    assert dec.info.num_items == 256
    compare_decode(d, o, lse)


@pytest.mark.parametrize("kv", ["f16", "fp8_e5m2", "fp8_e4m3_row"])
def test_decode_cache_format_variants_mfma(kv):
    """fp16 rows (fp16 MFMAs), e5m2 latent codes, and the whole row in e4m3
    (one block scale for c and k^R) on the MFMA kernel: ragged lengths, NaN
    tails, several splits and the combine, then the causal query pair."""
    d = small(kv, seq=(1, 700, 1500, 64, 0, 129), seed=31, heavy=0.02)
    o, lse, dec = run_decode(d, cus=8)
    assert dec.info.max_splits > 1
    compare_decode(d, o, lse)
    d = small(kv, seq=(2, 3, 64, 65, 500), q_len=2, seed=32)
    o, lse, _ = run_decode(d, cus=16)
    compare_decode(d, o, lse)


@pytest.mark.parametrize("kv", ["f16", "fp8_e5m2", "fp8_e4m3_row"])
def test_decode_cache_format_variants_generic(kv):
    """The same formats at a shape the MFMA kernel does not take (generic kernel)."""
    d = small(kv, seq=(1, 70, 200), n_h=8, d_c=64, d_r=16, seed=33)
    o, lse, _ = run_decode(d, cus=4)
    compare_decode(d, o, lse)


def test_debug_device_checks_reject_bad_tables():
    """With device checks on (mla_set_debug), a used block-table entry outside
    the pool, or a sequence length beyond the table, is reported as
    MLA_ERR_DEVICE_CHECK before any decode launch (the outputs keep their
    sentinel); valid inputs, unused entries holding anything, decode as
    without the checks.  The check kernel only reads the table and the
    lengths: no decode runs on the bad ones."""
    lib = L.load()
    d = small("bf16", seq=(1, 100, 333), seed=11)
    cache, bt, sl, ql, qr = to_device(d)
    dec = api.Decoder(d.cache.seq_lens, 1, d.wl.n_h, d.wl.d_c, d.wl.d_r, "bf16", DEV)
    assert bt.shape[1] >= 6
    assert lib.mla_set_debug(1) == L.MLA_OK
    try:
        # unused entries (sequence 0 has one block) may hold anything
        ok_bt = bt.clone()
        ok_bt[0, 1:] = -7
        o, lse = dec(ql, qr, cache, ok_bt, sl, d.scale)
        torch.cuda.synchronize()
        compare_decode(d, o, lse)

        def rejected(table, lens, what):
            o2 = torch.full_like(o, 7.0)
            lse2 = torch.full_like(lse, 7.0)
            with pytest.raises(L.MLAError) as ex:
                dec(ql, qr, cache, table, lens, d.scale, o_lat=o2, lse=lse2)
            torch.cuda.synchronize()
            assert ex.value.status == L.MLA_ERR_DEVICE_CHECK and what in str(ex.value), str(ex.value)
            assert bool((o2 == 7.0).all()) and bool((lse2 == 7.0).all())

        bad = bt.clone()
        bad[2, 3] = cache.num_blocks + 5          # sequence 2 (333 tokens) uses entry 3
        rejected(bad, sl, f"sequence 2, table entry 3 holds block id {cache.num_blocks + 5}")
        bad = bt.clone()
        bad[1, 0] = -1                            # an unallocated entry inside sequence 1
        rejected(bad, sl, "sequence 1, table entry 0 holds block id -1")
        long = sl.clone()
        long[1] = 64 * bt.shape[1] + 1
        rejected(bt, long, f"sequence 1 has length {64 * bt.shape[1] + 1}")
        bad = bt.clone()
        bad[2, 3] = cache.num_blocks
        with pytest.raises(L.MLAError) as ex:
            api.gather_paged(cache, bad, sl, 333)
        assert ex.value.status == L.MLA_ERR_DEVICE_CHECK
        # the flag was cleared: a valid call passes again
        o, lse = dec(ql, qr, cache, bt, sl, d.scale)
        torch.cuda.synchronize()
        compare_decode(d, o, lse)
    finally:
        lib.mla_set_debug(0)
