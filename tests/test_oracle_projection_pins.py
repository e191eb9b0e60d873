"""Pins of the oracle's projections (CPU): the cached row c = h W^DKV with the
shared rotary key k^R = RoPE(h W^KR) ([huny] §2-1 compression equation, §2-3
rotary key), and the per-head query [q^C_i ; q^R_i] ([huny] §2-2 low-rank
query, §2-3 rotary query and concatenation).

Every expected value here is written out from the definitions, not taken
from the oracle: a one-hot hidden state selects one row of a weight matrix
exactly (so the first d_c columns must come back as c and the rest as the
unrotated k^R at position 0), and at position p pair (2j, 2j+1) must be that
row's pair turned by the angle p * theta_j, theta_j = 10000^(-2j/d_R),
through an explicit 2x2 rotation.  Weights with distinct entries make a
wrong column split, a swapped pair or a position taken from another token
change the numbers."""
import math

import numpy as np

import oracle as O


def _distinct(rows, cols):
    # w[r][c] = r + c / 1024: every entry distinct, and sums of a few of them exact in fp64
    return np.arange(rows)[:, None] + np.arange(cols)[None, :] / 1024.0


def _turn(x0, x1, ang):
    """The pair (x0, x1) turned by ang: [[cos, -sin], [sin, cos]] (x0, x1)."""
    c, s = math.cos(ang), math.sin(ang)
    return c * x0 - s * x1, s * x0 + c * x1


def _rotated(row, p, d_r):
    out = np.empty(d_r)
    for j in range(d_r // 2):
        theta = math.pow(10000.0, -2.0 * j / d_r)
        out[2 * j], out[2 * j + 1] = _turn(row[2 * j], row[2 * j + 1], p * theta)
    return out


def test_rope_hand_values():
    # d_R = 4: theta_0 = 1, theta_1 = 10000^(-1/2) = 0.01
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    got = O.rope(x, np.array([1.0]))[0]
    want = [math.cos(1.0), math.sin(1.0), -math.sin(0.01), math.cos(0.01)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # position 0 is the identity, exactly
    y = np.array([[0.3, -1.5, 2.25, 7.0]])
    assert np.array_equal(O.rope(y, np.array([0.0])), y)


def test_project_kv_one_hot_rows_select_weight_rows():
    d_model, d_c, d_r = 6, 8, 4
    w = _distinct(d_model, d_c + d_r)
    h = np.eye(d_model)
    positions = np.array([0, 1, 5, 1000, 70000, 3], dtype=np.float64)
    c, kr = O.project_kv(h, w, d_c, positions)
    assert c.shape == (d_model, d_c) and kr.shape == (d_model, d_r)
    for k in range(d_model):
        # c: the first d_c columns of row k, exactly
        assert np.array_equal(c[k], w[k, :d_c])
        # k^R: the remaining columns, turned at the token's own position
        assert np.allclose(kr[k], _rotated(w[k, d_c:], positions[k], d_r), rtol=0, atol=1e-9)
    # the position-0 token keeps the unrotated columns exactly
    assert np.array_equal(kr[0], w[0, d_c:])


def test_project_kv_is_linear_in_h():
    d_model, d_c, d_r = 5, 8, 4
    w = _distinct(d_model, d_c + d_r)
    h = np.array([[2.0, 0.0, -3.0, 0.0, 0.5]])
    c, kr = O.project_kv(h, w, d_c, np.array([7.0]))
    z = 2.0 * w[0] - 3.0 * w[2] + 0.5 * w[4]
    assert np.array_equal(c[0], z[:d_c])
    assert np.allclose(kr[0], _rotated(z[d_c:], 7.0, d_r), rtol=0, atol=1e-9)


def test_project_queries_direct_one_hot_rows():
    n_h, d_nope, d_r = 3, 4, 4
    d_model = 5
    w_q = _distinct(d_model, n_h * (d_nope + d_r))
    h = np.eye(d_model)
    positions = np.array([0, 2, 9, 40000, 1], dtype=np.int64)
    q_nope, q_rope = O.project_queries_direct(h, w_q, n_h, d_nope, d_r, positions)
    assert q_nope.shape == (d_model, n_h, d_nope) and q_rope.shape == (d_model, n_h, d_r)
    for k in range(d_model):
        for i in range(n_h):
            blk = w_q[k, i * (d_nope + d_r):(i + 1) * (d_nope + d_r)]
            # head i's block is [q^C_i | q^R_i]
            assert np.array_equal(q_nope[k, i], blk[:d_nope])
            assert np.allclose(q_rope[k, i], _rotated(blk[d_nope:], positions[k], d_r), rtol=0, atol=1e-9)
    assert np.array_equal(q_rope[0], w_q[0].reshape(n_h, d_nope + d_r)[:, d_nope:])


def test_project_queries_lowrank_one_hot_rows():
    # W^DQ = I (q_lora = d_model), so c^Q = h exactly and q^C_i is row k of
    # W^UQ's head-i columns; q^R_i is row k of W^QR's head-i columns, turned
    n_h, d_nope, d_r, d_model = 2, 4, 4, 3
    w_dq = np.eye(d_model)
    w_uq = _distinct(d_model, n_h * d_nope)
    w_qr = _distinct(d_model, n_h * d_r) + 50.0
    h = np.eye(d_model)
    positions = np.array([3, 0, 123], dtype=np.int64)
    q_nope, q_rope = O.project_queries_lowrank(h, w_dq, w_uq, w_qr, n_h, d_nope, d_r, positions)
    for k in range(d_model):
        for i in range(n_h):
            assert np.array_equal(q_nope[k, i], w_uq[k, i * d_nope:(i + 1) * d_nope])
            want = _rotated(w_qr[k, i * d_r:(i + 1) * d_r], positions[k], d_r)
            assert np.allclose(q_rope[k, i], want, rtol=0, atol=1e-9)


def test_append_skips_unallocated_and_out_of_table_tokens():
    # tokens mapped to a -1 table entry or past the table are not written;
    # the other sequences' rows are written as without them
    d_model, d_c, d_r = 4, 8, 4
    rng = np.random.default_rng(0)
    w = rng.standard_normal((d_model, d_c + d_r))
    h = rng.standard_normal((3 * 2, d_model))
    nb = 6
    pool0 = rng.integers(0, 256, (nb, O.block_bytes(O.FMT_BF16, d_c, d_r)), dtype=np.uint8)
    bt = np.array([[0, 1], [-1, -1], [2, 3]], np.int32)
    pos = np.array([5, 5, 127], np.int32)           # sequence 2's second token is at p = 128
    got = pool0.copy()
    O.cache_append(got, None, O.FMT_BF16, d_c, d_r, bt, pos, 2, h, w)
    # only sequence 0 (block 0, slots 5-6) and sequence 2's first token
    # (block 3, slot 63) may change
    alone = pool0.copy()
    O.cache_append(alone, None, O.FMT_BF16, d_c, d_r, bt[[0]], pos[[0]], 2, h[:2], w)
    rb = (d_c + d_r) * 2
    assert np.array_equal(got[[1, 2, 4, 5]], pool0[[1, 2, 4, 5]])
    assert np.array_equal(got[0], alone[0])
    assert np.array_equal(got[3, :63 * rb], pool0[3, :63 * rb])
    c, kr = O.project_kv(h[4:5], w, d_c, np.array([127]))
    assert np.array_equal(got[3, 63 * rb:], O.f64_to_bf16(np.concatenate([c, kr], 1)).view(np.uint8).reshape(-1))
