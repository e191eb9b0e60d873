"""CPU model of the eight-wave 8-bit decode's LDS traffic (decode_f8w8.hip).

A stage (one 64-token block) sits in LDS with 16-byte chunk c of token t's
latent at chunk c ^ swz(t) and the rotary keys token-major with slot
c ^ rot_swz(t).  Eight waves copy it direct-to-LDS; the score operands are
read as 16x16x128 fragments (lane (G, r): token 16 T + r, 32 bytes of
features 128 G + 32 kc, chunks 8 G + 2 kc + {0, 1}: with G in the chunk
index's low bits the reads measured ~1.4x slower on gfx950, although every
16-lane pass covers the 16 bank groups either way); the P codes pass through
LDS: the score lane (G, r)
writes its tokens 16 T + 4 G + i at k position 32 (G & 1) + 8 T + 4 (G >> 1) + i
of its row, and the value MFMA reads row 32 nb + ln, k positions 32 g .. + 31
as its B fragment against V fragments read transposed (ds_read_b64_tr_b8:
lane 8 a + e of a 16-lane group receives, as its byte s, byte e of the 8 read
by lane 2 s + a, as probed on gfx950).
This test writes those formulas out and checks, byte by byte, that
  - the copies fill every byte of the stage once, as laid out, with at most 2
    cache lines per 16-lane quarter;
  - every score and rotary read returns the token and features of the
    fragment layout, with 16 distinct 16-byte bank groups per 16-lane pass;
  - the P code positions are a bijection onto the 64 k positions and put
    at each position the token that the V fragment holds there;
  - the P reads, the q^R reads and the P writes stay within their regions,
    with the reads in distinct bank groups per 16-lane pass;
  - the LDS regions do not overlap and fit in 160 KiB.
No GPU is needed; the formulas are those of the kernel's comments.
"""
import numpy as np

DC, BT = 512, 64
LAT = BT * DC
STAGE = LAT + BT * 128
NST, ROWS, WAVES = 3, 128, 8
P_PITCH, QR_PITCH, O_PITCH = 144, 144, 1040
P_OFF = NST * STAGE
ALPHA_OFF = P_OFF + ROWS * P_PITCH
FLAG_OFF = ALPHA_OFF + ROWS * 4
LIM_OFF = FLAG_OFF + 64
RING_OFF = LIM_OFF + ROWS * 4
L_OFF = RING_OFF + 4 * 256
QR_OFF = L_OFF + ROWS * 4
LDS_BYTES = QR_OFF + ROWS * QR_PITCH


def swz(t):
    return ((t & 3) << 2) | ((t >> 2) & 3)


def rot_swz(t):
    return ((t & 7) >> 1) ^ (((t >> 3) & 1) << 2)


def block_tags():
    lat = np.repeat(np.arange(64), 512) * 1000 + np.tile(np.arange(512), 64)
    rot = 100000 + np.repeat(np.arange(64), 128) * 1000 + np.tile(np.arange(128), 64)
    return np.concatenate([lat, rot])


def copy_stage():
    tags = block_tags()
    lds = -np.ones(STAGE, dtype=np.int64)
    worst_lines = 0
    for wave in range(WAVES):
        for k in range(4):                       # latent KiB 4 w + k
            kib = 4 * wave + k
            for q in range(4):
                lines = set()
                for lane in range(16 * q, 16 * q + 16):
                    h = lane >> 5
                    t = 2 * kib + h
                    voff = 512 * h + 16 * ((lane & 31) ^ swz(t))
                    src, dst = 1024 * kib + voff, 1024 * kib + 16 * lane
                    assert (lds[dst:dst + 16] == -1).all()
                    lds[dst:dst + 16] = tags[src:src + 16]
                    lines.add(src // 128)
                worst_lines = max(worst_lines, len(lines))
        for q in range(4):                       # rotary KiB w
            lines = set()
            for lane in range(16 * q, 16 * q + 16):
                u = (lane >> 3) & 7
                voff = 128 * u + 16 * ((lane & 7) ^ (u >> 1) ^ (4 * (wave & 1)))
                src, dst = LAT + 1024 * wave + voff, LAT + 1024 * wave + 16 * lane
                assert (lds[dst:dst + 16] == -1).all()
                lds[dst:dst + 16] = tags[src:src + 16]
                lines.add(src // 128)
            worst_lines = max(worst_lines, len(lines))
    return lds, worst_lines


def test_region_layout():
    regions = [(0, NST * STAGE), (P_OFF, ALPHA_OFF), (ALPHA_OFF, FLAG_OFF), (FLAG_OFF, FLAG_OFF + 32),
               (LIM_OFF, RING_OFF), (RING_OFF, L_OFF), (L_OFF, QR_OFF), (QR_OFF, LDS_BYTES)]
    for (a0, a1), (b0, b1) in zip(regions, regions[1:]):
        assert a1 <= b0 and a0 < a1
    assert LDS_BYTES <= 160 * 1024
    assert ROWS * O_PITCH <= ALPHA_OFF     # epilogue staging spares the per-row words


def test_copies_fill_the_stage_as_laid_out():
    lds, worst_lines = copy_stage()
    assert (lds >= 0).all()
    assert worst_lines <= 2
    for t in range(64):
        for c in range(32):
            o = t * 512 + 16 * (c ^ swz(t))
            assert (lds[o:o + 16] == t * 1000 + 16 * c + np.arange(16)).all()
        for c in range(8):
            o = LAT + (t >> 3) * 1024 + (t & 7) * 128 + 16 * (c ^ rot_swz(t))
            assert (lds[o:o + 16] == 100000 + t * 1000 + 16 * c + np.arange(16)).all()


def test_score_reads_return_the_16x16_fragments_without_bank_conflicts():
    lds, _ = copy_stage()
    for st in range(NST):
        so = st * STAGE
        for T in range(4):
            for kc in range(4):
                for hh in range(2):
                    groups = {}
                    for lane in range(64):
                        G, r = lane >> 4, lane & 15
                        kb = r * 512 + 16 * ((8 * G) ^ swz(r))
                        o = ((kb + so) ^ (32 * kc + 16 * hh)) + 8192 * T
                        assert so <= o and o + 16 <= so + LAT
                        want = (16 * T + r) * 1000 + 128 * G + 32 * kc + 16 * hh + np.arange(16)
                        assert (lds[o - so:o - so + 16] == want).all()
                        groups.setdefault(G, set()).add((o % 256) // 16)
                    assert all(len(v) == 16 for v in groups.values())
            for j in range(2):
                groups = {}
                for lane in range(64):
                    G, r = lane >> 4, lane & 15
                    rb = LAT + (r >> 3) * 1024 + (r & 7) * 128 + 16 * (G ^ rot_swz(r))
                    o = ((rb + so) ^ (64 * j)) + 2048 * T
                    assert so + LAT <= o and o + 16 <= so + STAGE
                    want = 100000 + (16 * T + r) * 1000 + 16 * (4 * j + G) + np.arange(16)
                    assert (lds[o - so:o - so + 16] == want).all()
                    groups.setdefault(G, set()).add((o % 256) // 16)
                assert all(len(v) == 16 for v in groups.values())


def v_token_at(g, b):
    """Token that byte b of lane half g of a transposed V fragment holds."""
    j, s = b // 8, b % 8
    return 16 * j + 8 * (s >> 2) + 4 * g + (s & 3)


def test_value_reads_hold_v_token_at():
    lds, _ = copy_stage()
    for mb in range(16):                      # wave w takes M-blocks 2 w, 2 w + 1
        frag = np.zeros((64, 32), dtype=np.int64)
        for j in range(4):
            addr = np.zeros(64, dtype=np.int64)
            for lane in range(64):
                g, G, i16 = lane >> 5, lane >> 4, lane & 15
                s, a = i16 >> 1, i16 & 1
                tv = 8 * (s >> 2) + 4 * g + (s & 3)
                vb = tv * 512 + 8 * a + 16 * ((G & 1) ^ swz(tv))
                addr[lane] = (vb ^ (32 * mb)) + 8192 * j
            for lane in range(64):
                G, i = lane >> 4, lane & 15
                for s in range(8):
                    frag[lane, 8 * j + s] = lds[addr[16 * G + 2 * s + (i >> 3)] + (i & 7)]
        for lane in range(64):
            g, d = lane >> 5, 32 * mb + (lane & 31)
            for b in range(32):
                assert frag[lane, b] == v_token_at(g, b) * 1000 + d


def test_p_code_positions_match_the_value_fragments():
    # k position of each (lane group G, tile T, entry i) of a score lane
    pos = {}
    for G in range(4):
        for T in range(4):
            for i in range(4):
                k = 32 * (G & 1) + 8 * T + 4 * (G >> 1) + i
                assert k not in pos
                pos[k] = 16 * T + 4 * G + i          # the token the score entry holds
    assert sorted(pos) == list(range(64))
    for g in range(2):
        for b in range(32):
            assert pos[32 * g + b] == v_token_at(g, b)


def test_p_and_qr_traffic_in_region_and_bank_groups():
    # writes: wave w, lane (G, r) -> row 16 w + r, 4-byte words at 8 T (+64 for l)
    written = set()
    for w in range(WAVES):
        for lane in range(64):
            G, r = lane >> 4, lane & 15
            pw = P_OFF + (16 * w + r) * P_PITCH + 32 * (G & 1) + 4 * (G >> 1)
            for T in range(4):
                for t in range(2):
                    o = pw + 64 * t + 8 * T
                    assert P_OFF <= o and o + 4 <= ALPHA_OFF
                    assert o not in written
                    written.add(o)
    assert len(written) == ROWS * 32
    # reads: row block nb, term t: lane (g, ln) reads row 32 nb + ln, 32 bytes at 64 t + 32 g
    for nb in range(4):
        for t in range(2):
            for half in range(2):
                groups = {}
                for lane in range(64):
                    g, ln = lane >> 5, lane & 31
                    o = P_OFF + ln * P_PITCH + 32 * g + nb * 32 * P_PITCH + 64 * t + 16 * half
                    assert P_OFF <= o and o + 16 <= ALPHA_OFF
                    # the 32 bytes cover exactly the words the row's writers put there
                    for wd in range(4):
                        assert o + 4 * wd in written
                    groups.setdefault(lane // 16, set()).add((o % 256) // 16)
                assert all(len(v) == 16 for v in groups.values())
    # q^R: each lane reads back its own 16 bytes; 16-lane passes in distinct bank groups
    for w in range(WAVES):
        for j in range(2):
            groups = {}
            for lane in range(64):
                G, r = lane >> 4, lane & 15
                o = QR_OFF + (16 * w + r) * QR_PITCH + 64 * j + 16 * G
                assert QR_OFF <= o and o + 16 <= LDS_BYTES
                groups.setdefault(G, set()).add((o % 256) // 16)
            assert all(len(v) == 16 for v in groups.values())
