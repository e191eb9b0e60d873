"""CPU model of the 8-bit MFMA decode's LDS layout and read addressing.

decode_f8mma.hip copies a paged block (64 tokens: [64][512] e4m3 latent codes,
then [64][64] bf16 rotary keys) into LDS with direct-to-LDS loads, 16-byte
chunk c of token t's latent at chunk c ^ swz(t), and reads it back as MFMA
fragments with per-lane bases XOR compile-time constants.  This test writes
the same formulas out in Python and checks, byte by byte, that:
  - the copies fill every byte of the stage once, as the layout states, and
    each 16-lane quarter of a copy reads at most 2 cache lines;
  - every score read (latent and rotary) returns the token and features the
    MFMA A-operand layout needs (lane l: token l % 32 of the tile; byte b of
    lane half g: feature 64 kc + 32 g + b), with 16 distinct 16-byte bank
    groups per 16-lane pass;
  - every transposed value read (ds_read_b64_tr_b8: lane 8 a + e of a 16-lane
    group receives, as its byte s, byte e of the 8 read by lane 2 s + a, as
    probed on gfx950) gives lane (g, d) the feature d of the token that the
    score accumulator layout holds at byte position b (tile b / 16,
    accumulator b % 16, token 32 T + 8 (q >> 2) + 4 g + (q & 3)), with no
    two 16-byte segments of a 32-lane pass in one bank group.
No GPU is needed; the formulas are those of the kernel's comments.
"""
import numpy as np

DC, BT = 512, 64
LAT = BT * DC
STAGE = LAT + BT * 128


def swz(t):
    return ((t & 3) << 2) | ((t >> 2) & 3)


def rot_swz(t):
    return ((t & 7) >> 1) ^ (((t >> 3) & 1) << 2)


def block_tags():
    """Tag of every byte of a block: token * 1000 + feature byte (latent),
    100000 + token * 1000 + byte (rotary)."""
    lat = np.repeat(np.arange(64), 512) * 1000 + np.tile(np.arange(512), 64)
    rot = 100000 + np.repeat(np.arange(64), 128) * 1000 + np.tile(np.arange(128), 64)
    return np.concatenate([lat, rot])


def copy_stage():
    tags = block_tags()
    lds = -np.ones(STAGE, dtype=np.int64)
    worst_lines = 0
    for wave in range(4):
        for k in range(8):                       # latent KiB 8 w + k
            kib = 8 * wave + k
            for q in range(4):
                lines = set()
                for lane in range(16 * q, 16 * q + 16):
                    h = lane >> 5
                    lat0 = 512 * h + 16 * ((lane & 31) ^ (4 * h))
                    voff = lat0 ^ (16 * (8 * (k & 1) + ((k >> 1) & 3)))
                    src, dst = 1024 * kib + voff, 1024 * kib + 16 * lane
                    assert (lds[dst:dst + 16] == -1).all()
                    lds[dst:dst + 16] = tags[src:src + 16]
                    lines.add(src // 128)
                worst_lines = max(worst_lines, len(lines))
        for k in range(2):                       # rotary KiB 2 w + k
            r = 2 * wave + k
            for lane in range(64):
                u = (lane >> 3) & 7
                voff = 128 * u + 16 * ((lane & 7) ^ (u >> 1) ^ (4 * k))
                src, dst = LAT + 1024 * r + voff, LAT + 1024 * r + 16 * lane
                assert (lds[dst:dst + 16] == -1).all()
                lds[dst:dst + 16] = tags[src:src + 16]
    return lds, worst_lines


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


def test_score_reads_return_the_fragment_layout_without_bank_conflicts():
    lds, _ = copy_stage()
    for T in range(2):
        for kc in range(8):
            for hh in range(2):
                groups = {}
                for lane in range(64):
                    g, ln = lane >> 5, lane & 31
                    kb = ln * 512 + ((32 * g) ^ (16 * swz(ln & 15)))
                    o = ((kb ^ (64 * kc)) + 16384 * T) ^ (16 * hh)
                    want = (32 * T + ln) * 1000 + 64 * kc + 32 * g + 16 * hh + np.arange(16)
                    assert (lds[o:o + 16] == want).all()
                    groups.setdefault(lane // 16, set()).add((o % 256) // 16)
                assert all(len(v) == 16 for v in groups.values())
        for j in range(4):
            groups = {}
            for lane in range(64):
                g, ln = lane >> 5, lane & 31
                rb = LAT + (ln >> 3) * 1024 + (ln & 7) * 128 + 16 * (g ^ rot_swz(ln))
                o = (rb ^ (32 * j)) + 4096 * T
                want = 100000 + (32 * T + ln) * 1000 + 16 * (2 * j + g) + np.arange(16)
                assert (lds[o:o + 16] == want).all()
                groups.setdefault(lane // 16, set()).add((o % 256) // 16)
            assert all(len(v) == 16 for v in groups.values())


def test_transposed_value_reads_match_the_score_accumulator_layout():
    lds, _ = copy_stage()

    def token_at(g, b):
        T, q = b // 16, b % 16
        return 32 * T + 8 * (q >> 2) + 4 * g + (q & 3)

    for mb in range(16):
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
            for half in range(2):
                segs = {}
                for lane in range(32 * half, 32 * half + 32):
                    segs.setdefault((addr[lane] % 256) // 16, set()).add(addr[lane] // 16)
                assert all(len(v) == 1 for v in segs.values())
        for lane in range(64):
            g, d = lane >> 5, 32 * mb + (lane & 31)
            for b in range(32):
                assert frag[lane, b] == token_at(g, b) * 1000 + d
