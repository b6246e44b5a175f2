"""CPU checks of the LDS maps the kernels use (no GPU).

The maps are restated here from the kernels' definitions and checked against
two facts: (1) every lane's fragment holds the right row and K bytes after the
stage copies place the tile in LDS, and (2) every 16-lane group of every
fragment read is free of bank conflicts under gfx950's rule for
ds_read_b128, measured with the LDS bank-conflict counter: lane l is served
in group 2 * bit5(l) + (bit2 ^ bit3 ^ bit4)(l), and a group is conflict-free
when its lanes hit distinct 16-byte slots modulo 256 bytes (or the same
address).  The transposing ds_read_b64_tr_b8 is served in two groups of 32
consecutive lanes, each needing distinct 8-byte slots modulo 256 bytes.
"""
import numpy as np
import pytest


def sigma(c):
    return ((c >> 1) & 1) | ((c & 1) << 1) | (c & 4)


def b128_group(l):
    return 2 * ((l >> 5) & 1) + (((l >> 2) ^ (l >> 3) ^ (l >> 4)) & 1)


def b128_conflict_free(addrs):
    for g in range(4):
        seen = {}
        for l in range(64):
            if b128_group(l) != g:
                continue
            s = (addrs[l] >> 4) & 15
            if seen.setdefault(s, addrs[l]) != addrs[l]:
                return False
    return True


def tr8_conflict_free(addrs):
    for g in range(2):
        seen = {}
        for l in range(32 * g, 32 * g + 32):
            s = (addrs[l] >> 3) & 31
            if seen.setdefault(s, addrs[l]) != addrs[l]:
                return False
    return True


def test_nt_fragments_and_banks():
    rng = np.random.default_rng(0)
    for SM in (4, 8):
        WTM, BM = 16 * SM, 32 * SM
        maps = {"A": (BM, lambda row: (row // (2 * SM)) & 7), "B": (256, lambda row: (row >> 1) & 7)}
        for kind, (rows, pos) in maps.items():
            g = rng.integers(0, 256, (rows, 128), dtype=np.uint8)
            lds = np.zeros(rows * 128, np.uint8)
            for u in range(rows // 8):          # stage copies: 8 rows x 128 B per wave copy
                for l in range(64):
                    row = 8 * u + (l >> 3)
                    ch = sigma((l & 7) ^ pos(row))
                    lds[u * 1024 + 16 * l: u * 1024 + 16 * l + 16] = g[row, 16 * ch: 16 * ch + 16]
            frags = range(SM) if kind == "A" else range(4)
            for i in frags:
                for h in (0, 1):
                    addrs = []
                    for l in range(64):
                        r16, c = l & 15, (l >> 4) * 2 + h
                        row = SM * r16 + (i ^ (r16 & 1)) if kind == "A" else 16 * i + r16
                        a = row * 128 + ((sigma(c) ^ pos(row)) << 4)
                        addrs.append(a)
                        assert (lds[a:a + 16] == g[row, 16 * c: 16 * c + 16]).all()
                    assert b128_conflict_free(addrs), (SM, kind, i, h)


def test_nt_and_tn_scale_reads_conflict_free():
    for SM in (4, 8):
        for i4 in range(SM // 4):
            assert b128_conflict_free([4 * (64 * i4 + 4 * (l & 15)) for l in range(64)])
    # the old layout (a lane's SM scales consecutive) conflicts for SM = 8
    assert not b128_conflict_free([4 * (8 * (l & 15)) for l in range(64)])


def test_tn_transposing_reads_conflict_free():
    def swz(W, row):
        return ((row >> 1) & 3) | (((row >> 5) & 1) << 2) if W == 128 else (row & 7) | (((row >> 5) & 1) << 3)
    for W in (128, 256):
        for chunk in range(W // 16):
            for q in range(4):
                addrs = []
                for l in range(64):
                    k16, grp = l & 15, l >> 4
                    row = 32 * grp + (k16 >> 1) + 8 * q
                    addrs.append(row * W + ((chunk ^ swz(W, row)) << 4) + 8 * (k16 & 1))
                assert tr8_conflict_free(addrs), (W, chunk, q)


def test_epilogue_staging_round_trip_and_banks():
    """The epilogues stage the fp32 tile through LDS in 16-byte chunks: chunk
    c of staged row r sits at position c ^ f(r), f(r) = (r / SM) & 15 for the
    NT row map (a lane owns rows SM r16 + (i ^ (r16 & 1))) and r & 15 for the
    TN map (rows 16 i + r16).  Every lane's MFMA-layout write must land where
    the row reads find it, and both the writes (checked with the same 16-lane
    grouping as the reads) and the row reads must be conflict-free."""
    cases = [  # (map, SM, SN, WAVES_N, BN)
        ("nt", 8, 4, 4, 256), ("nt", 4, 4, 2, 128), ("nt", 4, 2, 2, 64), ("nt", 4, 1, 4, 64),
        ("tn", 8, 4, 4, 256)]
    for kind, SM, SN, WN, BN in cases:
        WTM, WTN, RC = 16 * SM, 16 * SN, BN // 4
        f = (lambda r: (r // SM) & 15) if kind == "nt" else (lambda r: r & 15)
        lane_row = ((lambda i, r16: SM * r16 + (i ^ (r16 & 1))) if kind == "nt"
                    else (lambda i, r16: 16 * i + r16))
        stg = {}
        for wn in range(WN):
            for i in range(SM):
                for j in range(SN):
                    addrs = []
                    for l in range(64):
                        r16 = l & 15
                        row = lane_row(i, r16)
                        ch = (wn * WTN + 16 * j) // 4 + (l >> 4)
                        a = 4 * (row * BN + 4 * (ch ^ f(row)))
                        addrs.append(a)
                        assert a not in stg
                        stg[a] = (row, 4 * ch)          # fp32 values of row, columns 4 ch .. +3
                    assert b128_conflict_free(addrs), (kind, SM, SN, BN, wn, i, j)
        assert len(stg) == WTM * BN // 4
        for base in range(0, WTM, 64 // RC):               # one wave read instruction
            addrs = []
            for l in range(64):
                row, ch = base + l // RC, l % RC
                a = 4 * (row * BN + 4 * (ch ^ f(row)))
                addrs.append(a)
                assert stg[a] == (row, 4 * ch)
            assert b128_conflict_free(addrs), (kind, SM, SN, BN, base)


def test_k_contiguous_staging_of_the_mn_kernel_is_a_bijection_and_conflict_free():
    """The MN-major kernel's K-contiguous operand staging: chunk c of row r at
    position sigma(c) ^ ((r >> 1) & 7).  The copy (lane l of copy u fills row
    8u + l/8, position l % 8) covers every (row, chunk) once, and each 16-lane
    group of a fragment read (rows 16 c + (l & 15), chunks 2 (l >> 4) (+1))
    hits 16 distinct 16-byte slots modulo 256 bytes."""
    def sig(c):
        return ((c >> 1) & 1) | ((c & 1) << 1) | (c & 4)

    def pos(r, c):
        return sig(c) ^ ((r >> 1) & 7)

    rows = 256
    seen = set()
    for u in range(rows // 8):
        for l in range(64):
            r, p = 8 * u + l // 8, l % 8
            ch = sig(p ^ ((r >> 1) & 7))
            assert pos(r, ch) == p
            seen.add((r, ch))
    assert len(seen) == rows * 8
    for frag in range(rows // 16):
        for half in (0, 1):
            slots = {}
            for l in range(64):
                r, c = 16 * frag + (l & 15), 2 * (l >> 4) + half
                byte = r * 128 + pos(r, c) * 16
                grp = 2 * ((l >> 5) & 1) + (((l >> 2) ^ (l >> 3) ^ (l >> 4)) & 1)
                slots.setdefault(grp, set()).add((byte % 256) // 16)
            assert all(len(v) == 16 for v in slots.values()), (frag, half, slots)


def b64_write_conflict_free(addrs):
    for g in range(4):
        seen = {}
        for l in range(16 * g, 16 * g + 16):
            s = (addrs[l] >> 3) & 15
            if seen.setdefault(s, addrs[l]) != addrs[l]:
                return False
    return True


def test_b64_write_rule_matches_the_measured_patterns():
    """The rule reproduces the counter's verdicts: 16 lanes at an 8-byte
    stride (or 256 + 8) are conflict-free, at a 16-byte stride (or 256 + 16)
    they conflict."""
    for stride, free in [(8, True), (264, True), (520, True), (16, False), (272, False), (32, False)]:
        addrs = [(l & 15) * stride + 8 * ((l >> 4) & 1) for l in range(64)]
        assert b64_write_conflict_free(addrs) == free, stride


@pytest.mark.parametrize("kind", ["nt", "tn"])
def test_grouped_bf16_staging_round_trip_and_banks(kind):
    """The grouped 256 x 256 epilogues (NT contiguous / masked, MN-major
    grouped NN) stage the tile once in bf16: row r holds 32 16-byte chunks,
    chunk c at position c ^ f(r), and a lane's 8-byte write (4 columns of one
    row) goes to half ((l >> 4) & 1) ^ g(r) of chunk (64 wn + 16 j) / 8 +
    (l >> 5); rows with g(r) = 1 hold their chunks' halves swapped and the
    reads swap them back.  NT: lane rows 128 wm + 8 (l & 15) + (i ^ (l & 1)),
    f(r) = (r / 8) & 15, g(r) = bit 6 of r.  MN-major: rows 128 wm + 16 i +
    (l & 15), f(r) = r & 15, g(r) = bit 3 of r.  The writes must tile the 128 KB
    exactly once and land where the row reads (lane l: chunk l & 31 of row
    wave + 16 k + 8 (l >> 5)) find them.  Bank rules, measured on gfx950 with
    the bank-conflict counter: the reads by the ds_read_b128 rule above; an
    8-byte write is served in four groups of 16 consecutive lanes, each
    conflict-free when its lanes hit 16 distinct 8-byte slots modulo 128 bytes
    (16 lanes at a 16-byte stride conflict 2-way, at an 8-byte stride not at
    all)."""
    SM, SN, WTM, WTN, ROW = 8, 4, 128, 64, 512
    if kind == "nt":
        lane_row = lambda wm, i, r16: wm * WTM + SM * r16 + (i ^ (r16 & 1))
        f, g = (lambda r: (r // SM) & 15), (lambda r: (r >> 6) & 1)
    else:
        lane_row = lambda wm, i, r16: wm * WTM + 16 * i + r16
        f, g = (lambda r: r & 15), (lambda r: (r >> 3) & 1)
    stg = {}
    for wm in range(2):
        for wn in range(4):
            for i in range(SM):
                for j in range(SN):
                    addrs = []
                    for l in range(64):
                        row = lane_row(wm, i, l & 15)
                        c = (wn * WTN + 16 * j) // 8 + (l >> 5)
                        a = row * ROW + 16 * (c ^ f(row)) + 8 * (((l >> 4) & 1) ^ g(row))
                        addrs.append(a)
                        assert a not in stg
                        stg[a] = (row, wn * WTN + 16 * j + 4 * (l >> 4))   # first of 4 columns
                    assert b64_write_conflict_free(addrs), (kind, wm, wn, i, j)
    assert len(stg) == 256 * ROW // 8
    for wave in range(8):
        for k in range(16):
            addrs = []
            for l in range(64):
                row, c = wave + 16 * k + 8 * (l >> 5), l & 31
                a = row * ROW + 16 * (c ^ f(row))
                addrs.append(a)
                lo, hi = (a + 8, a) if g(row) else (a, a + 8)   # halves swapped back
                assert stg[lo] == (row, 8 * c) and stg[hi] == (row, 8 * c + 4)
            assert b128_conflict_free(addrs), (kind, wave, k)
        # wave w stores rows w + 8 j, j = 0 .. 31, two per instruction
        assert sorted(wave + 16 * k + 8 * h for k in range(16) for h in range(2)) == \
            [wave + 8 * j for j in range(32)]
