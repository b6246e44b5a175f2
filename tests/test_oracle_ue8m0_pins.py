"""Pins of the oracle's power-of-two (UE8M0) scale path against things other
than itself.

Reading (the "DeepGEMM" README, "Interfaces", "Notices", names packed UE8M0
scale factors, four per 32-bit integer, for its newer path): byte i of word
[k4][mn] is the exponent e of the scale 2^(e - 127) of K block 4 k4 + i for row
mn; both operands carry per-row scales (a 128 x 128 weight scale is given to
each of its rows).

* The packer against exponents computed with math.frexp, the byte order, the
  broadcast of block scales and its refusal of non-powers of two.
* The GEMM against exact rational arithmetic with every row and column of B
  on its own exponents, and against the fp32-scale oracle where the two
  definitions coincide (B exponents constant over 128-row blocks).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import random_codes, torch_decode


def rand_exponents(rng, shape, lo=110, hi=140):
    return rng.integers(lo, hi, size=shape).astype(np.int64)


def pack_bytes(e):
    """[KB, MN] exponent bytes -> [ceil(KB/4), MN] int32 words (byte i = block 4 k4 + i)."""
    KB, MN = e.shape
    K4 = (KB + 3) // 4
    w = np.zeros((K4, MN), np.uint32)
    for kb in range(KB):
        w[kb // 4] |= (e[kb].astype(np.uint32) << np.uint32(8 * (kb % 4)))
    return w.view(np.int32)


def test_pack_matches_frexp_and_byte_order():
    rng = np.random.default_rng(50)
    KB, MN = 6, 9
    e = rand_exponents(rng, (KB, MN), 1, 254)
    sf = np.ldexp(np.float32(1), (e - 127).astype(np.int32)).astype(np.float32)
    got = oracle.pack_ue8m0(sf, False, MN, KB * 128).view(np.uint32)
    assert got.shape == (2, MN)
    for kb in range(KB):
        for mn in range(MN):
            byte = (int(got[kb // 4, mn]) >> (8 * (kb % 4))) & 0xFF
            m, x = math.frexp(float(sf[kb, mn]))
            assert m == 0.5 and byte == x - 1 + 127
    assert np.all(got[1] >> 16 == 0)                   # blocks 6, 7 do not exist


def test_pack_broadcasts_block_scales_to_rows():
    rng = np.random.default_rng(51)
    N, KB = 300, 5
    e = rand_exponents(rng, (3, KB))
    sf = np.ldexp(np.float32(1), (e - 127).astype(np.int32)).astype(np.float32)
    got = oracle.pack_ue8m0(sf, True, N, KB * 128)
    want = pack_bytes(np.repeat(e.T, 128, axis=1)[:, :N])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bad", [3.0, 0.0, 2.0 ** -130, 1.5])
def test_pack_rejects_non_powers_of_two(bad):
    sf = np.ones((1, 4), np.float32)
    sf[0, 2] = bad
    with pytest.raises(ValueError):
        oracle.pack_ue8m0(sf, False, 4, 128)


def exact_ue8m0(a, ea, b, eb):
    """Exact D for tiny shapes: ea [KB, M], eb [KB, N] exponent bytes."""
    M, K = a.shape
    N = b.shape[0]
    da = [[Fraction(float(v)) for v in row] for row in torch_decode(a)]
    db = [[Fraction(float(v)) for v in row] for row in torch_decode(b)]
    val = np.zeros((M, N)); bound = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0); mag = Fraction(0)
            for kb in range(K // 128):
                p = sum(da[m][k] * db[n][k] for k in range(kb * 128, kb * 128 + 128))
                s = Fraction(2) ** (int(ea[kb, m]) - 127) * Fraction(2) ** (int(eb[kb, n]) - 127)
                tot += s * p; mag += abs(s * p)
            val[m, n] = float(tot)
            bound[m, n] = float(mag) * (2 * (K // 128) + 2) * 2.0 ** -53 + 1e-300
    return val, bound


@pytest.mark.parametrize("seed,M,N,K", [(52, 3, 5, 128), (53, 4, 6, 640), (54, 2, 17, 1152)])
def test_gemm_ue8m0_matches_exact_rationals(seed, M, N, K):
    rng = np.random.default_rng(seed)
    a = random_codes(rng, (M, K)); b = random_codes(rng, (N, K))
    ea = rand_exponents(rng, (K // 128, M)); eb = rand_exponents(rng, (K // 128, N))
    got = oracle.gemm_nt_ue8m0(a, pack_bytes(ea), b, pack_bytes(eb))
    val, bound = exact_ue8m0(a, ea, b, eb)
    assert np.all(np.abs(got - val) <= bound)


def test_gemm_ue8m0_equals_fp32_scale_definition_on_block_constant_b():
    rng = np.random.default_rng(55)
    M, N, K = 5, 256, 640
    a = random_codes(rng, (M, K)); b = random_codes(rng, (N, K))
    ea = rand_exponents(rng, (K // 128, M)); eb_blk = rand_exponents(rng, (N // 128, K // 128))
    sfa = np.ldexp(np.float32(1), (ea - 127).astype(np.int32)).astype(np.float32)
    sfb = np.ldexp(np.float32(1), (eb_blk - 127).astype(np.int32)).astype(np.float32)
    ref = oracle.gemm_nt(a, sfa, b, sfb)
    got = oracle.gemm_nt_ue8m0(a, oracle.pack_ue8m0(sfa, False, M, K), b,
                               oracle.pack_ue8m0(sfb, True, N, K))
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# K-grouped TN with per-group packed words
# --------------------------------------------------------------------------

def test_k_grouped_pack_layout_and_byte_order():
    """Each group starts on a word boundary: group g's blocks take
    ceil(KB_g / 4) word rows after the previous groups' rows."""
    rng = np.random.default_rng(56)
    k_sizes = np.array([640, 0, 128, 1152], np.int32)      # 5, 0, 1, 9 blocks
    MN = 7
    KB = int(k_sizes.sum()) // 128
    e = rand_exponents(rng, (KB, MN), 1, 254)
    sf = np.ldexp(np.float32(1), (e - 127).astype(np.int32)).astype(np.float32)
    got = oracle.pack_ue8m0_k_grouped(sf, k_sizes).view(np.uint32)
    assert got.shape == (2 + 0 + 1 + 3, MN)
    kb = 0
    w = 0
    for ksz in k_sizes:
        nkb = int(ksz) // 128
        want = pack_bytes(e[kb:kb + nkb]).view(np.uint32) if nkb else np.zeros((0, MN), np.uint32)
        assert np.array_equal(got[w:w + len(want)], want)
        kb += nkb
        w += len(want)
    assert oracle.k_grouped_word_rows(k_sizes) == 6


def test_k_grouped_ue8m0_equals_the_fp32_scale_definition():
    """With power-of-two scales the packed form is the fp32-scale K-grouped
    oracle, bit for bit (a second, separately pinned route)."""
    rng = np.random.default_rng(57)
    M, N = 5, 6
    k_sizes = np.array([384, 0, 640, 128], np.int32)
    K_tot = int(k_sizes.sum())
    a = random_codes(rng, (K_tot, M)); b = random_codes(rng, (K_tot, N))
    ea = rand_exponents(rng, (K_tot // 128, M)); eb = rand_exponents(rng, (K_tot // 128, N))
    sfa = np.ldexp(np.float32(1), (ea - 127).astype(np.int32)).astype(np.float32)
    sfb = np.ldexp(np.float32(1), (eb - 127).astype(np.int32)).astype(np.float32)
    c = rng.normal(0, 1, (4, M, N)).astype(np.float32)
    ref = oracle.k_grouped_tn(a, sfa, b, sfb, k_sizes, c)
    got = oracle.k_grouped_tn_ue8m0(a, oracle.pack_ue8m0_k_grouped(sfa, k_sizes), b,
                                    oracle.pack_ue8m0_k_grouped(sfb, k_sizes), k_sizes, c)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[1], c[1].astype(np.float64))   # empty group: D = C


def test_k_grouped_ue8m0_equals_dense_ue8m0_on_transposed_group_segments():
    """The K-grouped UE8M0 form, group by group, equals the dense UE8M0 oracle
    on the group's K segment transposed to K-contiguous storage with the
    group's own word rows (bit for bit; an empty group gives C).  The
    whole-output GPU checks use this route."""
    rng = np.random.default_rng(43)
    M, N, ks = 32, 48, np.array([640, 0, 128, 512], np.int32)
    K = int(ks.sum())
    a = rng.integers(0, 256, (K, M), dtype=np.uint8)
    b = rng.integers(0, 256, (K, N), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    b[(b & 0x7F) == 0x7F] = 0
    sfa = np.exp2(rng.integers(-6, 6, (K // 128, M))).astype(np.float32)
    sfb = np.exp2(rng.integers(-6, 6, (K // 128, N))).astype(np.float32)
    wa, wb = oracle.pack_ue8m0_k_grouped(sfa, ks), oracle.pack_ue8m0_k_grouped(sfb, ks)
    c = rng.standard_normal((len(ks), M, N)).astype(np.float32)
    want = oracle.k_grouped_tn_ue8m0(a, wa, b, wb, ks, c)
    k0 = w0 = 0
    for g, kg in enumerate(ks):
        nw = (int(kg) // 128 + 3) // 4
        if kg == 0:
            got = c[g].astype(np.float64)
        else:
            got = oracle.gemm_nt_ue8m0(np.ascontiguousarray(a[k0:k0 + kg].T), wa[w0:w0 + nw],
                                       np.ascontiguousarray(b[k0:k0 + kg].T), wb[w0:w0 + nw], c=c[g])
        assert np.array_equal(got, want[g]), g
        k0, w0 = k0 + int(kg), w0 + nw
