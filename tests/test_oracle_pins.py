"""Pins of the fp64 CPU oracle against things other than itself.

* The e4m3 decoder against torch's float8_e4m3fn (an independent
  implementation) on all 256 codes, plus the OCP E4M3FN special values.
* Every oracle entry point against exact rational arithmetic
  (fractions.Fraction) on tiny random shapes, including subnormal and extreme
  codes, with operands decoded by torch, not by the oracle.
* Closed forms: all-ones, power-of-two scales, one-hot operands.
* A float64 library matmul (numpy) on moderate shapes.
* A hand-worked example stored under tests/golden/.
* Group invariants: padding rows, masked rows, empty K groups.

The definition being pinned: D = C + A @ B^T with one fp32 scale per
(row, 128-K block) of A and per 128x128 block of B, the scaled block sums
promoted once per 128-wide K block ("DeepGEMM" README, "Interfaces",
"Notices"; news article "Deepseek AI Libera Deepgemm ...", section
"Details and technical benefits").
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent helpers (torch decode, exact rationals)
# --------------------------------------------------------------------------

def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def random_codes(rng, shape, extremes=True):
    """Random finite e4m3 codes (no 0x7F / 0xFF NaN patterns)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    if extremes:
        flat = c.reshape(-1)
        flat[: min(4, flat.size)] = [0x7E, 0xFE, 0x01, 0x81][: min(4, flat.size)]
    return c


def random_scales(rng, shape):
    return (np.exp(rng.normal(0, 2, size=shape))).astype(np.float32)


def exact_nt(a, sfa, b, sfb, c=None):
    """Exact rational D for a tiny dense NT problem; returns (value, bound)."""
    M, K = a.shape
    N = b.shape[0]
    KB = K // 128
    da = [[Fraction(float(x)) for x in row] for row in torch_decode(a)]
    db = [[Fraction(float(x)) for x in row] for row in torch_decode(b)]
    val = np.zeros((M, N))
    bound = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for kb in range(KB):
                p = sum(da[m][k] * db[n][k] for k in range(kb * 128, (kb + 1) * 128))
                s = Fraction(float(sfa[kb, m])) * Fraction(float(sfb[n // 128, kb]))
                tot += s * p
                mag += abs(s * p)
            if c is not None:
                tot += Fraction(float(c[m, n]))
                mag += abs(Fraction(float(c[m, n])))
            val[m, n] = float(tot)
            # fp64: one rounding per s*p and per running-sum step, plus C
            bound[m, n] = float(mag) * (2 * KB + 2) * 2.0 ** -53 + 1e-300
    return val, bound


def assert_exact(got, want, bound):
    err = np.abs(got - want)
    assert np.all(err <= bound), (err.max(), bound[err > bound][:4])


# --------------------------------------------------------------------------
# decoder
# --------------------------------------------------------------------------

def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros too
    assert math.copysign(1.0, mine[0x80]) == -1.0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0xB8, -1.0), (0x30, 0.5),
])
def test_decode_special_values(code, value):
    assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == value


# --------------------------------------------------------------------------
# dense NT vs exact rationals
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,M,N,K", [(0, 3, 5, 128), (1, 4, 3, 256), (2, 2, 130, 384),
                                        (3, 5, 4, 512)])
def test_dense_matches_exact_rationals(seed, M, N, K):
    rng = np.random.default_rng(seed)
    a = random_codes(rng, (M, K))
    b = random_codes(rng, (N, K))
    sfa = random_scales(rng, (K // 128, M))
    sfb = random_scales(rng, ((N + 127) // 128, K // 128))
    c = rng.normal(size=(M, N)).astype(np.float32) if seed % 2 else None
    got = oracle.gemm_nt(a, sfa, b, sfb, c)
    # keep the rational loop small: for wide N check a column subset that
    # straddles the 128-column scale blocks
    cols = range(N) if N <= 8 else [0, 1, 127, 128, 129, N - 1]
    for n in cols:
        want, bound = exact_nt(a, sfa, b[n:n + 1], sfb[n // 128: n // 128 + 1],
                               None if c is None else c[:, n:n + 1])
        assert_exact(got[:, n:n + 1], want, bound)


def test_dense_row_selection_is_consistent():
    rng = np.random.default_rng(7)
    M, N, K = 9, 16, 256
    a = random_codes(rng, (M, K)); b = random_codes(rng, (N, K))
    sfa = random_scales(rng, (2, M)); sfb = random_scales(rng, (1, 2))
    full = oracle.gemm_nt(a, sfa, b, sfb)
    rows = np.array([8, 0, 3, 3])
    assert np.array_equal(oracle.gemm_nt(a, sfa, b, sfb, rows=rows), full[rows])


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K", [128, 512, 7168])
def test_all_ones_gives_K(K):
    M, N = 3, 20
    a = np.full((M, K), 0x38, np.uint8)       # 1.0
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.ones((K // 128, M), np.float32)
    sfb = np.ones(((N + 127) // 128, K // 128), np.float32)
    assert np.all(oracle.gemm_nt(a, sfa, b, sfb) == K)


def test_power_of_two_scales_pick_the_right_blocks():
    """A = B = 1, sa[kb,m] = 2^(m+kb), sb[nb,kb] = 2^(-3kb - 5nb):
    D[m,n] = 128 * sum_kb 2^(m + kb - 3kb - 5 nb(n)), exact in fp64."""
    M, N, K = 4, 300, 512
    KB, NB = K // 128, 3
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.array([[2.0 ** (m + kb) for m in range(M)] for kb in range(KB)], np.float32)
    sfb = np.array([[2.0 ** (-3 * kb - 5 * nb) for kb in range(KB)] for nb in range(NB)],
                   np.float32)
    want = np.array([[128 * sum(2.0 ** (m + kb - 3 * kb - 5 * (n // 128)) for kb in range(KB))
                      for n in range(N)] for m in range(M)])
    assert np.array_equal(oracle.gemm_nt(a, sfa, b, sfb), want)


def test_one_hot_b_selects_a_column():
    """b[n, pi(n)] = 1, sfb = 1  =>  D[m, n] = dec(a[m, pi(n)]) * sa[pi(n)/128, m]."""
    rng = np.random.default_rng(3)
    M, N, K = 6, 32, 384
    a = random_codes(rng, (M, K))
    sfa = random_scales(rng, (K // 128, M))
    pi = rng.integers(0, K, N)
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), pi] = 0x38
    sfb = np.ones((1, K // 128), np.float32)
    got = oracle.gemm_nt(a, sfa, b, sfb)
    da = torch_decode(a)
    want = np.array([[da[m, pi[n]] * float(sfa[pi[n] // 128, m]) for n in range(N)]
                     for m in range(M)])
    assert np.array_equal(got, want)


def test_one_hot_a_selects_a_row_of_b():
    """a[m, pi(m)] = 1, sfa = 1 => D[m, n] = dec(b[n, pi(m)]) * sb[n/128, pi(m)/128]."""
    rng = np.random.default_rng(4)
    M, N, K = 5, 260, 256
    b = random_codes(rng, (N, K))
    sfb = random_scales(rng, (3, K // 128))
    pi = rng.integers(0, K, M)
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), pi] = 0x38
    sfa = np.ones((K // 128, M), np.float32)
    got = oracle.gemm_nt(a, sfa, b, sfb)
    db = torch_decode(b)
    want = np.array([[db[n, pi[m]] * float(sfb[n // 128, pi[m] // 128]) for n in range(N)]
                     for m in range(M)])
    assert np.array_equal(got, want)


def test_dense_against_float64_matmul():
    """numpy float64 matmul per K block on torch-decoded operands."""
    rng = np.random.default_rng(11)
    M, N, K = 48, 272, 1024
    a = random_codes(rng, (M, K)); b = random_codes(rng, (N, K))
    sfa = random_scales(rng, (K // 128, M)); sfb = random_scales(rng, (3, K // 128))
    c = rng.normal(size=(M, N)).astype(np.float32)
    da, db = torch_decode(a), torch_decode(b)
    want = c.astype(np.float64).copy()
    mag = np.abs(c).astype(np.float64)
    for kb in range(K // 128):
        p = da[:, kb * 128:(kb + 1) * 128] @ db[:, kb * 128:(kb + 1) * 128].T
        s = sfa[kb].astype(np.float64)[:, None] * np.repeat(sfb[:, kb], 128)[:N][None, :]
        want += s * p
        mag += np.abs(s * p)
    got = oracle.gemm_nt(a, sfa, b, sfb, c)
    assert np.all(np.abs(got - want) <= mag * 64 * 2.0 ** -52)


def test_hand_worked_golden():
    with open(os.path.join(GOLDEN, "hand_worked_nt.json")) as f:
        g = json.load(f)
    M, N, K = g["M"], g["N"], g["K"]
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    for (m, k, code) in g["a_nonzero"]:
        a[m, k] = int(code, 16)
    for (n, k, code) in g["b_nonzero"]:
        b[n, k] = int(code, 16)
    sfa = np.array(g["sfa"], np.float32)
    sfb = np.array(g["sfb"], np.float32)
    assert np.array_equal(oracle.gemm_nt(a, sfa, b, sfb), np.array(g["D"], np.float64))


# --------------------------------------------------------------------------
# grouped forms vs exact rationals and their invariants
# --------------------------------------------------------------------------

def test_contiguous_matches_exact_rationals():
    rng = np.random.default_rng(21)
    G, N, K = 3, 4, 256
    m_idx = np.array([0, 0, 2, -1, 1, 2, 7, 1], np.int32)     # 7 >= G: no reference
    M_tot = len(m_idx)
    a = random_codes(rng, (M_tot, K)); sfa = random_scales(rng, (K // 128, M_tot))
    b = random_codes(rng, (G, N, K)); sfb = random_scales(rng, (G, 1, K // 128))
    got = oracle.m_grouped_contiguous(a, sfa, b, sfb, m_idx)
    for r in range(M_tot):
        e = m_idx[r]
        if e < 0 or e >= G:
            assert np.all(np.isnan(got[r]))
            continue
        want, bound = exact_nt(a[r:r + 1], sfa[:, r:r + 1], b[e], sfb[e])
        assert_exact(got[r:r + 1], want, bound)


def test_masked_matches_exact_rationals_and_masks_rows():
    rng = np.random.default_rng(22)
    G, M_max, N, K = 3, 5, 3, 256
    mm = np.array([2, 0, 9], np.int32)                        # 9 clamps to 5
    a = random_codes(rng, (G, M_max, K)); sfa = random_scales(rng, (G, K // 128, M_max))
    b = random_codes(rng, (G, N, K)); sfb = random_scales(rng, (G, 1, K // 128))
    got = oracle.m_grouped_masked(a, sfa, b, sfb, mm)
    for g in range(G):
        valid = min(max(int(mm[g]), 0), M_max)
        assert np.all(np.isnan(got[g, valid:]))
        if valid:
            want, bound = exact_nt(a[g, :valid], sfa[g][:, :valid], b[g], sfb[g])
            assert_exact(got[g, :valid], want, bound)


def exact_tn(a, sfa, b, sfb, k_sizes, c):
    G = len(k_sizes)
    K_tot, M = a.shape
    N = b.shape[1]
    da, db = torch_decode(a), torch_decode(b)
    val = np.zeros((G, M, N)); bound = np.zeros((G, M, N))
    k0 = 0
    for g in range(G):
        for m in range(M):
            for n in range(N):
                tot = Fraction(float(c[g, m, n])) if c is not None else Fraction(0)
                mag = abs(tot)
                for kb in range(k0 // 128, (k0 + k_sizes[g]) // 128):
                    p = sum(Fraction(float(da[k, m])) * Fraction(float(db[k, n]))
                            for k in range(kb * 128, (kb + 1) * 128))
                    s = Fraction(float(sfa[kb, m])) * Fraction(float(sfb[kb, n]))
                    tot += s * p
                    mag += abs(s * p)
                val[g, m, n] = float(tot)
                bound[g, m, n] = float(mag) * (2 * (k_sizes[g] // 128) + 2) * 2.0 ** -53 + 1e-300
        k0 += k_sizes[g]
    return val, bound


def test_k_grouped_matches_exact_rationals_with_empty_group():
    rng = np.random.default_rng(23)
    M, N = 3, 4
    k_sizes = np.array([256, 0, 128], np.int32)
    K_tot = int(k_sizes.sum())
    a = random_codes(rng, (K_tot, M)); b = random_codes(rng, (K_tot, N))
    sfa = random_scales(rng, (K_tot // 128, M)); sfb = random_scales(rng, (K_tot // 128, N))
    c = rng.normal(0, 0.01, size=(3, M, N)).astype(np.float32)
    got = oracle.k_grouped_tn(a, sfa, b, sfb, k_sizes, c)
    want, bound = exact_tn(a, sfa, b, sfb, k_sizes, c)
    assert_exact(got, want, bound)
    assert np.array_equal(got[1], c[1].astype(np.float64))    # K_g = 0  =>  D_g = C_g
    got0 = oracle.k_grouped_tn(a, sfa, b, sfb, k_sizes, None)
    assert np.all(got0[1] == 0)


def test_k_grouped_equals_dense_when_b_scale_is_blockwise():
    """With G = 1 and sb[kb, n] constant over each 128-column block, the TN form
    is the NT form on A^T, B^T (a second route through the definition)."""
    rng = np.random.default_rng(24)
    K, M, N = 384, 6, 256
    a = random_codes(rng, (K, M)); b = random_codes(rng, (K, N))
    sfa = random_scales(rng, (K // 128, M))
    sfb_blk = random_scales(rng, (N // 128, K // 128))
    sfb_tn = np.repeat(sfb_blk.T, 128, axis=1)                # [KB, N]
    tn = oracle.k_grouped_tn(a, sfa, b, sfb_tn, np.array([K], np.int32))[0]
    nt = oracle.gemm_nt(a.T.copy(), sfa, b.T.copy(), sfb_blk)
    assert np.array_equal(tn, nt)


def test_oracle_rejects_bad_k_sizes():
    a = np.zeros((256, 2), np.uint8); b = np.zeros((256, 2), np.uint8)
    sf = np.ones((2, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.k_grouped_tn(a, sf, b, sf, np.array([100, 156], np.int32))
    with pytest.raises(ValueError):
        oracle.k_grouped_tn(a, sf, b, sf, np.array([128, 256], np.int32))
