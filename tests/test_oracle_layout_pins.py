"""Pins of the oracle's other memory layouts (NN, TN, TT) and the M-grouped
contiguous NN form against things other than the function itself.

Reading (the "DeepGEMM" README, "Interfaces", "Notices": D = C + A @ B named by
two layout letters, all four of NT, TN, NN and TT on the newer path): the first
letter is A's ("N": A stored [M, K]; "T": A stored [K, M]), the second is B's
("T": B stored [N, K]; "N": B stored [K, N]).  Each operand carries one fp32
scale per row of its output side (m or n) per 128-K block: sfa [K/128, M],
sfb [K/128, N].

* Exact rational arithmetic (fractions.Fraction on torch-decoded operands) on
  tiny shapes of every layout, with subnormal and +-448 codes.
* Transpose identities against the separately pinned NT and K-grouped TN
  oracles: NN(A, B) == NT(A, B^T), TT(A, B) == NT(A^T, B), TN == K-grouped TN
  with one group, bit for bit (block-constant B scales where NT needs them).
* All-ones operands with power-of-two scales: D = 128 * sum_kb sa[kb,m] sb[kb,n].
* One-hot B: a single element of A times its two scales.
* The grouped NN form equals NN per expert, and exact rationals with each row's
  own expert; padding rows have no reference.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import assert_exact, random_codes, random_scales, torch_decode


def operand_a(a, layout):
    """A(m, k) as an [M, K] array of decoded values."""
    d = torch_decode(a)
    return d if layout[0] == "n" else d.T


def operand_b(b, layout):
    """B(k, n) as a [K, N] array of decoded values."""
    d = torch_decode(b)
    return d.T if layout[1] == "t" else d


def exact_layout(layout, a, sfa, b, sfb, c=None):
    A, B = operand_a(a, layout), operand_b(b, layout)
    M, K = A.shape
    N = B.shape[1]
    val = np.zeros((M, N)); bound = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(float(c[m, n])) if c is not None else Fraction(0)
            mag = abs(tot)
            for kb in range(K // 128):
                p = sum(Fraction(float(A[m, k])) * Fraction(float(B[k, n]))
                        for k in range(kb * 128, (kb + 1) * 128))
                s = Fraction(float(sfa[kb, m])) * Fraction(float(sfb[kb, n]))
                tot += s * p
                mag += abs(s * p)
            val[m, n] = float(tot)
            bound[m, n] = float(mag) * (2 * (K // 128) + 2) * 2.0 ** -53 + 1e-300
    return val, bound


def make(layout, rng, M, N, K):
    a = random_codes(rng, (M, K) if layout[0] == "n" else (K, M))
    b = random_codes(rng, (N, K) if layout[1] == "t" else (K, N))
    return a, random_scales(rng, (K // 128, M)), b, random_scales(rng, (K // 128, N))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("seed,M,N,K", [(70, 3, 5, 128), (71, 4, 3, 384)])
def test_layouts_match_exact_rationals(layout, seed, M, N, K):
    rng = np.random.default_rng(seed)
    a, sfa, b, sfb = make(layout, rng, M, N, K)
    c = rng.normal(0, 1, size=(M, N)).astype(np.float32)
    got = oracle.gemm_layout(layout, a, sfa, b, sfb, c=c)
    want, bound = exact_layout(layout, a, sfa, b, sfb, c)
    assert_exact(got, want, bound)


def test_nn_and_tt_are_nt_on_transposed_storage():
    rng = np.random.default_rng(72)
    M, N, K = 7, 256, 384
    sfa = random_scales(rng, (K // 128, M))
    sfb_blk = random_scales(rng, (N // 128, K // 128))
    sfb = np.repeat(sfb_blk.T, 128, axis=1)                   # [KB, N], block-constant
    a_mk = random_codes(rng, (M, K))
    b_nk = random_codes(rng, (N, K))
    nt = oracle.gemm_nt(a_mk, sfa, b_nk, sfb_blk)
    assert np.array_equal(oracle.gemm_layout("nn", a_mk, sfa, b_nk.T.copy(), sfb), nt)
    assert np.array_equal(oracle.gemm_layout("tt", a_mk.T.copy(), sfa, b_nk, sfb), nt)
    assert np.array_equal(oracle.gemm_layout("nt", a_mk, sfa, b_nk, sfb), nt)


def test_tn_is_the_k_grouped_form_with_one_group():
    rng = np.random.default_rng(73)
    M, N, K = 6, 9, 512
    a, sfa, b, sfb = make("tn", rng, M, N, K)
    c = rng.normal(0, 1, size=(M, N)).astype(np.float32)
    kg = oracle.k_grouped_tn(a, sfa, b, sfb, np.array([K], np.int32), c[None])[0]
    assert np.array_equal(oracle.gemm_layout("tn", a, sfa, b, sfb, c=c), kg)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_all_ones_with_power_of_two_scales(layout):
    rng = np.random.default_rng(74)
    M, N, K = 5, 6, 640
    KB = K // 128
    a = np.full((M, K) if layout[0] == "n" else (K, M), 0x38, np.uint8)
    b = np.full((N, K) if layout[1] == "t" else (K, N), 0x38, np.uint8)
    sfa = np.exp2(rng.integers(-4, 5, size=(KB, M))).astype(np.float32)
    sfb = np.exp2(rng.integers(-4, 5, size=(KB, N))).astype(np.float32)
    want = 128.0 * (sfa.astype(np.float64).T @ sfb.astype(np.float64))
    assert np.array_equal(oracle.gemm_layout(layout, a, sfa, b, sfb), want)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_one_hot_b_selects_an_element_of_a(layout):
    rng = np.random.default_rng(75)
    M, N, K = 4, 5, 384
    a = random_codes(rng, (M, K) if layout[0] == "n" else (K, M))
    pi = rng.integers(0, K, size=N)
    bkn = np.zeros((K, N), np.uint8)
    bkn[pi, np.arange(N)] = 0x38
    b = bkn.T.copy() if layout[1] == "t" else bkn
    sfa = random_scales(rng, (K // 128, M)); sfb = random_scales(rng, (K // 128, N))
    A = operand_a(a, layout)
    want = (A[:, pi] * (sfa[pi // 128, :].T.astype(np.float64)
                        * sfb[pi // 128, np.arange(N)].astype(np.float64)))
    assert np.array_equal(oracle.gemm_layout(layout, a, sfa, b, sfb), want)


def test_grouped_nn_contiguous_is_nn_per_expert():
    rng = np.random.default_rng(76)
    G, N, K = 3, 5, 256
    m_idx = np.array([0] * 3 + [-1] * 125 + [2] * 128 + [7] * 2 + [-1] * 126, np.int32)
    M = len(m_idx)
    a = random_codes(rng, (M, K)); sfa = random_scales(rng, (K // 128, M))
    b = random_codes(rng, (G, K, N)); sfb = random_scales(rng, (G, K // 128, N))
    got = oracle.m_grouped_nn_contiguous(a, sfa, b, sfb, m_idx)
    for e in range(G):
        rows = np.nonzero(m_idx == e)[0]
        if len(rows):
            assert np.array_equal(got[rows], oracle.gemm_layout("nn", a, sfa, b[e], sfb[e], rows=rows))
    assert np.all(np.isnan(got[(m_idx < 0) | (m_idx >= G)]))
    rows = np.array([1, 200, 300], np.int64)
    assert np.array_equal(oracle.m_grouped_nn_contiguous(a, sfa, b, sfb, m_idx, rows=rows),
                          got[rows], equal_nan=True)


def test_grouped_nn_contiguous_matches_exact_rationals():
    """Each valid row of the grouped NN form against exact rational sums with
    the B operand and scales of that row's expert (a row picks its expert from
    m_indices; nothing else ties it to the per-expert NN route)."""
    rng = np.random.default_rng(78)
    G, N, K = 3, 4, 256
    m_idx = np.array([1] * 2 + [-1] * 126 + [0] * 3 + [2] * 125, np.int32)
    M = len(m_idx)
    a = random_codes(rng, (M, K)); sfa = random_scales(rng, (K // 128, M))
    b = random_codes(rng, (G, K, N)); sfb = random_scales(rng, (G, K // 128, N))
    rows = np.array([0, 1, 128, 130, 131, 255], np.int64)
    got = oracle.m_grouped_nn_contiguous(a, sfa, b, sfb, m_idx, rows=rows)
    for r_i, r in enumerate(rows):
        e = int(m_idx[r])
        want, bound = exact_layout("nn", a[r:r + 1], sfa[:, r:r + 1], b[e], sfb[e])
        assert_exact(got[r_i:r_i + 1], want, bound)


def test_k_grouped_equals_the_nt_route_on_transposed_group_segments():
    """The K-grouped TN form, group by group, equals the layout oracle's NT
    route on each group's K segment transposed to K-contiguous storage (same
    elements, same summation order: bit for bit), including an empty group
    (D = C).  The whole-output GPU checks use this route, which reads without
    a stride per K step."""
    rng = np.random.default_rng(41)
    M, N, ks = 48, 32, np.array([256, 0, 384, 128], np.int32)
    K = int(ks.sum())
    a = rng.integers(0, 256, (K, M), dtype=np.uint8)
    b = rng.integers(0, 256, (K, N), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    b[(b & 0x7F) == 0x7F] = 0
    sfa = rng.uniform(0.5, 2, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.5, 2, (K // 128, N)).astype(np.float32)
    c = rng.standard_normal((len(ks), M, N)).astype(np.float32)
    want = oracle.k_grouped_tn(a, sfa, b, sfb, ks, c)
    k0 = 0
    for g, kg in enumerate(ks):
        k1 = k0 + int(kg)
        if kg == 0:
            got = c[g].astype(np.float64)
        else:
            got = oracle.gemm_layout("nt", np.ascontiguousarray(a[k0:k1].T), sfa[k0 // 128:k1 // 128],
                                     np.ascontiguousarray(b[k0:k1].T), sfb[k0 // 128:k1 // 128], c=c[g])
        assert np.array_equal(got, want[g]), g
        k0 = k1
