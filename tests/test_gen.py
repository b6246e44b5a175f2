"""Input generators and the FP8 casting used to prepare inputs (CPU only).

The quantiser is not part of the GEMM (the pages leave casting to the user,
DeepGEMM Documentation, section 4); these tests check that its output is the
one the workloads describe: scale = amax / 448 per block, RNE e4m3 codes.
"""
import numpy as np
import pytest
import torch

from tests import gen


def decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_rows_quantiser_scale_and_error_bound():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((17, 384)).astype(np.float32)
    q, sf = gen.quantize_rows(x)
    assert q.dtype == np.uint8 and q.shape == x.shape and sf.shape == (3, 17)
    for kb in range(3):
        blk = x[:, kb * 128:(kb + 1) * 128]
        amax = np.abs(blk).max(axis=1)
        assert np.array_equal(sf[kb], (amax / np.float32(448)).astype(np.float32))
        deq = decode(q[:, kb * 128:(kb + 1) * 128]) * sf[kb][:, None]
        # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normal values
        normal = np.abs(blk) / sf[kb][:, None] >= 2.0 ** -6
        assert np.all(np.abs(deq - blk)[normal] <= 2.0 ** -4 * np.abs(blk)[normal] * 1.0001)
        # the amax element lands exactly on +-448
        idx = np.abs(blk).argmax(axis=1)
        assert np.all(np.abs(decode(q[np.arange(17), kb * 128 + idx])) == 448)


def test_blocks_quantiser_handles_partial_block():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((200, 256)).astype(np.float32)
    q, sf = gen.quantize_blocks(w)
    assert sf.shape == (2, 2)
    for nb in range(2):
        for kb in range(2):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert sf[nb, kb] == np.float32(np.abs(blk).max() / np.float32(448))


def test_cols_quantiser_layout():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((256, 40)).astype(np.float32)
    q, sf = gen.quantize_cols(x)
    assert sf.shape == (2, 40)
    assert np.array_equal(sf[1], (np.abs(x[128:]).max(axis=0) / np.float32(448)).astype(np.float32))


def test_ties_round_to_even_and_clamp():
    # 1.0625 is halfway between 1.0 and 1.125 -> 1.0 ; 1.1875 -> 1.25
    t = torch.tensor([1.0625, 1.1875, 500.0, -1000.0], dtype=torch.float32)
    codes = gen._cast_e4m3(t).numpy()
    assert list(codes) == [0x38, 0x3A, 0x7E, 0xFE]


def test_zero_block_gets_unit_scale():
    x = np.zeros((2, 128), np.float32)
    q, sf = gen.quantize_rows(x)
    assert np.all(sf == 1.0) and np.all(q == 0)


def test_generators_are_seeded():
    a = gen.gen_dense(128, 256, 512, seed=0)
    b = gen.gen_dense(128, 256, 512, seed=0)
    c = gen.gen_dense(128, 256, 512, seed=1)
    assert np.array_equal(a.a, b.a) and np.array_equal(a.sfb, b.sfb)
    assert not np.array_equal(a.a, c.a)


def test_routing_statistics_seed0():
    rng = gen._rng(0)
    counts = gen.route_topk_zipf(rng, 8192, 32, 6)
    assert counts.sum() == 8192 * 6
    assert counts.min() == 449 and counts.max() == 7484
    assert np.all(np.diff(counts[:4]) < 0)          # Zipf: the head is heaviest
    m_idx, offs = gen.contiguous_layout(counts)
    assert len(m_idx) == 51200 and np.all(offs % 128 == 0)
    # first row of each 128-row block is valid unless the whole block is padding
    blocks = m_idx.reshape(-1, 128)
    for blk in blocks:
        if blk[0] < 0:
            assert np.all(blk < 0)
        else:
            assert np.all((blk == blk[0]) | (blk == -1))


def test_masked_and_k_split_statistics_seed0():
    rng = gen._rng(0)
    mm = rng.integers(0, 257, 32)
    assert mm.sum() == 4319 and (mm == 0).sum() == 1
    rng = gen._rng(0)
    blocks = rng.multinomial(384, gen.zipf_probs(32))
    assert blocks.sum() * 128 == 49152 and blocks.max() * 128 == 12800


def test_small_grouped_generators_shapes():
    ci = gen.gen_contiguous(G=4, N=256, K=256, counts=np.array([130, 0, 5, 128]))
    assert ci.M_tot == 256 + 128 + 128 and ci.b.shape == (4, 256, 256)
    assert np.all(ci.a[130:256] == 0)                  # padding rows are zero
    mi = gen.gen_masked(G=3, M_max=64, N=128, K=256, masked_m=np.array([0, 64, 7]))
    assert mi.sfa.shape == (3, 2, 64) and mi.sfb.shape == (3, 1, 2)
    ki = gen.gen_k_grouped(G=3, M=64, N=32, K_tot=512, k_sizes=np.array([256, 0, 256]))
    assert ki.sfa.shape == (4, 64) and ki.c.shape == (3, 64, 32)
    assert np.all(ki.a[ki.valid_tokens[0]:256] == 0)


def test_pow2_quantisers_match_the_oracle_cast():
    """The generator's power-of-two scales and codes equal the oracle's casts
    with power-of-two scales (the recipe the UE8M0 inputs are made with)."""
    import oracle
    rng = np.random.default_rng(60)
    x = (rng.standard_normal((70, 384)) * np.exp(rng.uniform(-6, 6, (70, 1)))).astype(np.float32)
    q, sf = gen.quantize_rows(x, pow2=True)
    oq, osf = oracle.cast_rows(x, pow2=True)
    assert np.array_equal(q, oq) and np.array_equal(sf, osf)
    m, _ = np.frexp(sf)
    assert np.all(m == 0.5)
    w = rng.standard_normal((300, 256)).astype(np.float32)
    q, sf = gen.quantize_blocks(w, pow2=True)
    oq, osf = oracle.cast_blocks(w, pow2=True)
    assert np.array_equal(q, oq) and np.array_equal(sf, osf)


def test_ue8m0_words_match_the_oracle_packer():
    import oracle
    rng = np.random.default_rng(61)
    for KB, MN in ((1, 7), (4, 16), (5, 33), (9, 130)):
        e = rng.integers(1, 255, size=(KB, MN))
        sf = gen.pow2_scales(e)
        assert np.array_equal(gen.exponent_bytes(sf), e)
        assert np.array_equal(gen.ue8m0_words(e), oracle.pack_ue8m0(sf, False, MN, KB * 128))


def test_gen_dense_ue8m0_layout():
    import oracle
    x = gen.gen_dense_ue8m0(64, 300, 640, seed=3)
    assert x.sfa.dtype == np.int32 and x.sfa.shape == (2, 64)
    assert x.sfb.shape == (2, 300)
    assert np.array_equal(x.sfa, oracle.pack_ue8m0(x.sfa_f32, False, 64, 640))
    assert np.array_equal(x.sfb, oracle.pack_ue8m0(x.sfb_f32, True, 300, 640))


def test_k_grouped_ue8m0_words_match_the_oracle_packer():
    import oracle
    x = gen.gen_k_grouped(G=4, M=32, N=48, K_tot=1280, k_sizes=np.array([640, 0, 128, 512]),
                          seed=2, pow2=True)
    for sf in (x.sfa, x.sfb):
        assert np.array_equal(gen.k_grouped_ue8m0_words(sf, x.k_sizes),
                              oracle.pack_ue8m0_k_grouped(sf, x.k_sizes))


def test_gen_dense_sparse_structure():
    """Zero outside the live rows / blocks, scale 1 there, and the live part
    quantised (codes within e4m3 range, per-row and per-block scales)."""
    M, N, K = 300, 400, 256
    live = [0, 5, 150, 299]
    x = gen.gen_dense_sparse(M, N, K, live, [1, 3], seed=3)
    dead_rows = np.setdiff1d(np.arange(M), live)
    assert not x.a[dead_rows].any() and np.all(x.sfa[:, dead_rows] == 1)
    assert x.a[live].any(axis=1).all() and np.all(x.sfa[:, live] != 1)
    assert not x.b[:128].any() and not x.b[256:384].any()
    assert x.b[128:256].any(axis=1).all() and x.b[384:].any(axis=1).all()
    assert np.all(x.sfb[[0, 2]] == 1) and np.all(x.sfb[[1, 3]] != 1)
    assert x.sfa.shape == (K // 128, M) and x.sfb.shape == ((N + 127) // 128, K // 128)
