"""GPU parity of the NN, TN and TT layouts and the M-grouped contiguous NN form
against the CPU oracle (oracle.gemm_layout, oracle.m_grouped_nn_contiguous),
through the C ABI.

Layout reading ("DeepGEMM" README, "Interfaces", "Notices"): first letter A's
("N" = stored [M, K], "T" = stored [K, M]), second letter B's ("T" = stored
[N, K], "N" = stored [K, N]); sfa [K/128, M], sfb [K/128, N] on both sides.

* Tolerance parity over tile edges (ragged M and N, several 256 x 256 tiles),
  bf16 and fp32 out, with C and in place, K = 0.
* Bit-exact: all-ones operands with power-of-two per-row / per-column scales
  (every partial sum exact in fp32), one-hot B, and dense TN equal to the
  K-grouped TN form with one group.
* Grouped NN: parity per expert, padding rows untouched, equal bit for bit to
  the dense NN form on each segment, and the 32-expert MoE shape on every valid row.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_e4m3_amd as dg
import oracle
from tests import gen
from tests.parity import FullCheck, Guarded, announce, check_close, check_full_rows, dev, to64

pytestmark = pytest.mark.gpu

FN = {"nn": dg.fp8_gemm_nn, "tn": dg.fp8_gemm_tn, "tt": dg.fp8_gemm_tt}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield


def run(x, out_dtype=torch.bfloat16, c=None):
    d = Guarded((x.M, x.N), out_dtype)
    FN[x.layout]((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d.view, c=c)
    torch.cuda.synchronize()
    assert d.intact(), "store outside D"
    return d.view


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", [
    (128, 256, 512), (16, 16, 128), (144, 272, 640), (304, 528, 1152), (1024, 2064, 1024),
])
def test_layout_parity(layout, M, N, K):
    announce(f"layout {layout} {M}x{N}x{K}")
    x = gen.gen_layout(layout, M, N, K, seed=M + N + K)
    got = to64(run(x))
    ref = oracle.gemm_layout(layout, x.a, x.sfa, x.b, x.sfb)
    print(check_close(got, ref, f"{layout} {M}x{N}x{K}"))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_xcd_blocks_deterministic_under_cu_cap(layout):
    """1024 x 2048 gives 4 x 8 = 32 tiles, which take the XCD-block tile order
    (each XCD a 2 x 2 block); a grid capped to 5 workgroups (not a multiple of
    8) walks the same tiles in another order and must give the same bits, both
    with bf16 staging (no C) and with fp32 staging (C given)."""
    announce(f"layout {layout} xcd blocks + cu cap")
    x = gen.gen_layout(layout, 1024, 2048, 512, seed=77, with_c=True)
    c = dev(x.c).to(torch.bfloat16)
    d1, d1c = run(x), run(x, c=c)
    dg.set_num_cus(5)
    try:
        d2, d2c = run(x), run(x, c=c)
    finally:
        dg.set_num_cus(0)
    assert torch.equal(d1, d2) and torch.equal(d1c, d2c)
    print(check_close(to64(d1), oracle.gemm_layout(layout, x.a, x.sfa, x.b, x.sfb), f"{layout} xcd"))


@pytest.mark.parametrize("M", [1, 65, 300])
def test_nn_ragged_m(M):
    """NN takes any M (A rows are K-contiguous)."""
    announce(f"layout nn M={M}")
    x = gen.gen_layout("nn", M, 400, 384, seed=M)
    check_close(to64(run(x)), oracle.gemm_layout("nn", x.a, x.sfa, x.b, x.sfb), f"nn M={M}")


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_f32_with_c_in_place_and_bf16_c(layout):
    M, N, K = 272, 400, 768
    announce(f"layout {layout} with C")
    x = gen.gen_layout(layout, M, N, K, seed=5, with_c=True)
    ref = oracle.gemm_layout(layout, x.a, x.sfa, x.b, x.sfb, c=x.c)
    got = to64(run(x, torch.float32, c=dev(x.c)))
    check_close(got, ref, f"{layout} f32 + C")
    d = dev(x.c)
    FN[layout]((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d, c=d)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), torch.from_numpy(got.astype(np.float32)))
    cb = dev(x.c).to(torch.bfloat16)
    gotb = to64(run(x, torch.bfloat16, c=cb))
    check_close(gotb, ref, f"{layout} bf16 + C")


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_k0_gives_c(layout):
    M, N = 64, 256
    announce(f"layout {layout} K=0")
    c = torch.randn(M, N, device="cuda")
    d = torch.full((M, N), 7.0, device="cuda")
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    s = torch.empty(0, M, device="cuda"), torch.empty(0, N, device="cuda")
    a = e.view(M, 0) if layout[0] == "n" else e.view(0, M)
    b = e.view(N, 0) if layout[1] == "t" else e.view(0, N)
    FN[layout]((a, s[0]), (b, s[1]), d, c=c)
    torch.cuda.synchronize()
    assert torch.equal(d, c)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", [(144, 272, 640), (512, 512, 2048)])
def test_layout_all_ones_bit_exact(layout, M, N, K):
    """A = B = 1.0: D = 128 * sum_kb sa[kb,m] * sb[kb,n] with power-of-two
    scales in 2^-3 .. 2^3: every partial sum is a multiple of 2^-4 below 2^17."""
    announce(f"layout {layout} all-ones {M}x{N}x{K}")
    rng = np.random.default_rng(M + K)
    KB = K // 128
    sfa = np.exp2(rng.integers(-3, 4, size=(KB, M))).astype(np.float32)
    sfb = np.exp2(rng.integers(-3, 4, size=(KB, N))).astype(np.float32)
    a = np.full((M, K) if layout[0] == "n" else (K, M), 0x38, np.uint8)
    b = np.full((N, K) if layout[1] == "t" else (K, N), 0x38, np.uint8)
    x = gen.LayoutInputs(layout, a, sfa, b, sfb, M, N, K)
    want = 128.0 * (sfa.astype(np.float64).T @ sfb.astype(np.float64))
    got = run(x, torch.float32).cpu().numpy()
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_one_hot_b_bit_exact(layout):
    M, N, K = 144, 272, 1024
    announce(f"layout {layout} one-hot B")
    rng = np.random.default_rng(9)
    x = gen.gen_layout(layout, M, N, K, seed=9)
    pi = rng.integers(0, K, size=N)
    bkn = np.zeros((K, N), np.uint8)
    bkn[pi, np.arange(N)] = 0x38
    x.b = bkn.T.copy() if layout[1] == "t" else bkn
    x.sfb = np.ones((K // 128, N), np.float32)
    A = torch.from_numpy(x.a if layout[0] == "n" else x.a.T.copy()).view(torch.float8_e4m3fn).float()
    sa = torch.from_numpy(x.sfa)                               # [KB, M]
    want = (A[:, pi] * sa[pi // 128, :].T).to(torch.bfloat16)   # one fp32 product, one rounding
    got = run(x).cpu()
    want = want + 0.0
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
        (got.float() - want.float()).abs().max()


def test_dense_tn_equals_k_grouped_single_group():
    M, N, K = 256, 512, 1024
    announce("dense tn == k-grouped tn, one group")
    x = gen.gen_layout("tn", M, N, K, seed=13)
    a, sa, b, sb = dev(x.a), dev(x.sfa), dev(x.b), dev(x.sfb)
    d1 = torch.empty(M, N, device="cuda")
    dg.fp8_gemm_tn((a, sa), (b, sb), d1)
    d2 = torch.empty(1, M, N, device="cuda")
    dg.k_grouped_fp8_gemm_tn_contiguous((a, sa), (b, sb), d2, [K])
    torch.cuda.synchronize()
    assert torch.equal(d1, d2[0])


# ------------------------------------------------------------------------------
# M-grouped contiguous NN
# ------------------------------------------------------------------------------

def run_nn_contiguous(x):
    d = Guarded((x.M_tot, x.N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nn_contiguous((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d.view,
                                        dev(x.m_indices))
    torch.cuda.synchronize()
    assert d.intact()
    return d


@pytest.mark.parametrize("counts,N,K", [([130, 0, 300, 77], 512, 1024), ([256, 1, 129], 272, 640)])
def test_nn_contiguous(counts, N, K):
    announce(f"nn contiguous counts={counts} N={N} K={K}")
    G = len(counts)
    x = gen.gen_nn_contiguous(G=G, N=N, K=K, counts=np.array(counts), seed=17)
    d = run_nn_contiguous(x)
    got = to64(d.view)
    ref = oracle.m_grouped_nn_contiguous(x.a, x.sfa, x.b, x.sfb, x.m_indices)
    check_close(got, ref, "nn contiguous")
    pad = torch.from_numpy(np.nonzero(x.m_indices < 0)[0])
    assert d.untouched(pad.cuda())
    for e in range(G):
        rows = np.nonzero(x.m_indices == e)[0]
        if len(rows) == 0:
            continue
        dd = torch.empty(x.M_tot, N, dtype=torch.bfloat16, device="cuda")
        dg.fp8_gemm_nn((dev(x.a), dev(x.sfa)), (dev(x.b[e]), dev(x.sfb[e])), dd)
        torch.cuda.synchronize()
        assert torch.equal(dd.cpu().view(torch.int16)[rows], d.view.cpu().view(torch.int16)[rows])


def test_nn_contiguous_all_padding_untouched():
    announce("nn contiguous all padding")
    x = gen.gen_nn_contiguous(G=2, N=256, K=256, counts=np.array([5, 3]), seed=1)
    x.m_indices[:] = -1
    d = run_nn_contiguous(x)
    assert d.untouched(slice(None))


def test_nn_contiguous_moe_shape_full_output():
    """32 experts, N = K = 4096, Zipf top-6 routing of 8192 tokens: every valid row."""
    announce("nn contiguous 32x4096x4096 full output")
    x = gen.gen_nn_contiguous(seed=0)
    d = run_nn_contiguous(x)
    got = d.view.float().cpu().numpy()
    # expert e's rows against the layout oracle's K-contiguous route on the
    # expert's transposed B (the NN definition, read without a stride per K step)
    fc = FullCheck("nn contiguous MoE shape")
    for e in range(x.G):
        rows_e = np.nonzero(x.m_indices == e)[0].astype(np.int64)
        if len(rows_e) == 0:
            continue
        bt = np.ascontiguousarray(x.b[e].T)
        for r0 in range(0, len(rows_e), 1024):
            rows = rows_e[r0:r0 + 1024]
            fc.add(got[rows], oracle.gemm_layout("nt", x.a, x.sfa, bt, x.sfb[e], rows=rows),
                   label=f"expert {e}")
    fc.finish(expect_n=int(x.counts.sum()) * x.N)
    pad = torch.from_numpy(np.nonzero(x.m_indices < 0)[0])
    assert d.untouched(pad.cuda())


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_bench_shape_full_output(layout):
    """The 4096 x 4096 x 7168 shape bench.py times in each layout: every
    output element."""
    M, N, K = 4096, 4096, 7168
    announce(f"layout {layout} {M}x{N}x{K} full output")
    x = gen.gen_layout(layout, M, N, K, seed=0)
    got = run(x).float().cpu().numpy()
    # the layout oracle's K-contiguous route on transposed copies of the
    # MN-major operands: the same elements in the same summation order
    at = x.a if layout[0] == "n" else np.ascontiguousarray(x.a.T)
    bt = x.b if layout[1] == "t" else np.ascontiguousarray(x.b.T)
    check_full_rows(f"{layout} {M}x{N}x{K}", got,
                    lambda rows: oracle.gemm_layout("nt", at, x.sfa, bt, x.sfb, rows=rows), M,
                    expect_n=M * N)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_max_rows(layout):
    """M * K just below 2^31 (A is 2 GiB in either orientation; M a multiple
    of 16 when A is stored [K, M]).  A is zero except a few rows m (the first,
    the last, random ones), checked against the oracle; every other row of D
    must be exactly zero."""
    K, N = 16384, 256
    M = (2**31 - 1) // K if layout[0] == "n" else ((2**31 - 1) // K) // 16 * 16
    announce(f"layout {layout} max rows {M}x{N}x{K}")
    rng = np.random.default_rng(37)
    live = np.unique(np.concatenate([np.arange(4), np.arange(M - 4, M),
                                     rng.choice(M, size=8, replace=False)])).astype(np.int64)
    x = gen.gen_layout_sparse(layout, M, N, K, live, seed=37)
    d = run(x)
    live_t = torch.from_numpy(live).cuda()
    ref = oracle.gemm_layout(layout, x.a, x.sfa, x.b, x.sfb, rows=live)
    print(check_close(to64(d[live_t]), ref, f"{layout} max rows"))
    dead = torch.ones(M, dtype=torch.bool, device="cuda")
    dead[live_t] = False
    assert int(torch.count_nonzero(d[dead])) == 0
