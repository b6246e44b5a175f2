"""GPU parity of the power-of-two (packed UE8M0) scale path against the CPU
oracle, through the C ABI.

Packed layout (reading of the "DeepGEMM" README, "Interfaces", "Notices"):
byte i of int32 word [k4][mn] is the exponent e of the scale 2^(e - 127) of K
block 4 k4 + i of row mn; both operands carry per-row scales.  The oracle is
oracle.gemm_nt_ue8m0 / oracle.pack_ue8m0 (fp64, exact block sums).

* The packer, bit-exact against the oracle's packer (both layouts, batches,
  ragged row counts, partial last words).
* Dense GEMM: tolerance parity on every tile configuration (64x64, 64x256, 128x64,
  128x256, 128x128, 256x256) and on split-K shapes, ragged M / N, fp32 out with C and
  in place, and bit-exact results where the arithmetic is exact (all-ones
  operands with per-row, per-K-block exponents; one-hot B).
* B exponents that differ row by row inside a 128-row block (the packed
  format carries one exponent per row).
* Contiguous and masked grouped forms: parity, untouched padding / masked
  rows, grouped == dense bitwise per segment.
* The pipeline cast (power-of-two scales) -> pack -> GEMM against the oracle.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_e4m3_amd as dg
import oracle
from tests import gen
from tests.parity import FullCheck, Guarded, announce, check_close, check_full_rows, dev, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield
    dg.set_num_cus(0)


def run_dense(a, sfa_w, b, sfb_w, M, N, out_dtype=torch.bfloat16, c=None):
    d = Guarded((M, N), out_dtype)
    dg.fp8_gemm_nt((dev(a), dev(sfa_w)), (dev(b), dev(sfb_w)), d.view, c=c)
    torch.cuda.synchronize()
    assert d.intact(), "store outside D"
    return d.view


def sample_rows(M, n, rng):
    base = {0, M - 1, M // 2}
    base |= set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


def random_codes(rng, shape):
    """Random e4m3 codes without the two NaN codes."""
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)          # skip 0x7F
    return np.where(c >= 0xFF, 0xFE, c).astype(np.uint8)


# ------------------------------------------------------------------------------
# packer
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("per_block,G,MN,KB", [
    (False, 1, 7, 1), (False, 1, 300, 5), (False, 3, 4096, 16), (False, 2, 130, 9),
    (True, 1, 300, 5), (True, 3, 4096, 32), (True, 1, 64, 3),
])
def test_pack_ue8m0_bit_exact(per_block, G, MN, KB):
    announce(f"pack_ue8m0 per_block={per_block} G={G} MN={MN} KB={KB}")
    rng = np.random.default_rng(100 + MN + KB)
    rows = (MN + 127) // 128 if per_block else MN
    e = rng.integers(1, 255, size=(G, rows, KB) if per_block else (G, KB, MN))
    sf = gen.pow2_scales(e)
    got = dg.pack_ue8m0_scales(dev(sf), mn=MN, per_block=per_block).cpu().numpy()
    assert got.shape == (G, (KB + 3) // 4, MN)
    for g in range(G):
        want = oracle.pack_ue8m0(sf[g], per_block, MN, KB * 128)
        assert np.array_equal(got[g], want), g
    got2 = dg.pack_ue8m0_scales(dev(sf[0]), mn=MN, per_block=per_block).cpu().numpy()
    assert np.array_equal(got2, got[0])


# ------------------------------------------------------------------------------
# dense
# ------------------------------------------------------------------------------

def test_dense_ue8m0_128x256x512_full():
    announce("dense ue8m0 128x256x512 seed0")
    x = gen.gen_dense_ue8m0(128, 256, 512, seed=0)
    got = to64(run_dense(x.a, x.sfa, x.b, x.sfb, x.M, x.N))
    ref = oracle.gemm_nt_ue8m0(x.a, x.sfa, x.b, x.sfb)
    print(check_close(got, ref, "ue8m0 128x256x512"))
    # the fp32-scale definition with the same power-of-two scales is the same number
    assert np.array_equal(ref, oracle.gemm_nt(x.a, x.sfa_f32, x.b, x.sfb_f32))


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128), (16, 16, 128), (65, 144, 384), (127, 272, 640), (129, 400, 256),
    (300, 528, 1152), (257, 2112, 640),
    (64, 2112, 7168),      # 64x64 tiles, split along K
    (64, 4224, 16384),     # 64x256 tiles (N * K >= 64 Mi), split along K, ragged N
    (128, 4096, 7168),     # 128x64 tiles, split along K
    (100, 4224, 16384),    # 128x256 tiles (N * K >= 64 Mi), split along K, ragged M and N
    (640, 1024, 2048),     # 128x128 tiles
    (4096, 2048, 1024),    # 256x256 tiles
])
def test_dense_ue8m0_shapes(M, N, K):
    announce(f"dense ue8m0 {M}x{N}x{K} ({dg.kernel_config_name(0, M, N, K)})")
    x = gen.gen_dense_ue8m0(M, N, K, seed=M + N + K)
    got = to64(run_dense(x.a, x.sfa, x.b, x.sfb, M, N))
    rows = sample_rows(M, 48, np.random.default_rng(M)) if M * N * K > (1 << 31) else None
    ref = oracle.gemm_nt_ue8m0(x.a, x.sfa, x.b, x.sfb, rows=rows)
    print(check_close(got if rows is None else got[rows], ref, f"ue8m0 {M}x{N}x{K}"))


def test_dense_ue8m0_full_size_dominant_shape():
    """4096 x 7168 x 16384, the launch bench.py times: every output element."""
    M, N, K = 4096, 7168, 16384
    announce(f"dense ue8m0 {M}x{N}x{K} full output")
    x = gen.gen_dense_ue8m0(M, N, K, seed=0)
    got = run_dense(x.a, x.sfa, x.b, x.sfb, M, N).float().cpu().numpy()
    check_full_rows("ue8m0 dominant shape", got,
                    lambda rows: oracle.gemm_nt_ue8m0(x.a, x.sfa, x.b, x.sfb, rows=rows), M,
                    expect_n=M * N)


@pytest.mark.parametrize("M,N,K", [(200, 272, 640), (64, 2112, 4096)])
def test_dense_ue8m0_f32_out_with_c_and_in_place(M, N, K):
    announce(f"dense ue8m0 f32 +C {M}x{N}x{K}")
    x = gen.gen_dense_ue8m0(M, N, K, seed=9)
    c = np.random.default_rng(9).standard_normal((M, N)).astype(np.float32)
    ref = oracle.gemm_nt_ue8m0(x.a, x.sfa, x.b, x.sfb, c=c)
    got = to64(run_dense(x.a, x.sfa, x.b, x.sfb, M, N, torch.float32, c=dev(c)))
    check_close(got, ref, "ue8m0 f32 + C")
    d = dev(c)
    dg.fp8_gemm_nt((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d, c=d)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), torch.from_numpy(got.astype(np.float32)))


@pytest.mark.parametrize("M,N,K", [
    (300, 272, 640),       # 128x128, last word holds one K block
    (64, 144, 1280),       # 64x64
    (64, 2112, 4096),      # 64x64, split along K
    (128, 528, 2560),      # 128x64
    (4096, 2048, 640),     # 256x256
])
def test_dense_ue8m0_all_ones_bit_exact(M, N, K):
    """A = B = 1.0 (0x38): D[m,n] = sum_kb 128 * 2^(ea[kb,m] - 127) * 2^(eb[kb,n] - 127).
    With exponents in 124 .. 130 every term is a power of two in 2^1 .. 2^13 and
    every partial sum a multiple of 2 below 2^19, exact in fp32 whatever the
    summation order.  Exponents differ per row, per column and per K block, so
    a wrong byte, row or column shows."""
    announce(f"dense ue8m0 all-ones bit-exact {M}x{N}x{K}")
    rng = np.random.default_rng(M * 7 + K)
    KB = K // 128
    ea = rng.integers(124, 131, size=(KB, M))
    eb = rng.integers(124, 131, size=(KB, N))
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    want = 128.0 * (np.exp2(ea - 127.0).T @ np.exp2(eb - 127.0))   # exact: few terms, pow2
    got = run_dense(a, gen.ue8m0_words(ea), b, gen.ue8m0_words(eb), M, N, torch.float32)
    assert np.array_equal(got.cpu().numpy(), want.astype(np.float32))


def test_dense_ue8m0_one_hot_b_bit_exact():
    """One-hot B (b[n, pi(n)] = 1): D[m,n] = dec(a[m,pi(n)]) * 2^(ea - 127) * 2^(eb - 127),
    one exact product, so bf16 of it is bit-exact."""
    M, N, K = 130, 272, 1024
    announce("dense ue8m0 one-hot B")
    rng = np.random.default_rng(77)
    a = random_codes(rng, (M, K))
    pi = rng.integers(0, K, size=N)
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), pi] = 0x38
    KB = K // 128
    ea = rng.integers(120, 135, size=(KB, M))
    eb = rng.integers(120, 135, size=(KB, N))
    dec = torch.from_numpy(a).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    want = dec[:, pi] * np.exp2(ea[pi // 128, :].T - 127.0 + eb[pi // 128, np.arange(N)] - 127.0)
    want = want + 0.0   # -0 (code 0x80) sums with the zero products to +0
    got = run_dense(a, gen.ue8m0_words(ea), b, gen.ue8m0_words(eb), M, N)
    want_bf16 = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(got.cpu().view(torch.int16), want_bf16.view(torch.int16))


def test_dense_ue8m0_per_row_b_exponents():
    """Random codes with exponents that change from row to row inside every
    128-row block of B (and inside every A row block)."""
    M, N, K = 257, 400, 1536
    announce("dense ue8m0 per-row B exponents")
    rng = np.random.default_rng(78)
    a, b = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    ea = rng.integers(100, 140, size=(K // 128, M))
    eb = rng.integers(100, 140, size=(K // 128, N))
    sa, sb = gen.ue8m0_words(ea), gen.ue8m0_words(eb)
    got = to64(run_dense(a, sa, b, sb, M, N, torch.float32))
    check_close(got, oracle.gemm_nt_ue8m0(a, sa, b, sb), "per-row exponents")


def test_dense_ue8m0_deterministic_and_cu_cap():
    M, N, K = 64, 2112, 7168
    announce("dense ue8m0 determinism under a CU cap")
    x = gen.gen_dense_ue8m0(M, N, K, seed=5)
    r1 = run_dense(x.a, x.sfa, x.b, x.sfb, M, N).cpu()
    r2 = run_dense(x.a, x.sfa, x.b, x.sfb, M, N).cpu()
    dg.set_num_cus(5)
    try:
        r3 = run_dense(x.a, x.sfa, x.b, x.sfb, M, N).cpu()
    finally:
        dg.set_num_cus(0)
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    assert torch.equal(r1.view(torch.int16), r3.view(torch.int16))


def test_cast_pack_gemm_pipeline():
    """bf16 activations and weights -> casting kernels with power-of-two
    scales -> packer -> UE8M0 GEMM, against the oracle on the same bytes."""
    M, N, K = 256, 640, 1024
    announce("pipeline cast(pow2) -> pack -> gemm ue8m0")
    x = torch.from_numpy(gen.gen_activations((M, K), seed=11)).cuda().to(torch.bfloat16)
    w = torch.from_numpy(gen.gen_activations((N, K), seed=12)).cuda().to(torch.bfloat16)
    qa, sfa = dg.per_token_cast_to_fp8(x, pow2_scale=True)
    qb, sfb = dg.per_block_cast_to_fp8(w, pow2_scale=True)
    wa = dg.pack_ue8m0_scales(sfa)
    wb = dg.pack_ue8m0_scales(sfb, mn=N, per_block=True)
    d = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt((qa, wa), (qb, wb), d)
    d32 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d32)   # fp32-scale path, same power-of-two scales
    torch.cuda.synchronize()
    A, B = qa.cpu().numpy(), qb.cpu().numpy()
    ref = oracle.gemm_nt_ue8m0(A, wa.cpu().numpy(), B, wb.cpu().numpy())
    check_close(to64(d), ref, "pipeline ue8m0")
    check_close(to64(d32), ref, "pipeline fp32 scales")
    assert np.array_equal(ref, oracle.gemm_nt(A, sfa.cpu().numpy(), B, sfb.cpu().numpy()))


# ------------------------------------------------------------------------------
# grouped
# ------------------------------------------------------------------------------

def run_contiguous(x, wa, wb):
    d = Guarded((x.M_tot, x.N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nt_contiguous((dev(x.a), dev(wa)), (dev(x.b), dev(wb)), d.view,
                                        dev(x.m_indices))
    torch.cuda.synchronize()
    assert d.intact()
    return d


@pytest.mark.parametrize("counts,N,K", [
    ([130, 0, 300, 77], 512, 1024),
    ([256, 1, 129], 272, 640),
])
def test_contiguous_ue8m0(counts, N, K):
    announce(f"contiguous ue8m0 counts={counts} N={N} K={K}")
    G = len(counts)
    x = gen.gen_contiguous(G=G, N=N, K=K, counts=np.array(counts), seed=21, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, N)
    d = run_contiguous(x, wa, wb)
    got = to64(d.view)
    for e in range(G):
        rows = np.nonzero(x.m_indices == e)[0].astype(np.int64)
        if len(rows) == 0:
            continue
        ref = oracle.gemm_nt_ue8m0(x.a, wa, x.b[e], wb[e], rows=rows)
        check_close(got[rows], ref, f"expert {e}")
        # the same rows through the dense UE8M0 path: bitwise equal
        dd = torch.empty(x.M_tot, N, dtype=torch.bfloat16, device="cuda")
        dg.fp8_gemm_nt((dev(x.a), dev(wa)), (dev(x.b[e]), dev(wb[e])), dd)
        torch.cuda.synchronize()
        assert torch.equal(dd.cpu().view(torch.int16)[rows], d.view.cpu().view(torch.int16)[rows])
    pad = torch.from_numpy(np.nonzero(x.m_indices < 0)[0])
    assert d.untouched(pad.cuda())


def test_contiguous_ue8m0_c3_full_output():
    """The contiguous MoE workload (32 experts, N = K = 4096, Zipf top-6
    routing of 8192 tokens) with power-of-two scales: every valid row, each
    against the dense definition with its expert's weights."""
    announce("contiguous ue8m0 C3 full output")
    x = gen.gen_contiguous(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    d = run_contiguous(x, wa, wb)
    got = d.view.float().cpu().numpy()
    fc = FullCheck("C3 ue8m0")
    for e in range(x.G):
        rows_e = np.nonzero(x.m_indices == e)[0].astype(np.int64)
        for r0 in range(0, len(rows_e), 1024):
            rows = rows_e[r0:r0 + 1024]
            fc.add(got[rows], oracle.gemm_nt_ue8m0(x.a, wa, x.b[e], wb[e], rows=rows),
                   label=f"expert {e}")
    fc.finish(expect_n=int(x.counts.sum()) * x.N)
    pad = torch.from_numpy(np.nonzero(x.m_indices < 0)[0])
    assert d.untouched(pad.cuda())


@pytest.mark.parametrize("M_max,masked", [
    (256, [0, 1, 127, 128, 129, 256]),
    (384, [383, 0, 200, 5]),
    (40, [40, 3, 0]),
    (100, [100, 64, 65, 0]),
])
def test_masked_ue8m0(M_max, masked):
    G, N, K = len(masked), 528, 1152
    announce(f"masked ue8m0 M_max={M_max} masked_m={masked}")
    x = gen.gen_masked(G=G, M_max=M_max, N=N, K=K, masked_m=np.array(masked), seed=31,
                       pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, N)
    d = Guarded((G, M_max, N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nt_masked((dev(x.a), dev(wa)), (dev(x.b), dev(wb)), d.view,
                                    dev(x.masked_m))
    torch.cuda.synchronize()
    assert d.intact()
    got = to64(d.view)
    for g in range(G):
        mm = int(masked[g])
        if mm:
            ref = oracle.gemm_nt_ue8m0(x.a[g], wa[g], x.b[g], wb[g],
                                       rows=np.arange(mm, dtype=np.int64))
            check_close(got[g, :mm], ref, f"group {g}")
        if mm < M_max:
            assert d.untouched((g, slice(mm, None))), f"group {g} rows >= masked_m written"


def test_masked_ue8m0_c4_full_output():
    """The masked decode workload (32 groups, M_max = 256, N = 4096, K = 2048)
    with power-of-two scales: every valid row, untouched rows past masked_m."""
    announce("masked ue8m0 C4 full output")
    x = gen.gen_masked(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    d = Guarded((x.G, x.M_max, x.N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nt_masked((dev(x.a), dev(wa)), (dev(x.b), dev(wb)), d.view,
                                    dev(x.masked_m))
    torch.cuda.synchronize()
    assert d.intact()
    got = d.view.float().cpu().numpy()
    fc = FullCheck("C4 ue8m0")
    for g in range(x.G):
        mm = int(x.masked_m[g])
        if mm:
            rows = np.arange(mm, dtype=np.int64)
            fc.add(got[g, :mm], oracle.gemm_nt_ue8m0(x.a[g], wa[g], x.b[g], wb[g], rows=rows),
                   label=f"group {g}")
        if mm < x.M_max:
            assert d.untouched((int(g), slice(mm, None)))
    fc.finish(expect_n=int(x.masked_m.sum()) * x.N)


def test_graph_capture_replays_masked_ue8m0():
    """The UE8M0 masked form captured into a HIP graph replays correctly with
    masked_m changed in device memory between replays (and eager work between
    them)."""
    announce("graph capture masked ue8m0")
    G, M_max, N, K = 4, 256, 528, 1152
    x = gen.gen_masked(G=G, M_max=M_max, N=N, K=K, masked_m=np.array([256, 5, 0, 77]), seed=41,
                       pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, N)
    a, sa, b, sb, mm = dev(x.a), dev(wa), dev(x.b), dev(wb), dev(x.masked_m)
    d = Guarded((G, M_max, N), torch.bfloat16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d.view, mm)   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d.view, mm)
    for rep, counts in enumerate([[256, 5, 0, 77], [3, 129, 64, 0], [0, 0, 1, 256]]):
        d.raw.fill_(d.bits)
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to64(d.view)
        for gi, c in enumerate(counts):
            if c:
                ref = oracle.gemm_nt_ue8m0(x.a[gi], wa[gi], x.b[gi], wb[gi],
                                           rows=np.arange(c, dtype=np.int64))
                check_close(got[gi, :c], ref, f"replay {rep} group {gi}")
            if c < M_max:
                assert d.untouched((gi, slice(c, None))), f"replay {rep} group {gi}"
        assert d.intact()


# ------------------------------------------------------------------------------
# K-grouped TN with per-group packed words
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("k_sizes,MN", [([640, 0, 128, 1152], 300), ([128] * 9, 64),
                                        ([0, 2048], 4096)])
def test_pack_ue8m0_k_grouped_bit_exact(k_sizes, MN):
    announce(f"pack_ue8m0 k-grouped k_sizes={k_sizes} MN={MN}")
    rng = np.random.default_rng(MN)
    KB = sum(k_sizes) // 128
    sf = gen.pow2_scales(rng.integers(1, 255, size=(KB, MN)))
    got = dg.pack_ue8m0_scales_k_grouped(dev(sf), k_sizes).cpu().numpy()
    assert np.array_equal(got, oracle.pack_ue8m0_k_grouped(sf, np.array(k_sizes, np.int32)))


def run_kg(x, wa, wb, c=None, in_place=False):
    d = Guarded((x.G, x.M, x.N), torch.float32)
    cc = None
    if c is not None:
        if in_place:
            d.view.copy_(dev(c))
            cc = d.view
        else:
            cc = dev(c)
    dg.k_grouped_fp8_gemm_tn_contiguous((dev(x.a), dev(wa)), (dev(x.b), dev(wb)), d.view,
                                        x.k_sizes, c=cc)
    torch.cuda.synchronize()
    assert d.intact()
    return to64(d.view)


@pytest.mark.parametrize("with_c,in_place", [(True, False), (False, False), (True, True)])
def test_k_grouped_ue8m0_small(with_c, in_place):
    announce(f"k-grouped ue8m0 small c={with_c} in_place={in_place}")
    ks = np.array([384, 0, 640, 128, 1152], np.int32)
    x = gen.gen_k_grouped(G=5, M=272, N=528, K_tot=int(ks.sum()), k_sizes=ks, seed=61,
                          with_c=with_c, pow2=True)
    wa, wb = gen.k_grouped_ue8m0_words(x.sfa, ks), gen.k_grouped_ue8m0_words(x.sfb, ks)
    got = run_kg(x, wa, wb, c=x.c, in_place=in_place)
    ref = oracle.k_grouped_tn_ue8m0(x.a, wa, x.b, wb, ks, x.c)
    check_close(got, ref, "k-grouped ue8m0")
    want_empty = x.c[1] if with_c else np.zeros((x.M, x.N))
    assert np.array_equal(got[1], want_empty.astype(np.float64))   # K_g = 0: D = C


def test_k_grouped_ue8m0_all_ones_bit_exact():
    """A = B = 1.0 with per-column exponents in 124 .. 130: every partial sum
    is a multiple of 2 below 2^19, exact in fp32."""
    announce("k-grouped ue8m0 all-ones bit-exact")
    ks = np.array([640, 128, 0, 1280], np.int32)
    M, N = 144, 272
    K_tot = int(ks.sum())
    rng = np.random.default_rng(62)
    ea = rng.integers(124, 131, size=(K_tot // 128, M))
    eb = rng.integers(124, 131, size=(K_tot // 128, N))
    x = gen.KGroupedInputs(np.full((K_tot, M), 0x38, np.uint8), gen.pow2_scales(ea),
                           np.full((K_tot, N), 0x38, np.uint8), gen.pow2_scales(eb), ks,
                           ks.astype(np.int64), None, len(ks), M, N, K_tot)
    wa, wb = gen.k_grouped_ue8m0_words(x.sfa, ks), gen.k_grouped_ue8m0_words(x.sfb, ks)
    got = run_kg(x, wa, wb)
    kb = 0
    for g, k in enumerate(ks):
        nkb = int(k) // 128
        want = 128.0 * (np.exp2(ea[kb:kb + nkb] - 127.0).T @ np.exp2(eb[kb:kb + nkb] - 127.0))
        assert np.array_equal(got[g], want), g
        kb += nkb


def test_k_grouped_ue8m0_c5_full_output():
    """The MoE weight-gradient workload (32 groups, M = 2048, N = 4096, Zipf K
    split of 49152, fp32 C) with power-of-two scales: every (group, m) row."""
    announce("k-grouped ue8m0 C5 full output")
    x = gen.gen_k_grouped(seed=0, pow2=True)
    wa, wb = gen.k_grouped_ue8m0_words(x.sfa, x.k_sizes), gen.k_grouped_ue8m0_words(x.sfb, x.k_sizes)
    got = run_kg(x, wa, wb, c=x.c)
    # group g against the dense UE8M0 oracle on its transposed K segment and
    # its own word rows (each group's blocks start on a word boundary): the
    # same definition, read K-contiguously
    fc = FullCheck("C5 ue8m0")
    k0 = w0 = 0
    for g in range(x.G):
        kg = int(x.k_sizes[g])
        nw = (kg // 128 + 3) // 4
        if kg == 0:
            ref = x.c[g].astype(np.float64)
        else:
            ref = oracle.gemm_nt_ue8m0(np.ascontiguousarray(x.a[k0:k0 + kg].T), wa[w0:w0 + nw],
                                       np.ascontiguousarray(x.b[k0:k0 + kg].T), wb[w0:w0 + nw],
                                       c=x.c[g])
        fc.add(got[g], ref, label=f"group {g}")
        k0, w0 = k0 + kg, w0 + nw
    fc.finish(expect_n=x.G * x.M * x.N)


def test_dense_ue8m0_max_rows():
    """M * K just below 2^31 on the 256 x 256 tiles with packed scales (the A
    word rows are 131071 wide): A is zero except a few rows, power-of-two
    scales everywhere (1 on the zero rows); every other row must be exactly
    zero."""
    K, N = 16384, 1024
    M = (2**31 - 1) // K
    announce(f"ue8m0 dense max rows {M}x{N}x{K}")
    rng = np.random.default_rng(38)
    live = np.unique(np.concatenate([np.arange(4), np.arange(M - 4, M),
                                     rng.choice(M, size=8, replace=False)])).astype(np.int64)
    x = gen.gen_dense_sparse(M, N, K, live, range(N // 128), seed=38, pow2=True)
    sfa_w, sfb_w = gen.to_ue8m0(x.sfa, x.sfb, N)
    d = run_dense(x.a, sfa_w, x.b, sfb_w, M, N)
    live_t = torch.from_numpy(live).cuda()
    ref = oracle.gemm_nt_ue8m0(x.a, sfa_w, x.b, sfb_w, rows=live)
    print(check_close(to64(d[live_t]), ref, "ue8m0 max rows"))
    dead = torch.ones(M, dtype=torch.bool, device="cuda")
    dead[live_t] = False
    assert int(torch.count_nonzero(d[dead])) == 0
