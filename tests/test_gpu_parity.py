"""GPU parity: the HIP kernels (through the C ABI) against the fp64 CPU oracle.

Every test builds seeded inputs with tests/gen, runs the GPU path and compares
element by element to the oracle under the stated tolerance (tests/parity.py),
or bit-exactly where the arithmetic is exact (one-hot operands, all-ones,
power-of-two scales, grouped-vs-dense identities, run-to-run determinism).
Full-size workloads are compared on sampled rows the oracle computes one by
one; guard bands and sentinel rows catch out-of-bounds and masked-row stores.
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


def run_dense(x, out_dtype=torch.bfloat16, c=None, guarded=True):
    d = Guarded((x.M, x.N), out_dtype) if guarded else None
    out = d.view if guarded else torch.empty(x.M, x.N, dtype=out_dtype, device="cuda")
    dg.fp8_gemm_nt((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), out, c=c)
    torch.cuda.synchronize()
    if guarded:
        assert d.intact(), "store outside D"
    return out


def sample_rows(M, n, rng):
    base = {0, M - 1, M // 2}
    base |= set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


# ------------------------------------------------------------------------------
# dense NT
# ------------------------------------------------------------------------------

def test_c1_dense_128x256x512_full():
    announce("dense C1 128x256x512 seed0")
    x = gen.gen_dense(128, 256, 512, seed=0)
    got = to64(run_dense(x))
    stats = check_close(got, oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb), "C1")
    print(stats)


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128), (16, 16, 128), (65, 144, 384), (127, 272, 640), (129, 400, 256),
    (300, 528, 1152), (64, 2112, 1024), (257, 2112, 256),
])
def test_dense_ragged_shapes(M, N, K):
    announce(f"dense ragged {M}x{N}x{K}")
    x = gen.gen_dense(M, N, K, seed=M * 7 + N)
    got = to64(run_dense(x))
    check_close(got, oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb), f"{M}x{N}x{K}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dense_with_c_and_in_place(out):
    announce(f"dense with C ({out})")
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    x = gen.gen_dense(200, 384, 768, seed=5, with_c=True)
    c = dev(x.c).to(dt)
    ref = oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, c=x.c)
    out = run_dense(x, dt, c=c)
    check_close(to64(out), ref, "with C")
    # in place (c == d) must give the same bits
    d = c.clone()
    dg.fp8_gemm_nt((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d, c=d)
    torch.cuda.synchronize()
    assert torch.equal(d, out)


@pytest.mark.parametrize("M,N,K,out", [(64, 256, 4096, "bf16"), (96, 1024, 4096, "f32"),
                                       (200, 384, 2048, "f32"), (1024, 1024, 8192, "bf16"),
                                       (64, 4096, 16384, "f32"), (37, 4160, 16384, "bf16"),
                                       (96, 4160, 16384, "f32")])
def test_dense_split_k_with_c_in_place_and_reproducible(M, N, K, out):
    """Shapes with far fewer output tiles than workgroup slots run with K split
    over several workgroups (64x64, 128x64, 128x128 and, for decode-size rows
    with N * K >= 64 Mi, 64x256 and 128x256 tiles here, the last two with a
    ragged N).  With C,
    in place, both output types: parity with the oracle, bitwise identical
    across runs (the partial sums are added in a fixed order), in place equal
    to out of place, and unchanged under a CU cap."""
    announce(f"dense split-K {M}x{N}x{K} {out}")
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    x = gen.gen_dense(M, N, K, seed=M + K, with_c=True)
    c = dev(x.c).to(dt)
    rows = sample_rows(M, 24, np.random.default_rng(3)) if M > 256 else None
    ref = oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, c=to64(c), rows=rows)
    d1 = run_dense(x, dt, c=c)
    got = to64(d1) if rows is None else to64(d1[torch.from_numpy(rows).cuda()])
    check_close(got, ref, "split-K")
    d2 = run_dense(x, dt, c=c)
    assert torch.equal(d1, d2)
    d = c.clone()
    dg.fp8_gemm_nt((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d, c=d)
    torch.cuda.synchronize()
    assert torch.equal(d, d1)
    dg.set_num_cus(7)
    try:
        d3 = run_dense(x, dt, c=c)
    finally:
        dg.set_num_cus(0)
    assert torch.equal(d1, d3)


def test_dense_k_zero_gives_c():
    announce("dense K=0")
    M, N = 32, 64
    c = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    d = torch.empty_like(c)
    a = torch.empty(M, 0, dtype=torch.uint8, device="cuda")
    b = torch.empty(N, 0, dtype=torch.uint8, device="cuda")
    sa = torch.empty(0, M, device="cuda")
    sb = torch.empty(1, 0, device="cuda")
    dg.fp8_gemm_nt((a, sa), (b, sb), d, c=c)
    torch.cuda.synchronize()
    assert torch.equal(d, c)


@pytest.mark.parametrize("idx", range(len(gen.DENSE_SWEEP)))
def test_c2_dense_sweep_full_size(idx):
    M, N, K = gen.DENSE_SWEEP[idx]
    announce(f"dense C2 {M}x{N}x{K} seed0")
    x = gen.gen_dense(M, N, K, seed=0)
    out = run_dense(x)
    # every output element against the oracle
    got = out.float().cpu().numpy()
    check_full_rows(f"C2 {M}x{N}x{K}", got,
                    lambda rows: oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, rows=rows), M,
                    expect_n=M * N)


# ------------------------------------------------------------------------------
# maximum sizes: the largest operands the entry point accepts (M*K and N*K just
# below 2^31, where the kernels' 32-bit offsets inside one matrix end).  The
# operands are zero outside a few live rows / blocks, so the oracle checks the
# live outputs and every other output must be exactly zero.
# ------------------------------------------------------------------------------

MAX_K = 16384


@pytest.mark.parametrize("N,tile", [(256, "128x128"), (1024, "256x256")])
def test_dense_max_rows(N, tile):
    M, K = (2**31 - 1) // MAX_K, MAX_K               # M = 131071: ragged last M tile
    announce(f"dense max rows {M}x{N}x{K}")
    assert dg.kernel_config_name(dg.FORM_DENSE, M, N, K) == f"nt_dense_bf16_{tile}"
    rng = np.random.default_rng(31)
    live = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                     rng.choice(M, size=16, replace=False)])).astype(np.int64)
    x = gen.gen_dense_sparse(M, N, K, live, range(N // 128), seed=31)
    out = run_dense(x)
    live_t = torch.from_numpy(live).cuda()
    ref = oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, rows=live)
    print(check_close(to64(out[live_t]), ref, "max rows"))
    dead = torch.ones(M, dtype=torch.bool, device="cuda")
    dead[live_t] = False
    assert int(torch.count_nonzero(out[dead])) == 0


@pytest.mark.parametrize("M", [64, 128])
def test_dense_max_cols(M):
    K = MAX_K
    N = ((2**31 - 1) // K) // 16 * 16                 # 131056: ragged last B block
    NB = (N + 127) // 128
    announce(f"dense max cols {M}x{N}x{K}")
    blocks = [0, 517, NB - 1]
    x = gen.gen_dense_sparse(M, N, K, range(M), blocks, seed=32)
    out = run_dense(x)
    cols = np.concatenate([np.arange(128 * b, min(N, 128 * b + 128)) for b in blocks])
    ref = oracle.gemm_nt(x.a, x.sfa, np.ascontiguousarray(x.b[cols]),
                         np.ascontiguousarray(x.sfb[blocks]))
    cols_t = torch.from_numpy(cols).cuda()
    print(check_close(to64(out[:, cols_t]), ref, "max cols"))
    dead = torch.ones(N, dtype=torch.bool, device="cuda")
    dead[cols_t] = False
    assert int(torch.count_nonzero(out[:, dead])) == 0


# ------------------------------------------------------------------------------
# bit-exact pins on the GPU
# ------------------------------------------------------------------------------

def test_one_hot_b_is_bit_exact():
    """b[n, pi(n)] = 1, sfb = 1: D[m,n] = fp32(dec(a[m,pi(n)]) * sa) exactly
    (one nonzero product), then one RNE to bf16 / exact in fp32."""
    announce("one-hot B")
    rng = np.random.default_rng(1)
    M, N, K = 160, 272, 512
    x = gen.gen_dense(M, N, K, seed=3)
    pi = rng.integers(0, K, N)
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), pi] = 0x38
    sfb = np.ones(((N + 127) // 128, K // 128), np.float32)
    x.b, x.sfb = b, sfb
    ref = oracle.gemm_nt(x.a, x.sfa, b, sfb)
    got32 = run_dense(x, torch.float32).cpu().numpy()
    assert np.array_equal(got32.astype(np.float64), ref.astype(np.float32).astype(np.float64))
    got16 = run_dense(x, torch.bfloat16).cpu()
    assert torch.equal(got16, torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))


def test_one_hot_a_is_bit_exact():
    announce("one-hot A")
    rng = np.random.default_rng(2)
    M, N, K = 144, 400, 384
    x = gen.gen_dense(M, N, K, seed=4)
    pi = rng.integers(0, K, M)
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), pi] = 0x38
    x.a, x.sfa = a, np.ones((K // 128, M), np.float32)
    ref = oracle.gemm_nt(a, x.sfa, x.b, x.sfb)
    got32 = run_dense(x, torch.float32).cpu().numpy()
    assert np.array_equal(got32.astype(np.float64), ref.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("K", [128, 1536, 7168])
def test_all_ones_gives_exactly_K(K):
    announce(f"all ones K={K}")
    M, N = 130, 160
    x = gen.DenseInputs(np.full((M, K), 0x38, np.uint8), np.ones((K // 128, M), np.float32),
                        np.full((N, K), 0x38, np.uint8),
                        np.ones(((N + 127) // 128, K // 128), np.float32), M, N, K)
    got = run_dense(x, torch.float32)
    assert torch.all(got == K)


def test_power_of_two_scales_are_bit_exact():
    """A = B = 1, sa = 2^(m%5 + kb%3), sb = 2^-(kb + 2 nb): every block product is
    128 and every promoted term is a power of two -> exact fp32 sums."""
    announce("power-of-two scales")
    M, N, K = 96, 384, 1024
    KB, NB = K // 128, 3
    sfa = np.array([[2.0 ** ((m % 5) + (kb % 3)) for m in range(M)] for kb in range(KB)], np.float32)
    sfb = np.array([[2.0 ** (-kb - 2 * nb) for kb in range(KB)] for nb in range(NB)], np.float32)
    x = gen.DenseInputs(np.full((M, K), 0x38, np.uint8), sfa, np.full((N, K), 0x38, np.uint8), sfb,
                        M, N, K)
    ref = oracle.gemm_nt(x.a, sfa, x.b, sfb)
    got = run_dense(x, torch.float32).cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)


def test_determinism_and_cu_cap():
    """Bitwise identical results run to run, and with the persistent grid capped
    to a few CUs (each workgroup then walks many tiles)."""
    announce("determinism + cu cap")
    x = gen.gen_dense(512, 1024, 1024, seed=9)
    d1 = run_dense(x)
    d2 = run_dense(x)
    assert torch.equal(d1, d2)
    dg.set_num_cus(3)
    try:
        assert dg.get_num_cus() == 3
        d3 = run_dense(x)
    finally:
        dg.set_num_cus(0)
    assert torch.equal(d1, d3)


# ------------------------------------------------------------------------------
# M-grouped contiguous
# ------------------------------------------------------------------------------

def run_contiguous(x):
    d = Guarded((x.M_tot, x.N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nt_contiguous((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d.view,
                                        dev(x.m_indices))
    torch.cuda.synchronize()
    assert d.intact(), "store outside D"
    return d


def test_contiguous_small_with_empty_expert_and_padding():
    announce("contiguous small, empty expert")
    x = gen.gen_contiguous(G=5, N=272, K=384, counts=np.array([130, 0, 5, 256, 1]), seed=11)
    d = run_contiguous(x)
    ref = oracle.m_grouped_contiguous(x.a, x.sfa, x.b, x.sfb, x.m_indices)
    got = to64(d.view)
    check_close(got, ref, "contiguous small")
    pad = np.nonzero(x.m_indices < 0)[0]
    assert d.untouched(torch.from_numpy(pad).cuda()), "padding rows were written"


def test_contiguous_all_padding_is_noop():
    announce("contiguous all -1")
    x = gen.gen_contiguous(G=2, N=128, K=256, counts=np.array([3, 0]), seed=12)
    x.m_indices[:] = -1
    d = run_contiguous(x)
    assert d.untouched(slice(None))


def test_contiguous_matches_dense_bitwise():
    """Each expert segment of the grouped call equals a dense call on that
    segment, bit for bit (same kernel arithmetic, same order)."""
    announce("contiguous vs dense bitwise")
    x = gen.gen_contiguous(G=3, N=256, K=512, counts=np.array([200, 128, 70]), seed=13)
    d = run_contiguous(x).view
    start = 0
    for e in range(3):
        rows = int(x.counts[e])
        seg = gen.DenseInputs(x.a[start:start + rows], np.ascontiguousarray(x.sfa[:, start:start + rows]),
                              x.b[e], x.sfb[e], rows, x.N, x.K)
        de = run_dense(seg)
        assert torch.equal(d[start:start + rows], de), f"expert {e}"
        start += ((rows + 127) // 128) * 128


def test_contiguous_expert_isolation():
    """Changing expert 1's weights changes only expert 1's rows."""
    announce("contiguous expert isolation")
    x = gen.gen_contiguous(G=3, N=128, K=256, counts=np.array([128, 128, 128]), seed=14)
    d0 = run_contiguous(x).view.clone()
    x.b[1] = np.roll(x.b[1], 1, axis=1)
    d1 = run_contiguous(x).view
    assert torch.equal(d0[:128], d1[:128]) and torch.equal(d0[256:], d1[256:])
    assert not torch.equal(d0[128:256], d1[128:256])


def test_contiguous_xcd_blocks_and_band_rest():
    """N = 4096 (16 N tiles) and 20 M tiles of 256 rows: at 256 workgroups
    the first 16 M tiles run in XCD blocks, the other 4 in band order.  One
    random row in each 128-row half of every M tile, all columns, so every
    (tile, half) pass is checked."""
    announce("contiguous XCD blocks + band rest, N=4096 K=256")
    x = gen.gen_contiguous(G=6, N=4096, K=256, counts=np.array([1000, 0, 1500, 777, 1300, 130]), seed=15)
    assert x.M_tot == 20 * 256
    d = run_contiguous(x)
    rng = np.random.default_rng(15)
    rows = np.arange(0, x.M_tot, 128) + rng.integers(0, 128, x.M_tot // 128)
    rows = rows[x.m_indices[rows] >= 0]
    got = to64(d.view[torch.from_numpy(rows).cuda()])
    ref = oracle.m_grouped_contiguous(x.a, x.sfa, x.b, x.sfb, x.m_indices, rows=rows)
    print(check_close(got, ref, "contiguous XCD blocks"))
    pad = np.nonzero(x.m_indices < 0)[0]
    assert d.untouched(torch.from_numpy(pad).cuda()), "padding rows were written"


def test_c3_contiguous_full_size():
    announce("contiguous C3 32 experts N=K=4096 zipf top6 seed0")
    x = gen.gen_contiguous(seed=0)
    d = run_contiguous(x)
    # every valid row (padding rows have no reference: NaN from the oracle)
    got = d.view.float().cpu().numpy()
    check_full_rows("C3", got,
                    lambda rows: oracle.m_grouped_contiguous(x.a, x.sfa, x.b, x.sfb, x.m_indices,
                                                             rows=rows),
                    x.M_tot, expect_n=int(x.counts.sum()) * x.N)
    pad = np.nonzero(x.m_indices < 0)[0]
    assert d.untouched(torch.from_numpy(pad).cuda())


def test_contiguous_max_rows():
    """M_tot * K just below 2^31 (the A operand is 2 GiB): segments of 32768
    rows, an empty expert, a padding block, and a last segment that ends at
    M_tot; A is zero except rows at the segment edges and a few random ones."""
    K, N, G = MAX_K, 1024, 4
    M_tot = ((2**31 - 1) // K) // 128 * 128          # 130944
    announce(f"contiguous max rows {M_tot}x{N}x{K}")
    mi = np.full(M_tot, -1, np.int32)
    mi[:32768], mi[32768:65536], mi[65664:] = 0, 1, 3      # expert 2 empty, one padding block
    rng = np.random.default_rng(33)
    live = np.unique(np.concatenate([
        np.arange(4), np.arange(32764, 32772), np.arange(65532, 65540), np.arange(65660, 65668),
        np.arange(M_tot - 4, M_tot), rng.choice(M_tot, size=8, replace=False)])).astype(np.int64)
    x = gen.gen_contiguous_sparse(mi, N, K, G, live, seed=33)
    d = run_contiguous(x)
    valid = mi >= 0
    rows = live[valid[live]]
    rows_t = torch.from_numpy(rows).cuda()
    ref = oracle.m_grouped_contiguous(x.a, x.sfa, x.b, x.sfb, mi, rows=rows)
    print(check_close(to64(d.view[rows_t]), ref, "contiguous max rows"))
    assert d.untouched(torch.from_numpy(np.nonzero(~valid)[0]).cuda())
    dead = torch.from_numpy(valid).cuda()
    dead[rows_t] = False
    assert int(torch.count_nonzero(d.view[dead])) == 0


# ------------------------------------------------------------------------------
# M-grouped masked
# ------------------------------------------------------------------------------

def run_masked(x, masked_m=None):
    mm = x.masked_m if masked_m is None else masked_m
    d = Guarded((x.G, x.M_max, x.N), torch.bfloat16)
    dg.m_grouped_fp8_gemm_nt_masked((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d.view,
                                    dev(np.asarray(mm, np.int32)))
    torch.cuda.synchronize()
    assert d.intact(), "store outside D"
    return d


def check_masked_rows_untouched(d, mm, M_max):
    for g, m in enumerate(mm):
        v = min(max(int(m), 0), M_max)
        if v < M_max:
            assert d.untouched((g, slice(v, None))), f"group {g}: rows >= {v} written"


def test_masked_edge_counts():
    mm = np.array([0, 1, 127, 128, 129, 256, -5, 999], np.int32)
    announce(f"masked edges {mm.tolist()}")
    x = gen.gen_masked(G=8, M_max=256, N=272, K=384, masked_m=mm, seed=21)
    d = run_masked(x)
    ref = oracle.m_grouped_masked(x.a, x.sfa, x.b, x.sfb, mm)
    check_close(to64(d.view), ref, "masked edges")
    check_masked_rows_untouched(d, mm, 256)


def test_masked_two_m_tiles_per_group():
    """M_max = 384: groups span one or two 256-row tiles; A rows past
    masked_m are replaced by placeholder copies and must not reach D."""
    mm = np.array([384, 300, 256, 255, 200, 8, 0], np.int32)
    announce(f"masked M_max=384 {mm.tolist()}")
    x = gen.gen_masked(G=7, M_max=384, N=528, K=640, masked_m=mm, seed=24)
    d = run_masked(x)
    ref = oracle.m_grouped_masked(x.a, x.sfa, x.b, x.sfb, mm)
    check_close(to64(d.view), ref, "masked 384")
    check_masked_rows_untouched(d, mm, 384)


def test_masked_max_rows():
    """M_max * K just below 2^31 per group (A is 2 x 2 GiB): one full group
    and one that stops at masked_m = 70000, with live A rows past masked_m
    that must not reach D."""
    K, N, G = MAX_K, 512, 2
    M_max = (2**31 - 1) // K                          # 131071
    mm = np.array([M_max, 70000], np.int32)
    announce(f"masked max rows G={G} M_max={M_max} N={N} K={K}")
    rng = np.random.default_rng(34)
    live = [np.unique(np.concatenate([np.arange(4), np.arange(M_max - 4, M_max),
                                      rng.choice(M_max, size=4, replace=False)])),
            np.unique(np.concatenate([np.arange(4), np.arange(69996, 70004),
                                      rng.choice(70000, size=4, replace=False),
                                      [M_max - 1]]))]
    x = gen.gen_masked_sparse(G, M_max, N, K, mm, live, seed=34)
    d = run_masked(x)
    groups, rows = [], []
    for g in range(G):
        r = live[g][live[g] < mm[g]]
        groups += [g] * len(r)
        rows += r.tolist()
    groups, rows = np.array(groups, np.int64), np.array(rows, np.int64)
    got = to64(d.view[torch.from_numpy(groups).cuda(), torch.from_numpy(rows).cuda()])
    ref = oracle.m_grouped_masked(x.a, x.sfa, x.b, x.sfb, mm, groups=groups, rows=rows)
    print(check_close(got, ref, "masked max rows"))
    check_masked_rows_untouched(d, mm, M_max)
    dead = torch.zeros(G, M_max, dtype=torch.bool, device="cuda")
    for g in range(G):
        dead[g, :int(mm[g])] = True
    dead[torch.from_numpy(groups).cuda(), torch.from_numpy(rows).cuda()] = False
    assert int(torch.count_nonzero(d.view[dead])) == 0


def test_masked_all_zero_writes_nothing():
    announce("masked all zero")
    x = gen.gen_masked(G=3, M_max=64, N=128, K=256, masked_m=np.zeros(3, np.int32), seed=22)
    d = run_masked(x)
    assert d.untouched(slice(None))


def test_masked_small_m_max():
    announce("masked M_max=40 (64-row tiles)")
    mm = np.array([40, 17, 0, 33], np.int32)
    x = gen.gen_masked(G=4, M_max=40, N=144, K=256, masked_m=mm, seed=23)
    d = run_masked(x)
    check_close(to64(d.view), oracle.m_grouped_masked(x.a, x.sfa, x.b, x.sfb, mm), "masked small")
    check_masked_rows_untouched(d, mm, 40)


def test_c4_masked_full_size():
    announce("masked C4 32 groups M_max=256 N=4096 K=2048 seed0")
    x = gen.gen_masked(seed=0)
    d = run_masked(x)
    # every valid row of every group
    got = d.view.float().cpu().numpy()
    fc = FullCheck("C4")
    for g in range(x.G):
        v = int(x.masked_m[g])
        if v == 0:
            continue
        rows = np.arange(v, dtype=np.int64)
        fc.add(got[g, :v], oracle.m_grouped_masked(x.a, x.sfa, x.b, x.sfb, x.masked_m,
                                                   groups=np.full(v, g), rows=rows), label=f"group {g}")
    fc.finish(expect_n=int(x.masked_m.sum()) * x.N)
    check_masked_rows_untouched(d, x.masked_m, x.M_max)


# ------------------------------------------------------------------------------
# K-grouped TN
# ------------------------------------------------------------------------------

def run_tn(x, c=None, in_place=False):
    d = Guarded((x.G, x.M, x.N), torch.float32)
    cc = None
    if c is not None:
        if in_place:
            d.view.copy_(dev(c))
            cc = d.view
        else:
            cc = dev(c)
    dg.k_grouped_fp8_gemm_tn_contiguous((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)), d.view,
                                        x.k_sizes, c=cc)
    torch.cuda.synchronize()
    assert d.intact(), "store outside D"
    return d.view


def test_k_grouped_max_k():
    """K_tot * M just below 2^31 (A [K_tot, M] is 2 GiB): groups of 2^19 and
    2^18 tokens, an empty group and a last group ending at K_tot; live tokens
    sit at the group edges and at random places."""
    M, N = 2048, 256
    K_tot = ((2**31 - 1) // M) // 128 * 128          # 1048448
    ks = np.array([2**19, 0, 2**18, K_tot - 2**19 - 2**18], np.int64)
    announce(f"k-grouped max K_tot={K_tot} M={M} N={N} k_sizes={ks.tolist()}")
    starts = np.concatenate([[0], np.cumsum(ks)[:-1]])
    rng = np.random.default_rng(35)
    live = [rng.choice(K_tot, size=8, replace=False)]
    for g in np.nonzero(ks)[0]:
        live += [starts[g] + np.arange(3), starts[g] + ks[g] - 3 + np.arange(3)]
    x = gen.gen_k_grouped_sparse(ks, M, N, np.concatenate(live), seed=35)
    d = run_tn(x, c=x.c)
    groups = np.repeat(np.arange(4), 4).astype(np.int64)
    rows = np.tile([0, 1, 1029, M - 1], 4).astype(np.int64)
    got = to64(d[torch.from_numpy(groups).cuda(), torch.from_numpy(rows).cuda()])
    ref = oracle.k_grouped_tn(x.a, x.sfa, x.b, x.sfb, x.k_sizes, x.c, groups=groups, rows=rows)
    print(check_close(got, ref, "k-grouped max K"))
    assert torch.equal(d[1], dev(x.c[1]))            # empty group: D = C


@pytest.mark.parametrize("in_place", [False, True])
def test_k_grouped_small_with_empty_groups(in_place):
    announce(f"k-grouped small in_place={in_place}")
    ks = np.array([256, 0, 640, 128, 0], np.int32)
    x = gen.gen_k_grouped(G=5, M=144, N=272, K_tot=int(ks.sum()), k_sizes=ks, seed=31)
    d = run_tn(x, c=x.c, in_place=in_place)
    ref = oracle.k_grouped_tn(x.a, x.sfa, x.b, x.sfb, x.k_sizes, x.c)
    got = d.cpu().numpy().astype(np.float64)
    check_close(got, ref, "tn small")
    for g in (1, 4):
        assert np.array_equal(got[g], x.c[g].astype(np.float64)), "K_g = 0 must give C"


def test_k_grouped_without_c():
    announce("k-grouped no C")
    ks = np.array([384, 128, 0], np.int32)
    x = gen.gen_k_grouped(G=3, M=128, N=256, K_tot=512, k_sizes=ks, seed=32, with_c=False)
    d = run_tn(x)
    ref = oracle.k_grouped_tn(x.a, x.sfa, x.b, x.sfb, x.k_sizes, None)
    got = d.cpu().numpy().astype(np.float64)
    check_close(got[:2], ref[:2], "tn no C")
    assert np.all(got[2] == 0)


def test_k_grouped_power_of_two_is_bit_exact():
    announce("k-grouped pow2 exact")
    ks = np.array([256, 128], np.int32)
    K_tot, M, N = 384, 64, 96
    a = np.full((K_tot, M), 0x38, np.uint8)
    b = np.full((K_tot, N), 0x38, np.uint8)
    sfa = np.array([[2.0 ** ((m % 4) - kb) for m in range(M)] for kb in range(3)], np.float32)
    sfb = np.array([[2.0 ** ((n % 3) + kb) for n in range(N)] for kb in range(3)], np.float32)
    x = gen.KGroupedInputs(a, sfa, b, sfb, ks, ks.astype(np.int64), None, 2, M, N, K_tot)
    got = run_tn(x).cpu().numpy().astype(np.float64)
    assert np.array_equal(got, oracle.k_grouped_tn(a, sfa, b, sfb, ks))


@pytest.mark.parametrize("M,N,ks", [(16, 16, [128, 0, 256]), (272, 528, [1280, 384]),
                                    (256, 256, [2560]), (512, 144, [128] * 7)])
def test_k_grouped_shapes(M, N, ks):
    """Tiles smaller than, equal to and ragged against the 256x256 tile; one
    long group (many K blocks through the stage ring); many short groups."""
    announce(f"k-grouped shapes M={M} N={N} ks={ks}")
    ks = np.array(ks, np.int32)
    x = gen.gen_k_grouped(G=len(ks), M=M, N=N, K_tot=int(ks.sum()), k_sizes=ks, seed=M + N)
    d = run_tn(x, c=x.c)
    ref = oracle.k_grouped_tn(x.a, x.sfa, x.b, x.sfb, x.k_sizes, x.c)
    check_close(d.cpu().numpy().astype(np.float64), ref, f"tn {M}x{N}")


def test_k_grouped_xcd_blocks_deterministic_under_cu_cap():
    """Groups of 2 x 8 tiles take the XCD-block tile order (each XCD a 2 x 1
    block of every group); capping the grid to 5 workgroups (not a multiple of
    8, each walking many tiles) must give the same bits, and both match the
    oracle."""
    announce("k-grouped xcd blocks + cu cap")
    ks = np.array([384, 0, 1024, 128], np.int32)
    x = gen.gen_k_grouped(G=len(ks), M=512, N=2048, K_tot=int(ks.sum()), k_sizes=ks, seed=41)
    d1 = run_tn(x, c=x.c)
    dg.set_num_cus(5)
    try:
        d2 = run_tn(x, c=x.c)
    finally:
        dg.set_num_cus(0)
    assert torch.equal(d1, d2)
    ref = oracle.k_grouped_tn(x.a, x.sfa, x.b, x.sfb, x.k_sizes, x.c)
    check_close(d1.cpu().numpy().astype(np.float64), ref, "tn xcd blocks")


def test_k_grouped_one_hot_k_mapping_is_bit_exact():
    """Column m of A and column n of B each hold a single 1.0 at a random K
    index inside the group; D[g][m, n] = 1 exactly where the two indices meet,
    which pins which K row every lane's transposed fragment reads."""
    announce("k-grouped one-hot K map")
    ks = np.array([256, 384], np.int32)
    K_tot, M, N = 640, 272, 528
    rng = np.random.default_rng(77)
    a = np.zeros((K_tot, M), np.uint8)
    b = np.zeros((K_tot, N), np.uint8)
    off = 0
    for kg in ks:
        # few distinct K indices so that matches are frequent
        ka = off + rng.integers(0, 8, M) * (kg // 8) + rng.integers(0, 2, M)
        kb = off + rng.integers(0, 8, N) * (kg // 8) + rng.integers(0, 2, N)
        a[ka, np.arange(M)] = 0x38
        b[kb, np.arange(N)] = 0x38
        off += int(kg)
    sfa = np.ones((K_tot // 128, M), np.float32)
    sfb = np.ones((K_tot // 128, N), np.float32)
    x = gen.KGroupedInputs(a, sfa, b, sfb, ks, ks.astype(np.int64), None, 2, M, N, K_tot)
    got = run_tn(x).cpu().numpy().astype(np.float64)
    ref = oracle.k_grouped_tn(a, sfa, b, sfb, ks)
    assert ref.sum() > 100
    assert np.array_equal(got, ref)


def test_c5_k_grouped_full_size():
    announce("k-grouped C5 32 groups M=2048 N=4096 K_tot=49152 seed0")
    x = gen.gen_k_grouped(seed=0)
    d = run_tn(x, c=x.c)
    # every (group, m) row; the reference of group g is the layout oracle's
    # K-contiguous route on the group's transposed K segment (the same
    # definition and summation order as the K-grouped route, which reads the
    # MN-major operands with a stride per K step)
    got = d.cpu().numpy()
    fc = FullCheck("C5")
    k0 = 0
    for g in range(x.G):
        k1 = k0 + int(x.k_sizes[g])
        if k1 == k0:
            ref = x.c[g].astype(np.float64)
        else:
            ref = oracle.gemm_layout("nt", np.ascontiguousarray(x.a[k0:k1].T), x.sfa[k0 // 128:k1 // 128],
                                     np.ascontiguousarray(x.b[k0:k1].T), x.sfb[k0 // 128:k1 // 128],
                                     c=x.c[g])
        fc.add(got[g], ref, label=f"group {g}")
        k0 = k1
    fc.finish(expect_n=x.G * x.M * x.N)


# ------------------------------------------------------------------------------
# small-M dense (narrow tiles, deep pipelines) and graph capture
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (128, 4096, 2048), (33, 528, 4096),
                                   (96, 208, 1280)])
def test_small_m_matches_oracle_and_is_reproducible(M, N, K):
    """Decode-size rows take the narrow-tile, multi-stage path; results match the
    oracle and are bitwise reproducible, also under a CU cap."""
    announce(f"small-M {M}x{N}x{K}")
    x = gen.gen_dense(M, N, K, seed=M + N)
    d1 = run_dense(x)
    check_close(to64(d1), oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb), "small-M")
    d2 = run_dense(x)
    assert torch.equal(d1, d2)
    dg.set_num_cus(5)
    try:
        d3 = run_dense(x)
    finally:
        dg.set_num_cus(0)
    assert torch.equal(d1, d3)


def test_graph_capture_replays_dense_and_masked():
    """Dense and masked calls captured into a HIP graph replay correctly several
    times, with eager work in between; the masked replay reads masked_m from
    device memory at replay time."""
    announce("graph capture dense + masked")
    x = gen.gen_dense(64, 1024, 2048, seed=77)
    a, sa, b, sb = dev(x.a), dev(x.sfa), dev(x.b), dev(x.sfb)
    eager = torch.empty(64, 1024, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt((a, sa), (b, sb), eager)
    torch.cuda.synchronize()
    mi = gen.gen_masked(G=4, M_max=128, N=256, K=512, masked_m=np.array([128, 5, 0, 77]), seed=78)
    ma, msa, mb, msb = dev(mi.a), dev(mi.sfa), dev(mi.b), dev(mi.sfb)
    mm = dev(mi.masked_m)
    out = torch.empty(64, 1024, dtype=torch.bfloat16, device="cuda")
    mout = Guarded((4, 128, 256), torch.bfloat16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.fp8_gemm_nt((a, sa), (b, sb), out)        # warm-up on the capture stream
        dg.m_grouped_fp8_gemm_nt_masked((ma, msa), (mb, msb), mout.view, mm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.fp8_gemm_nt((a, sa), (b, sb), out)
        dg.m_grouped_fp8_gemm_nt_masked((ma, msa), (mb, msb), mout.view, mm)
    for rep, counts in enumerate([[128, 5, 0, 77], [3, 128, 64, 0], [0, 0, 1, 128]]):
        out.zero_()
        mout.raw.fill_(mout.bits)
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"dense replay {rep}"
        ref = oracle.m_grouped_masked(mi.a, mi.sfa, mi.b, mi.sfb, np.array(counts, np.int32))
        check_close(to64(mout.view), ref, f"masked replay {rep}")
        check_masked_rows_untouched(mout, counts, 128)
        assert mout.intact()


def test_split_k_workspace_is_caller_owned_and_reusable():
    """One caller workspace serves several split shapes back to back on one
    stream (each call leaves its counters zero for the next), giving bitwise
    the results of calls that each get a fresh zero-filled workspace; a split
    shape without a workspace is refused through the C ABI."""
    announce("split-K caller workspace reuse")
    shapes = [(64, 2112, 7168), (128, 4096, 2048), (33, 528, 4096), (64, 7168, 16384),
              (128, 2112, 7168)]
    need = [dg.get_fp8_gemm_nt_workspace_bytes(*s) for s in shapes]
    assert all(n > 0 for n in need)
    ws = torch.zeros(max(need), dtype=torch.uint8, device="cuda")
    xs = [gen.gen_dense(*s, seed=300 + i) for i, s in enumerate(shapes)]
    ops = [((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb))) for x in xs]
    fresh = []
    for (M, N, K), (a, b) in zip(shapes, ops):
        d = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        dg.fp8_gemm_nt(a, b, d, workspace=dg.make_fp8_gemm_nt_workspace(M, N, K))
        fresh.append(d)
    for rep in range(3):
        outs = []
        for (M, N, K), (a, b) in zip(shapes, ops):
            d = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            dg.fp8_gemm_nt(a, b, d, workspace=ws)
            outs.append(d)
        torch.cuda.synchronize()
        for s_, d, f in zip(shapes, outs, fresh):
            assert torch.equal(d, f), f"reuse {rep} {s_}"
    assert int(ws[:1024].view(torch.int32).abs().sum().item()) == 0, "counters left non-zero"
    check_close(to64(fresh[0]), oracle.gemm_nt(xs[0].a, xs[0].sfa, xs[0].b, xs[0].sfb), "reuse[0]")
    lib = dg.load_library()
    (a, sa), (b, sb) = ops[0]
    d = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
    st = lib.dg_fp8_gemm_nt(dg._ptr(a), dg._ptr(sa), dg._ptr(b), dg._ptr(sb), None, dg._ptr(d),
                            dg.DG_BF16, 64, 2112, 7168, None, 0,
                            torch.cuda.current_stream().cuda_stream)
    assert st == dg.DG_ERR_INVALID_ARG and b"workspace" in lib.dg_last_error()


def test_captured_split_k_survives_later_eager_calls():
    """A split-K call captured into a graph with a caller workspace replays
    bitwise equal to the eager call, also after eager calls of larger split
    shapes ran on the capture stream in between (nothing the graph holds is
    freed or regrown behind it)."""
    announce("captured split-K vs later eager split-K")
    small = gen.gen_dense(64, 1024, 2048, seed=91)
    big = gen.gen_dense(128, 7168, 16384, seed=92)
    sa_, sb_ = (dev(small.a), dev(small.sfa)), (dev(small.b), dev(small.sfb))
    ba_, bb_ = (dev(big.a), dev(big.sfa)), (dev(big.b), dev(big.sfb))
    assert 0 < dg.get_fp8_gemm_nt_workspace_bytes(64, 1024, 2048) < \
        dg.get_fp8_gemm_nt_workspace_bytes(128, 7168, 16384)
    eager = torch.empty(64, 1024, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt(sa_, sb_, eager)
    big_ref = torch.empty(128, 7168, dtype=torch.bfloat16, device="cuda")
    dg.fp8_gemm_nt(ba_, bb_, big_ref)
    torch.cuda.synchronize()
    ws_small = dg.make_fp8_gemm_nt_workspace(64, 1024, 2048)
    ws_big = dg.make_fp8_gemm_nt_workspace(128, 7168, 16384)
    out = torch.empty(64, 1024, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.fp8_gemm_nt(sa_, sb_, out, workspace=ws_small)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.fp8_gemm_nt(sa_, sb_, out, workspace=ws_small)
    for rep in range(3):
        big_out = torch.empty(128, 7168, dtype=torch.bfloat16, device="cuda")
        with torch.cuda.stream(s):
            dg.fp8_gemm_nt(ba_, bb_, big_out, workspace=ws_big)     # eager, capture stream
        torch.cuda.synchronize()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        assert torch.equal(big_out, big_ref), f"eager big {rep}"
    check_close(to64(eager), oracle.gemm_nt(small.a, small.sfa, small.b, small.sfb), "captured split")
