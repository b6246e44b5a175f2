"""GPU parity of the FP8 casting kernels (through the C ABI) against the CPU
oracle: codes and scales must match bit for bit.

Casting is integer work decided by floating point (a code per element), and
both sides take each decision in fp32 the same way (correctly rounded
amax / 448 and x / s, nearest code, ties to even), so any difference is a bug.
Full-size operands (4096 x 7168 and 51200 x 4096 per token, 8 x 4096 x 4096
per block) are checked over every row and block, streamed through the oracle
in chunks; the maximum-size cases check their live rows (blocks) against the
oracle and every other block against its closed form (zero codes, scale 1).
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_e4m3_amd as dg
import oracle
from tests import gen
from tests.parity import announce, check_close
from tests.test_oracle_cast_pins import magnitudes, quotient_ties

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield


def to_dev(x: np.ndarray, bf16: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


def cast_tokens(x: np.ndarray, bf16: bool, pow2: bool = False):
    codes, sf = dg.per_token_cast_to_fp8(to_dev(x, bf16), pow2_scale=pow2)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def cast_blocks(w: np.ndarray, bf16: bool, pow2: bool = False):
    codes, sf = dg.per_block_cast_to_fp8(to_dev(w, bf16), pow2_scale=pow2)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def assert_same(got, ref, what):
    gc, gs = got
    rc, rs = ref
    assert gs.shape == rs.shape and gc.shape == rc.shape, what
    bad_s = np.nonzero(gs.view(np.uint32) != rs.view(np.uint32))
    assert len(bad_s[0]) == 0, f"{what}: {len(bad_s[0])} scales differ, first at {bad_s[0][:4]}"
    bad = np.argwhere(gc != rc)
    assert len(bad) == 0, f"{what}: {len(bad)} codes differ, first {bad[:4].tolist()} " \
                          f"got {gc[tuple(bad[0])]:#04x} want {rc[tuple(bad[0])]:#04x}"


# ------------------------------------------------------------------------------
# per token (1 x 128)
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("pow2", [False, True])
def test_per_token_ragged_rows(bf16, pow2):
    announce(f"cast per token 200x640 bf16={bf16} pow2={pow2}")
    x = gen.gen_activations((200, 640), seed=30, bf16=bf16)
    assert_same(cast_tokens(x, bf16, pow2), oracle.cast_rows(x, pow2=pow2), "per token")


def test_per_token_every_code_midpoint_and_neighbour():
    """s = 1 (each block holds 448): every code value, every midpoint between
    neighbouring codes and the fp32 values either side of it, subnormals,
    signed zeros, with both signs."""
    announce("cast per token, exhaustive code/midpoint sweep")
    mags = magnitudes()
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mags.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf)),
                           np.float32(2.0 ** -10) * np.arange(0, 16, dtype=np.float32),
                           np.array([1e-30, 1e-40, 447.9, 448.0], np.float32)])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    per_row = 127
    rows = (len(vals) + per_row - 1) // per_row
    x = np.zeros((rows, 128), np.float32)
    flat = np.zeros(rows * per_row, np.float32)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(rows, per_row)
    x[:, 0] = 448.0
    got = cast_tokens(x, bf16=False)
    assert np.all(got[1] == 1.0)
    assert_same(got, oracle.cast_rows(x), "code sweep")


def test_per_token_quotient_ties_need_true_division():
    """Values whose fp32 quotient by s = 3/448 sits exactly on a midpoint
    while x * (1/s) does not."""
    announce("cast per token, quotient ties at s=3/448")
    ties = quotient_ties(np.float32(3.0) / np.float32(448.0), 200)
    assert len(ties) >= 20
    x = np.zeros((4, 128), np.float32)
    x[:, 0] = 3.0
    flat = np.resize(ties, 4 * 127)
    x[:, 1:] = (flat * np.where(np.arange(4 * 127) % 2, -1, 1)).reshape(4, 127)
    assert_same(cast_tokens(x, bf16=False), oracle.cast_rows(x), "quotient ties")


def test_per_token_masked_layout_batched():
    announce("cast per token G=3 R=77 K=256 (masked layout)")
    x = gen.gen_activations((3, 77, 256), seed=31)
    got = cast_tokens(x, bf16=True)
    assert got[1].shape == (3, 2, 77)
    assert_same(got, oracle.cast_rows(x), "batched")


def test_per_token_empty_and_out_buffers():
    x = torch.zeros(0, 256, dtype=torch.bfloat16, device="cuda")
    codes, sf = dg.per_token_cast_to_fp8(x)
    assert codes.shape == (0, 256) and sf.shape == (2, 0)
    xs = gen.gen_activations((64, 256), seed=32)
    codes = torch.full((64, 256), 0x5A, dtype=torch.uint8, device="cuda")
    sf = torch.full((2, 64), -1.0, device="cuda")
    dg.per_token_cast_to_fp8(to_dev(xs, True), out=(codes, sf))
    torch.cuda.synchronize()
    assert_same((codes.cpu().numpy(), sf.cpu().numpy()), oracle.cast_rows(xs), "out buffers")
    with pytest.raises(ValueError):
        dg.per_token_cast_to_fp8(torch.zeros(4, 200, dtype=torch.bfloat16, device="cuda"))


# ------------------------------------------------------------------------------
# per block (128 x 128)
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("bf16,pow2", [(True, False), (False, False), (True, True)])
def test_per_block_ragged_n_batched(bf16, pow2):
    announce(f"cast per block G=2 N=300 K=384 bf16={bf16} pow2={pow2}")
    w = gen.gen_activations((2, 300, 384), seed=33, bf16=bf16)
    got = cast_blocks(w, bf16, pow2)
    assert got[1].shape == (2, 3, 3)
    assert_same(got, oracle.cast_blocks(w, pow2=pow2), "per block")


# ------------------------------------------------------------------------------
# cast -> GEMM: the kernels' outputs are the GEMM's operands
# ------------------------------------------------------------------------------

def test_cast_then_gemm_matches_oracle_pipeline():
    announce("cast x and w on the GPU, then dense GEMM 192x384x512")
    x = gen.gen_activations((192, 512), seed=34)
    w = gen.gen_activations((384, 512), seed=35)
    a, sfa = dg.per_token_cast_to_fp8(to_dev(x, True))
    b, sfb = dg.per_block_cast_to_fp8(to_dev(w, True))
    d = torch.empty(192, 384, dtype=torch.float32, device="cuda")
    dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    ra, rsa = oracle.cast_rows(x)
    rb, rsb = oracle.cast_blocks(w)
    assert_same((a.cpu().numpy(), sfa.cpu().numpy()), (ra, rsa), "A")
    assert_same((b.cpu().numpy(), sfb.cpu().numpy()), (rb, rsb), "B")
    ref = oracle.gemm_nt(ra, rsa, rb, rsb)
    print(check_close(d.cpu().numpy().astype(np.float64), ref, "cast -> GEMM"))


# ------------------------------------------------------------------------------
# full sizes, every output compared (bit-exact), streamed in row chunks
# ------------------------------------------------------------------------------

def device_activations(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    x *= torch.exp(1.5 * torch.randn(shape[:-1] + (1,), generator=g, device="cuda"))
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("R,K", [(4096, 7168), (51200, 4096)])
def test_per_token_full_size_every_row(R, K):
    announce(f"cast per token full size {R}x{K} bf16, every row")
    x = device_activations((R, K), seed=R)
    codes, sf = dg.per_token_cast_to_fp8(x)
    torch.cuda.synchronize()
    for r0 in range(0, R, 4096):
        rr = slice(r0, min(R, r0 + 4096))
        ref = oracle.cast_rows(x[rr].float().cpu().numpy())
        assert_same((codes[rr].cpu().numpy(), sf[:, rr].cpu().numpy()), ref, f"rows {r0}..")


def test_per_block_full_size_every_block():
    G, N, K = 8, 4096, 4096
    announce(f"cast per block full size G={G} N={N} K={K} bf16, every block")
    w = device_activations((G, N, K), seed=36)
    codes, sf = dg.per_block_cast_to_fp8(w)
    torch.cuda.synchronize()
    for g in range(G):
        ref = oracle.cast_blocks(w[g].float().cpu().numpy())
        assert_same((codes[g].cpu().numpy(), sf[g].cpu().numpy()), ref, f"group {g}")


# ------------------------------------------------------------------------------
# maximum sizes: rows * K just below 2^31 in each of two groups, so offsets
# pass 2^32.  The input is zero except a few rows (blocks); those are checked
# against the oracle, and every zero block must give zero codes and scale 1.
# ------------------------------------------------------------------------------

MAX_K = 16384


def test_per_token_max_rows():
    G, R, K = 2, (2**31 - 1) // MAX_K, MAX_K
    announce(f"cast per token max G={G} R={R} K={K} bf16")
    rng = np.random.default_rng(39)
    live = sorted({(0, 0), (0, R - 1), (1, 0), (1, R - 1), (1, 65543)} |
                  {(int(rng.integers(G)), int(rng.integers(R))) for _ in range(6)})
    x = torch.zeros((G, R, K), dtype=torch.bfloat16, device="cuda")
    tg = torch.Generator(device="cuda")
    tg.manual_seed(39)
    for g, r in live:
        x[g, r] = (3 * torch.randn(K, generator=tg, device="cuda")).to(torch.bfloat16)
    codes, sf = dg.per_token_cast_to_fp8(x)
    torch.cuda.synchronize()
    for g, r in live:
        ref = oracle.cast_rows(x[g, r][None].float().cpu().numpy())
        got = (codes[g, r][None].cpu().numpy(), sf[g, :, r][:, None].cpu().numpy())
        assert_same(got, ref, f"row {(g, r)}")
        codes[g, r] = 0
        sf[g, :, r] = 1.0
    assert int(torch.count_nonzero(codes)) == 0
    assert bool((sf == 1.0).all())


def test_per_block_max_rows():
    N, K = (2**31 - 1) // MAX_K, MAX_K               # 131071 rows: ragged last block
    NB, KB = (N + 127) // 128, K // 128
    announce(f"cast per block max N={N} K={K} bf16")
    rng = np.random.default_rng(40)
    live = sorted({(0, 0), (NB - 1, KB - 1), (NB - 1, 0)} |
                  {(int(rng.integers(NB)), int(rng.integers(KB))) for _ in range(5)})
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    tg = torch.Generator(device="cuda")
    tg.manual_seed(40)

    def blk(nb, kb):
        return slice(nb * 128, min(N, nb * 128 + 128)), slice(kb * 128, kb * 128 + 128)

    for nb, kb in live:
        rows, cols = blk(nb, kb)
        shape = (rows.stop - rows.start, 128)
        w[rows, cols] = (3 * torch.randn(shape, generator=tg, device="cuda")).to(torch.bfloat16)
    codes, sf = dg.per_block_cast_to_fp8(w)
    torch.cuda.synchronize()
    for nb, kb in live:
        rows, cols = blk(nb, kb)
        ref = oracle.cast_blocks(w[rows, cols].float().cpu().numpy())
        got = (codes[rows, cols].cpu().numpy(), sf[nb:nb + 1, kb:kb + 1].cpu().numpy())
        assert_same(got, ref, f"block {(nb, kb)}")
        codes[rows, cols] = 0
        sf[nb, kb] = 1.0
    assert int(torch.count_nonzero(codes)) == 0
    assert bool((sf == 1.0).all())
