"""GPU parity of the FP8 MQA logits kernel (the indexer kernel, non-paged)
against the CPU oracle (oracle.mqa_logits), through the C ABI.

Definition ("DeepGEMM" README, "Interfaces", "V3.2 MQA kernels for the
indexer"): logits[i, j] = sum_h relu(q[i, h] . kv[j] * sf[j]) * weights[i, h]
for j in [ks[i], ke[i]), -inf elsewhere when cleaning.

* Tolerance parity (1 - cos < 1e-5, |err| <= 1e-2 |ref| + 1e-2 rms(ref)) over
  the in-range entries, for 16, 32 and 64 heads, ragged S and S_kv, causal
  packed sequences with and without a shared kv prefix, arbitrary ranges
  (clamped, empty, reversed).
* Out-of-range entries: exactly -inf with cleaning; untouched (sentinel
  bytes) without it.
* Closed forms, bit-exact: all q negative against positive kv gives 0; one
  head with weight 0.5 and all-ones operands gives 64 sf[j].
* The 4096 x 4096 x 64-head causal prefill shape over every output entry.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_e4m3_amd as dg
import oracle
from tests import gen
from tests.parity import FullCheck, announce, check_close, dev

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0DEAD


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield


def run(x, clean=True):
    out = torch.full((x.S, x.S_kv), SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
    dg.fp8_mqa_logits(dev(x.q), (dev(x.kv), dev(x.kv_sf)), dev(x.weights), dev(x.ks), dev(x.ke),
                      clean_logits=clean, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare(got, ref, clean, what, raw=None):
    inside = np.isfinite(ref) if clean else ~np.isnan(ref)
    if inside.any():
        check_close(got[inside].astype(np.float64), ref[inside], what)
    if clean:
        assert np.all(np.isneginf(got[~inside])), f"{what}: out-of-range entries not -inf"
    else:
        assert np.all(raw[~inside] == SENTINEL), f"{what}: out-of-range entries written"


@pytest.mark.parametrize("H", [16, 32, 64])
@pytest.mark.parametrize("S,S_kv,lens", [
    (128, 256, None), (37, 300, None), (200, 200, [70, 130]), (64, 1000, [30, 34]), (1, 5, None),
])
def test_mqa_parity(H, S, S_kv, lens):
    announce(f"mqa H={H} S={S} S_kv={S_kv} lens={lens}")
    x = gen.gen_mqa(S, S_kv, H=H, seed=S + S_kv + H, seq_lens=lens)
    ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, x.ks, x.ke, clean=True)
    compare(run(x, True), ref, True, f"H={H} {S}x{S_kv}")


def test_mqa_without_cleaning_leaves_the_rest_untouched():
    announce("mqa clean=False")
    x = gen.gen_mqa(70, 520, H=64, seed=3, seq_lens=[40, 30])
    got = run(x, False)
    raw = got.view(np.int32)
    ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, x.ks, x.ke, clean=False)
    compare(got, ref, False, "unclean", raw=raw)


def test_mqa_arbitrary_ranges():
    announce("mqa arbitrary ranges")
    x = gen.gen_mqa(40, 700, H=32, seed=4)
    rng = np.random.default_rng(4)
    x.ks = rng.integers(-50, 700, size=40).astype(np.int32)
    x.ke = (x.ks + rng.integers(-20, 400, size=40)).astype(np.int32)
    x.ke[3] = 10_000; x.ks[5] = 800; x.ke[7] = x.ks[7]        # clamped, empty, empty
    ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, x.ks, x.ke, clean=True)
    compare(run(x, True), ref, True, "arbitrary ranges")


def test_mqa_closed_forms_bit_exact():
    announce("mqa closed forms")
    S, S_kv, H = 20, 300, 64
    x = gen.gen_mqa(S, S_kv, H=H, seed=5)
    x.q[:] = 0xB8                            # -1
    x.kv[:] = 0x38                           # +1
    x.ks[:] = 0; x.ke[:] = S_kv
    assert np.all(run(x, True) == 0.0)       # every head negative: relu -> 0
    x.q[:, 7, :] = 0x38                      # head 7: dot = 128
    x.weights[:] = 0.0
    x.weights[:, 7] = 0.5
    want = (64.0 * x.kv_sf.astype(np.float64)).astype(np.float32)
    assert np.array_equal(run(x, True), np.broadcast_to(want, (S, S_kv)))


def test_mqa_prefill_4096_full_output():
    """4096 queries x 4096 kv tokens, 64 heads, one causal sequence: every
    in-range logit against the oracle (streamed over query chunks), every
    other entry -inf."""
    announce("mqa 4096x4096 H=64 causal full output")
    x = gen.gen_mqa(4096, 4096, H=64, seed=0)
    got = run(x, True)
    fc = FullCheck("prefill 4096")
    for r0 in range(0, x.S, 512):
        rows = np.arange(r0, min(x.S, r0 + 512), dtype=np.int64)
        ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, x.ks, x.ke, clean=True, rows=rows)
        inside = np.isfinite(ref)
        assert np.all(np.isneginf(got[rows][~inside])), "out-of-range entries not -inf"
        fc.add(got[rows], np.where(inside, ref, np.nan), label=f"queries {r0}..")
    pairs = int((np.clip(x.ke, 0, x.S_kv) - np.clip(x.ks, 0, x.S_kv)).clip(0).sum())
    fc.finish(expect_n=pairs)


def test_mqa_graph_capture_replays_with_new_ranges():
    """MQA logits captured into a HIP graph: the ranges live in device memory,
    so each replay sees the values written before it."""
    announce("mqa graph capture")
    x = gen.gen_mqa(96, 700, H=64, seed=8)
    q, kv, sf, w = dev(x.q), dev(x.kv), dev(x.kv_sf), dev(x.weights)
    ks, ke = dev(x.ks), dev(x.ke)
    out = torch.empty(x.S, x.S_kv, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.fp8_mqa_logits(q, (kv, sf), w, ks, ke, True, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.fp8_mqa_logits(q, (kv, sf), w, ks, ke, True, out=out)
    rng = np.random.default_rng(8)
    for rep in range(3):
        lo = rng.integers(0, 700, size=96).astype(np.int32)
        hi = (lo + rng.integers(0, 300, size=96)).astype(np.int32)
        ks.copy_(torch.from_numpy(lo)); ke.copy_(torch.from_numpy(hi))
        out.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, lo, hi, clean=True)
        compare(out.cpu().numpy(), ref, True, f"replay {rep}")


def test_max_queries():
    """The largest seq_len the entry point accepts (65535 workgroup rows of 16
    queries), 64 heads: q is 8 GiB, so its offsets pass 2^32.  q is zero
    except a few queries (the first, the last, random ones), checked against
    the oracle; every other row must be exactly 0 inside its range and -inf
    outside."""
    S, S_kv, H = 65535 * 16, 2048, 64
    announce(f"mqa max queries S={S} S_kv={S_kv} H={H}")
    rng = np.random.default_rng(36)
    live = np.unique(np.concatenate([np.arange(4), np.arange(S - 4, S),
                                     rng.choice(S, size=8, replace=False)])).astype(np.int64)
    x = gen.gen_mqa_sparse(S, S_kv, H, live, seed=36)
    out = torch.empty((S, S_kv), dtype=torch.float32, device="cuda")
    ks_t, ke_t = dev(x.ks), dev(x.ke)
    dg.fp8_mqa_logits(dev(x.q), (dev(x.kv), dev(x.kv_sf)), dev(x.weights), ks_t, ke_t,
                      clean_logits=True, out=out)
    torch.cuda.synchronize()
    live_t = torch.from_numpy(live).cuda()
    ref = oracle.mqa_logits(x.q, x.kv, x.kv_sf, x.weights, x.ks, x.ke, rows=live)
    compare(out[live_t].cpu().numpy(), ref, True, "mqa max queries")
    dead = torch.ones(S, dtype=torch.bool, device="cuda")
    dead[live_t] = False
    j = torch.arange(S_kv, device="cuda")
    for r0 in range(0, S, 1 << 16):
        rr = slice(r0, min(S, r0 + (1 << 16)))
        inside = (j[None] >= ks_t[rr, None].long()) & (j[None] < ke_t[rr, None].long())
        expect = torch.where(inside, 0.0, float("-inf"))
        assert bool(((out[rr] == expect) | ~dead[rr, None]).all()), f"rows {r0}.."
