"""Pins of the oracle's FP8 casting (the step before the GEMM) against things
other than itself.

The reading being pinned (the pages leave casting to the caller, "DeepGEMM"
README, "Interfaces", "Notices", and give no formula): per block (1 x 128 for
activations, 128 x 128 for weights) scale = amax / 448 in fp32 (1 when amax is
0; with pow2, rounded up to a power of two), code = the e4m3 value nearest to
clamp(x / scale) with the quotient in fp32, ties to the even mantissa, sign
kept on zero.

* The encoder against torch's float8_e4m3fn cast (an independent RNE
  implementation), against every code's own value, and at every midpoint.
* The casts against brute-force nearest-code search over all 127 magnitudes,
  against the error bound of a 3-bit mantissa, against the input generator's
  torch-based quantisers, and against a hand-worked example.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAGS = None


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def magnitudes():
    """Values of the non-negative finite codes 0x00 .. 0x7E, decoded by torch."""
    global MAGS
    if MAGS is None:
        MAGS = torch_decode(np.arange(0x7F, dtype=np.uint8))
    return MAGS


def brute_nearest(q):
    """Nearest code to each fp32 value (|q| <= 448) by exhaustive search, ties
    to the even code (the code's low bit is the mantissa's low bit)."""
    mags = magnitudes()
    out = np.empty(q.shape, np.uint8)
    flat, res = q.reshape(-1).astype(np.float64), out.reshape(-1)
    for i, v in enumerate(flat):
        d = np.abs(mags - abs(v))
        best = np.nonzero(d == d.min())[0]
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        res[i] = code | (0x80 if np.signbit(v) else 0)
    return out


def rand_activations(rng, shape):
    """Normal values with per-row magnitude spread and a few exact zeros."""
    x = rng.normal(size=shape) * np.exp(rng.normal(0, 3, size=shape[:-1] + (1,)))
    x[..., 5] = 0.0
    return x.astype(np.float32)


# --------------------------------------------------------------------------
# encoder
# --------------------------------------------------------------------------

def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(torch_decode(codes)), codes)


def test_encode_midpoints_tie_to_even_and_neighbours_round_to_nearest():
    mags = magnitudes()
    lo = np.arange(0x7E)
    mid = (mags[lo] + mags[lo + 1]) / 2          # exact in fp64
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(oracle.e4m3_encode(mid), even)
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)
    eps = (mags[lo + 1] - mags[lo]) * 1e-6
    assert np.array_equal(oracle.e4m3_encode(mid - eps), lo)
    assert np.array_equal(oracle.e4m3_encode(mid + eps), lo + 1)


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(40)
    v = np.concatenate([rng.uniform(-448, 448, 20000),
                        np.exp(rng.uniform(np.log(2.0 ** -13), np.log(448.0), 20000))
                        * rng.choice([-1, 1], 20000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), ref)


def test_encode_saturates():
    got = oracle.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e30, -500.0, -448.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


# --------------------------------------------------------------------------
# 1 x 128 activation casting
# --------------------------------------------------------------------------

def test_cast_rows_hand_worked_golden():
    with open(os.path.join(GOLDEN, "hand_worked_cast.json")) as f:
        g = json.load(f)
    x = np.zeros((1, 128), np.float32)
    n = len(g["x_first"])
    x[0, :n] = g["x_first"]
    codes, sf = oracle.cast_rows(x)
    assert codes[0, :n].tolist() == g["codes_first"]
    assert not codes[0, n:].any()
    assert sf.shape == (1, 1) and sf[0, 0] == g["scale"]


def quotient_ties(s, count):
    """fp32 values x whose fp32 quotient x / s lands exactly on a midpoint
    between two codes, while x times the fp32 reciprocal of s does not: they
    tell a correctly rounded division from a multiply by 1/s."""
    s = np.float32(s)
    inv = np.float32(1) / s
    mags = magnitudes()
    found = []
    for lo in range(0x10, 0x7D):
        mid = np.float32((mags[lo] + mags[lo + 1]) / 2)
        bits = np.array([mid * s], np.float32).view(np.int32)[0]
        for k in (0, 1, -1, 2, -2, 3, -3):            # neighbouring fp32 values
            x = np.array([bits + k], np.int32).view(np.float32)[0]
            if np.float32(x / s) == mid and np.float32(x * inv) != mid:
                found.append(x)
                break
        if len(found) == count:
            break
    return np.array(found, np.float32)


def test_cast_rows_is_the_nearest_code_of_the_fp32_quotient():
    rng = np.random.default_rng(41)
    x = rand_activations(rng, (6, 256))
    # row 0, block 0: amax 3 (scale 3/448, not a power of two) and quotient ties
    ties = quotient_ties(np.float32(3.0) / np.float32(448.0), 40)
    assert len(ties) >= 10
    x[0, :128] = np.clip(x[0, :128], -2.9, 2.9)
    x[0, 0] = 3.0
    x[0, 1:1 + len(ties)] = ties
    codes, sf = oracle.cast_rows(x)
    s = np.repeat(sf.T, 128, axis=1)                       # [R, K]
    q = np.clip(x / s, -448, 448)                          # numpy fp32 division
    assert q.dtype == np.float32
    assert np.array_equal(codes, brute_nearest(q))


def test_cast_rows_scale_layout_and_block_max():
    """Each (row, block) gets its own amax at a random position: the scale sits
    at sf[kb, r] and the largest element becomes +-448."""
    rng = np.random.default_rng(42)
    R, KB = 5, 3
    x = rng.uniform(-1, 1, (R, KB * 128)).astype(np.float32)
    peak = np.zeros((R, KB), np.float32)
    for r in range(R):
        for kb in range(KB):
            p = np.float32(2.0 + 3 * r + 17 * kb + rng.uniform(0, 1))
            pos = kb * 128 + rng.integers(0, 128)
            x[r, pos] = p if (r + kb) % 2 else -p
            peak[r, kb] = p
    codes, sf = oracle.cast_rows(x)
    assert sf.shape == (KB, R)
    assert np.array_equal(sf, (peak / np.float32(448)).T)
    for r in range(R):
        for kb in range(KB):
            blk = np.abs(x[r, kb * 128:(kb + 1) * 128])
            c = codes[r, kb * 128 + int(np.argmax(blk))]
            assert c & 0x7F == 0x7E


def test_cast_rows_dequantisation_error_bound():
    """A 3-bit mantissa: |dec(q) s - x| <= (2^-4 + 2^-23) |x| + 2^-10 s."""
    rng = np.random.default_rng(43)
    x = rand_activations(rng, (16, 512))
    codes, sf = oracle.cast_rows(x)
    s = np.repeat(sf.T, 128, axis=1).astype(np.float64)
    err = np.abs(torch_decode(codes) * s - x)
    assert np.all(err <= (2.0 ** -4 + 2.0 ** -23) * np.abs(x) + 2.0 ** -10 * s)


def test_cast_rows_zero_block():
    x = np.zeros((3, 256), np.float32)
    x[1, 130] = 2.0
    codes, sf = oracle.cast_rows(x)
    assert sf[0].tolist() == [1.0, 1.0, 1.0]
    assert sf[1].tolist() == [1.0, np.float32(2.0) / np.float32(448.0), 1.0]
    assert codes[1, 130] == 0x7E and np.count_nonzero(codes) == 1


def test_cast_rows_matches_generator_quantiser():
    rng = np.random.default_rng(44)
    x = rand_activations(rng, (33, 640))
    codes, sf = oracle.cast_rows(x)
    gc, gs = gen.quantize_rows(x)
    assert np.array_equal(codes, gc) and np.array_equal(sf, gs)


def test_cast_rows_batched_is_per_group():
    rng = np.random.default_rng(45)
    x = rand_activations(rng, (3, 7, 256))
    codes, sf = oracle.cast_rows(x)
    assert sf.shape == (3, 2, 7)
    for g in range(3):
        c1, s1 = oracle.cast_rows(x[g])
        assert np.array_equal(codes[g], c1) and np.array_equal(sf[g], s1)


def test_cast_rows_pow2_scales():
    rng = np.random.default_rng(46)
    x = rand_activations(rng, (9, 384))
    x[2, :128] = 0.0
    codes, sf = oracle.cast_rows(x, pow2=True)
    amax = np.abs(x).reshape(9, 3, 128).max(axis=2).T       # [KB, R]
    m, _ = np.frexp(sf)
    assert np.all(m == 0.5)                                 # powers of two
    nz = amax > 0
    exact = amax[nz].astype(np.float64) / 448
    assert np.all(sf[nz] >= np.float32(amax[nz] / np.float32(448)))
    assert np.all(sf[nz] < 2 * exact)
    assert sf[0, 2] == 1.0
    s = np.repeat(sf.T, 128, axis=1)
    q = np.clip(x / s, -448, 448)
    assert np.array_equal(codes, brute_nearest(q))
    top = np.abs(torch_decode(codes)).reshape(9, 3, 128).max(axis=2).T
    assert np.all((top[nz] > 224) & (top[nz] <= 448))


# --------------------------------------------------------------------------
# 128 x 128 weight casting
# --------------------------------------------------------------------------

def test_cast_blocks_matches_generator_quantiser_with_ragged_n():
    rng = np.random.default_rng(47)
    w = rand_activations(rng, (300, 384))
    codes, sf = oracle.cast_blocks(w)
    gc, gs = gen.quantize_blocks(w)
    assert sf.shape == (3, 3)
    assert np.array_equal(codes, gc) and np.array_equal(sf, gs)


def test_cast_blocks_is_the_nearest_code_of_the_fp32_quotient():
    rng = np.random.default_rng(48)
    w = rand_activations(rng, (2, 140, 256))
    codes, sf = oracle.cast_blocks(w, pow2=True)
    assert sf.shape == (2, 2, 2)
    s = np.repeat(np.repeat(sf, 128, axis=1)[:, :140], 128, axis=2)
    q = np.clip(w / s, -448, 448)
    assert np.array_equal(codes, brute_nearest(q))
    amax = np.abs(np.pad(w, ((0, 0), (0, 116), (0, 0)))).reshape(2, 2, 128, 2, 128).max(axis=(2, 4))
    assert np.all(sf >= amax / np.float32(448)) and np.all(sf < 2 * amax.astype(np.float64) / 448)
