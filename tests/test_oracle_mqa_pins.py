"""Pins of the oracle's MQA logits (the "DeepGEMM" README, "Interfaces",
"V3.2 MQA kernels for the indexer": out[i, j] = sum_h relu(q[i, h] . kv_j) *
weights[i, h] with kv_j = kv[j] * sf[j], for j in [ks[i], ke[i]), -inf
elsewhere when cleaning) against things other than the function itself.

* Exact rational arithmetic on tiny shapes (torch-decoded operands).
* A float64 numpy route through the formula (einsum of decoded values, relu,
  weights) on a mid-size case.
* Closed forms: all q rows negative against positive kv give 0; a one-hot
  weight picks one head; doubling sf doubles the logits.
* Ranges: -inf (clean) or NaN outside, clamping of out-of-range bounds,
  empty ranges, the causal generator.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import gen
from tests.test_oracle_pins import random_codes, torch_decode


def small(rng, S, S_kv, H, D=128):
    q = random_codes(rng, (S, H, D))
    kv = random_codes(rng, (S_kv, D))
    sf = np.exp(rng.normal(0, 1, S_kv)).astype(np.float32)
    w = rng.normal(0, 1, (S, H)).astype(np.float32)
    return q, kv, sf, w


def exact(q, kv, sf, w, ks, ke):
    S, H, D = q.shape
    S_kv = kv.shape[0]
    dq, dk = torch_decode(q), torch_decode(kv)
    out = np.full((S, S_kv), -np.inf)
    bound = np.zeros((S, S_kv))
    for i in range(S):
        for j in range(max(ks[i], 0), min(ke[i], S_kv)):
            tot = Fraction(0); mag = Fraction(0)
            for h in range(H):
                dot = sum(Fraction(float(dq[i, h, d])) * Fraction(float(dk[j, d])) for d in range(D))
                s = dot * Fraction(float(sf[j]))
                term = max(s, Fraction(0)) * Fraction(float(w[i, h]))
                tot += term; mag += abs(term)
            out[i, j] = float(tot)
            bound[i, j] = float(mag) * (3 * H + 2) * 2.0 ** -53 + 1e-300
    return out, bound


def test_matches_exact_rationals():
    rng = np.random.default_rng(90)
    S, S_kv, H = 3, 5, 4
    q, kv, sf, w = small(rng, S, S_kv, H)
    ks = np.array([0, 1, 3], np.int32); ke = np.array([5, 3, 4], np.int32)
    got = oracle.mqa_logits(q, kv, sf, w, ks, ke)
    want, bound = exact(q, kv, sf, w, ks, ke)
    inside = np.isfinite(want)
    assert np.all(np.abs(got[inside] - want[inside]) <= bound[inside])
    assert np.all(np.isneginf(got[~inside]))


def test_matches_float64_numpy_formula():
    rng = np.random.default_rng(91)
    S, S_kv, H = 17, 40, 16
    q, kv, sf, w = small(rng, S, S_kv, H)
    ks, ke = gen.causal_ranges([9, 8], S_kv)
    dq, dk = torch_decode(q), torch_decode(kv)
    logits = np.einsum("ihd,jd->ijh", dq, dk) * sf.astype(np.float64)[None, :, None]
    want = (np.maximum(logits, 0) * w.astype(np.float64)[:, None, :]).sum(-1)
    j = np.arange(S_kv)[None, :]
    want = np.where((j >= ks[:, None]) & (j < ke[:, None]), want, -np.inf)
    got = oracle.mqa_logits(q, kv, sf, w, ks, ke)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=1e-9)


def test_relu_zeroes_negative_logits_and_one_hot_weights():
    rng = np.random.default_rng(92)
    S, S_kv, H, D = 2, 6, 4, 128
    q = np.full((S, H, D), 0xB8, np.uint8)            # -1.0
    kv = np.full((S_kv, D), 0x38, np.uint8)           # +1.0
    sf = np.ones(S_kv, np.float32); w = rng.normal(0, 1, (S, H)).astype(np.float32)
    ks = np.zeros(S, np.int32); ke = np.full(S, S_kv, np.int32)
    assert np.all(oracle.mqa_logits(q, kv, sf, w, ks, ke) == 0.0)
    q[:, 2, :] = 0x38                                  # head 2 positive: dot = 128
    w1 = np.zeros((S, H), np.float32); w1[:, 2] = 0.5
    assert np.all(oracle.mqa_logits(q, kv, sf, w1, ks, ke) == 64.0)
    sf2 = (2 * sf).astype(np.float32)
    assert np.all(oracle.mqa_logits(q, kv, sf2, w1, ks, ke) == 128.0)


def test_ranges_clean_and_unclean_clamped_and_empty():
    rng = np.random.default_rng(93)
    S, S_kv, H = 4, 7, 2
    q, kv, sf, w = small(rng, S, S_kv, H)
    ks = np.array([-3, 2, 5, 6], np.int32); ke = np.array([2, 99, 5, 3], np.int32)
    clean = oracle.mqa_logits(q, kv, sf, w, ks, ke, clean=True)
    raw = oracle.mqa_logits(q, kv, sf, w, ks, ke, clean=False)
    j = np.arange(S_kv)[None, :]
    lo = np.clip(ks, 0, S_kv)[:, None]; hi = np.clip(ke, 0, S_kv)[:, None]
    inside = (j >= lo) & (j < hi)
    assert np.array_equal(np.isfinite(clean), inside)
    assert np.all(np.isneginf(clean[~inside])) and np.all(np.isnan(raw[~inside]))
    assert np.array_equal(clean[inside], raw[inside])
    assert not inside[2].any() and not inside[3].any()   # empty ranges


def test_rows_selection_and_causal_generator():
    x = gen.gen_mqa(12, 20, H=16, seed=1, seq_lens=[5, 7])
    assert np.array_equal(x.ks, np.zeros(12, np.int32))          # shared prefix of 8
    assert np.array_equal(x.ke, np.arange(12, dtype=np.int32) + 9)
    y = gen.gen_mqa(12, 12, H=16, seed=1, seq_lens=[5, 7])
    assert list(y.ks) == [0] * 5 + [5] * 7 and list(y.ke) == list(range(1, 13))
    full = oracle.mqa_logits(y.q, y.kv, y.kv_sf, y.weights, y.ks, y.ke)
    rows = np.array([0, 6, 11], np.int64)
    part = oracle.mqa_logits(y.q, y.kv, y.kv_sf, y.weights, y.ks, y.ke, rows=rows)
    assert np.array_equal(part, full[rows])
