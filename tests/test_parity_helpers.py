"""The whole-output comparator used by the GPU parity tests, on the CPU:
it accepts bf16-level rounding, and rejects one bad element, a slightly
rotated output, a non-finite value and a count that does not cover every
valid entry."""
import numpy as np
import pytest

from tests.parity import COS_TOL, FullCheck, check_full_rows


def _ref(shape=(300, 96), seed=0):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(shape) * 40.0
    r[::7, 3] = np.nan              # entries without a reference are skipped
    return r


def _bf16(x):
    """Round-to-nearest-even to bf16, returned as float64."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_bf16_rounding_passes_streamed_over_chunks():
    ref = _ref()
    got = _bf16(np.nan_to_num(ref))
    st = check_full_rows("bf16", got, lambda rows: ref[rows], ref.shape[0], chunk=64,
                         expect_n=int(np.sum(~np.isnan(ref))))
    assert st["one_minus_cos"] < 1e-5


def test_one_bad_element_fails():
    ref = _ref()
    got = np.nan_to_num(ref).copy()
    got[123, 45] += 0.5 * np.sqrt(np.nanmean(ref * ref))     # 0.5 rms: past 1e-2 rel + 1e-2 rms
    with pytest.raises(AssertionError, match="per-entry"):
        check_full_rows("bad element", got, lambda rows: ref[rows], ref.shape[0], chunk=50)


def test_small_rotation_fails_on_cosine():
    ref = _ref()
    rng = np.random.default_rng(1)
    noise = rng.standard_normal(ref.shape) * np.sqrt(np.nanmean(ref * ref))
    got = np.nan_to_num(ref) + 0.006 * noise        # per entry inside the bound, 1-cos ~ 1.8e-5
    fc = FullCheck("rotation")
    fc.add(got, ref)
    with pytest.raises(AssertionError, match="1-cos"):
        fc.finish()
    assert COS_TOL == 1e-5


def test_non_finite_and_incomplete_coverage_fail():
    ref = _ref()
    got = np.nan_to_num(ref).copy()
    got[0, 0] = np.inf
    with pytest.raises(AssertionError, match="non-finite"):
        check_full_rows("inf", got, lambda rows: ref[rows], ref.shape[0])
    got[0, 0] = ref[0, 0]
    with pytest.raises(AssertionError, match="compared"):
        check_full_rows("count", got, lambda rows: ref[rows], ref.shape[0] - 1,
                        expect_n=int(np.sum(~np.isnan(ref))))
