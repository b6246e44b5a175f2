"""Helpers shared by the GPU parity tests: device upload, the tolerance check
and guard-banded output buffers.

Tolerance (the stated acceptance bar of these workloads), over the outputs
that have a reference value:
    1 - cos(D_gpu, D_ref) < 1e-5                                (overall)
    |D_gpu - D_ref| <= 1e-2 * |D_ref| + 1e-2 * rms(D_ref)       (per element)
Why it holds with margin: the oracle is exact up to fp64 rounding; the GPU
keeps fp32 accumulators (relative error ~1e-7 per promotion step) and rounds
once to bf16 (relative error <= 2^-9 per element, RMS about 1.1e-3), so
1 - cos is about 1e-6 and the per-element error is far inside 1e-2 * |ref|.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

COS_TOL = 1e-5
REL_TOL = 1e-2
RMS_TOL = 1e-2

SENTINEL_BF16 = 0xFFFF          # a bf16 NaN pattern the kernels never produce
SENTINEL_F32 = 0x7FC0DEAD       # an fp32 NaN pattern


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """Apply the tolerance to the entries whose reference is not NaN."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    mask = ~np.isnan(ref)
    g, r = got[mask], ref[mask]
    assert g.size > 0, f"{what}: nothing to compare"
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    denom = np.sqrt(np.sum(g * g) * np.sum(r * r))
    cos = float(np.sum(g * r) / denom) if denom > 0 else (1.0 if np.all(g == r) else 0.0)
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    bound = REL_TOL * np.abs(r) + RMS_TOL * rms
    worst = int(np.argmax(err - bound))
    stats = dict(one_minus_cos=1.0 - cos, max_abs=float(err.max()),
                 max_rel=float(np.max(err / np.maximum(np.abs(r), 1e-30 + rms))),
                 n=int(g.size))
    assert 1.0 - cos < COS_TOL, f"{what}: 1-cos = {1 - cos:.3e} {stats}"
    assert np.all(err <= bound), (f"{what}: element {worst} |err|={err[worst]:.4e} > "
                                  f"bound {bound[worst]:.4e} (ref {r[worst]:.4e}) {stats}")
    return stats


class Guarded:
    """A device buffer of `shape` surrounded by sentinel-filled guard bands.

    `view` is the output the kernel writes; `intact()` checks the guards (and,
    for rows that must stay untouched, callers check `view` directly)."""

    GUARD = 4096   # elements on each side

    def __init__(self, shape, dtype: torch.dtype, fill_bits: int | None = None):
        self.shape = tuple(shape)
        self.dtype = dtype
        n = int(np.prod(self.shape))
        itype = torch.int16 if dtype == torch.bfloat16 else torch.int32
        bits = fill_bits if fill_bits is not None else (
            SENTINEL_BF16 if dtype == torch.bfloat16 else SENTINEL_F32)
        if itype == torch.int16 and bits >= 0x8000:
            bits -= 0x10000
        self.bits = bits
        self.raw = torch.full((n + 2 * self.GUARD,), bits, dtype=itype, device="cuda")
        self.view = self.raw[self.GUARD:self.GUARD + n].view(dtype).view(self.shape)

    def intact(self) -> bool:
        head = self.raw[:self.GUARD]
        tail = self.raw[-self.GUARD:]
        return bool(torch.all(head == self.bits).item() and torch.all(tail == self.bits).item())

    def untouched(self, index) -> bool:
        itype = torch.int16 if self.dtype == torch.bfloat16 else torch.int32
        return bool(torch.all(self.view.view(itype)[index] == self.bits).item())


class FullCheck:
    """The tolerance applied to a whole output, streamed over row chunks so a
    large output never needs one fp64 array.

    add(got, ref) takes the GPU values and the oracle's for some rows (NaN in
    ref marks entries without a reference); finish() applies
        1 - cos(D_gpu, D_ref) < COS_TOL                  over every valid entry
        |D_gpu - D_ref| <= REL_TOL * |D_ref| + RMS_TOL * rms(D_ref)   per entry
    with rms over every valid entry (the per-entry check keeps, per chunk,
    the largest |err| - REL_TOL * |ref|, compared once rms is known)."""

    def __init__(self, what: str):
        self.what = what
        self.sgr = self.sgg = self.srr = 0.0
        self.n = 0
        self.excess = -np.inf      # max over entries of |err| - REL_TOL * |ref|
        self.excess_at = None
        self.max_abs = 0.0
        self.max_rel_num = 0.0

    def add(self, got: np.ndarray, ref: np.ndarray, label=None) -> None:
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        mask = ~np.isnan(ref)
        g, r = got[mask], ref[mask]
        if g.size == 0:
            return
        assert np.all(np.isfinite(g)), f"{self.what}: non-finite GPU output ({label})"
        self.sgr += float(np.dot(g, r))
        self.sgg += float(np.dot(g, g))
        self.srr += float(np.dot(r, r))
        self.n += int(g.size)
        err = np.abs(g - r)
        ex = err - REL_TOL * np.abs(r)
        i = int(np.argmax(ex))
        if ex[i] > self.excess:
            self.excess = float(ex[i])
            self.excess_at = (label, float(err[i]), float(r[i]))
        self.max_abs = max(self.max_abs, float(err.max()))

    def finish(self, expect_n: int | None = None) -> dict:
        assert self.n > 0, f"{self.what}: nothing compared"
        if expect_n is not None:
            assert self.n == expect_n, f"{self.what}: compared {self.n} of {expect_n} entries"
        denom = np.sqrt(self.sgg * self.srr)
        cos = self.sgr / denom if denom > 0 else (1.0 if self.sgg == self.srr == 0 else 0.0)
        rms = float(np.sqrt(self.srr / self.n))
        stats = dict(what=self.what, n=self.n, one_minus_cos=float(1.0 - cos), max_abs=self.max_abs,
                     rms_ref=rms, worst_excess_over_rms=float(self.excess / rms) if rms > 0 else 0.0)
        print(f"[full-output] {stats}", flush=True)
        assert 1.0 - cos < COS_TOL, f"{self.what}: 1-cos = {1 - cos:.3e} {stats}"
        assert self.excess <= RMS_TOL * rms, (
            f"{self.what}: per-entry bound broken at {self.excess_at} (rms {rms:.4e}) {stats}")
        return stats


def check_full_rows(what: str, got_host: np.ndarray, ref_fn, n_rows: int, chunk: int = 256,
                    expect_n: int | None = None) -> dict:
    """FullCheck over rows [0, n_rows) of got_host (host array, first axis =
    rows), the oracle's rows coming from ref_fn(row_indices)."""
    fc = FullCheck(what)
    for r0 in range(0, n_rows, chunk):
        rows = np.arange(r0, min(n_rows, r0 + chunk), dtype=np.int64)
        fc.add(got_host[r0:r0 + len(rows)], ref_fn(rows), label=f"rows {r0}..")
    return fc.finish(expect_n)
