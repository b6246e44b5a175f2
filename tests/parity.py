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
