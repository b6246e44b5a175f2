"""Seeded synthetic inputs for the fine-grained FP8 e4m3 GEMM workloads.

This module is shared by the CPU oracle and the HIP path: both must consume the
same bytes.  It holds input preparation only -- random draws, MoE routing /
masking / K-splitting, and the FP8 casting that the pages leave to the
library's users (DeepGEMM Documentation, section 4 "Understand DeepGEMM GEMM
Naming and Layouts": casting and transposition happen outside the GEMM).  It
holds none of the GEMM arithmetic (no decode, no block product, no promotion).

Quantisation recipe (the pages say only "fine grain scale"; the 1x128 and
128x128 granularities and scale = amax/448 are the workload definitions):
  * activations: one fp32 scale per row per 128-wide K block, stored MN-major
    as SF[K/128, rows] (the pages ask for a transposed, MN-major LHS scale
    layout, DeepGEMM Documentation, section 4);
  * weights: one fp32 scale per 128x128 block, SF[ceil(N/128), K/128];
  * K-grouped operands: one scale per column per 128-row block of the
    [K_total, M] / [K_total, N] matrices, SF[K_total/128, M|N].
  scale = amax / 448 in fp32 (amax == 0 -> scale 1.0), q = e4m3fn(RNE(clamp(x/scale,
  -448, 448))).  torch's float8_e4m3fn cast is RNE but does not saturate, hence
  the clamp.

Every generator takes a seed and uses numpy.random.Generator(PCG64(seed)).
Draw order: routing / mask / K-split first, then A, then B (per expert, in
expert order), then C.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0
BLOCK = 128

# --------------------------------------------------------------------------
# FP8 casting (input preparation)
# --------------------------------------------------------------------------

def _cast_e4m3(y: torch.Tensor) -> torch.Tensor:
    """fp32 -> e4m3fn codes (uint8), RNE, after clamping to +-448."""
    y = torch.clamp(y, -E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _safe_scale(amax: torch.Tensor, pow2: bool = False) -> torch.Tensor:
    scale = amax / torch.tensor(E4M3_MAX, dtype=torch.float32)
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    if pow2:   # round up to a power of two (the UE8M0-representable scales)
        m, e = torch.frexp(scale)
        scale = torch.where(m == 0.5, scale, torch.ldexp(torch.ones_like(scale), e))
    return scale


def quantize_rows(x: np.ndarray | torch.Tensor, pow2: bool = False):
    """Per-row, per-128-K-block quantisation of an activation matrix.

    x: fp32 [R, K] with K % 128 == 0.
    Returns (codes uint8 [R, K], sf fp32 [K/128, R]) as numpy arrays; sf is
    MN-major (row index fastest).
    """
    xt = torch.as_tensor(x, dtype=torch.float32)
    R, K = xt.shape
    assert K % BLOCK == 0
    KB = K // BLOCK
    xb = xt.reshape(R, KB, BLOCK)
    scale = _safe_scale(xb.abs().amax(dim=2), pow2)      # [R, KB]
    codes = _cast_e4m3(xb / scale[:, :, None]).reshape(R, K)
    return codes.numpy(), scale.t().contiguous().numpy()


def quantize_blocks(w: np.ndarray | torch.Tensor, pow2: bool = False):
    """Per-128x128-block quantisation of a weight matrix [N, K].

    Partial blocks (N % 128 != 0) take their amax over the rows that exist.
    Returns (codes uint8 [N, K], sf fp32 [ceil(N/128), K/128]).
    """
    wt = torch.as_tensor(w, dtype=torch.float32)
    N, K = wt.shape
    assert K % BLOCK == 0
    KB = K // BLOCK
    NB = (N + BLOCK - 1) // BLOCK
    pad = NB * BLOCK - N
    wp = torch.nn.functional.pad(wt, (0, 0, 0, pad)) if pad else wt
    blocks = wp.reshape(NB, BLOCK, KB, BLOCK)
    scale = _safe_scale(blocks.abs().amax(dim=(1, 3)), pow2)   # [NB, KB]
    full = scale[:, None, :, None].expand(NB, BLOCK, KB, BLOCK).reshape(NB * BLOCK, K)[:N]
    codes = _cast_e4m3(wt / full)
    return codes.numpy(), scale.contiguous().numpy()


def quantize_cols(x: np.ndarray | torch.Tensor, pow2: bool = False):
    """Per-column, per-128-row-block quantisation of an MN-major operand [Kt, C].

    Used by the K-grouped TN form: A is [K_total, M], B is [K_total, N].
    Returns (codes uint8 [Kt, C], sf fp32 [Kt/128, C]).
    """
    xt = torch.as_tensor(x, dtype=torch.float32)
    Kt, C = xt.shape
    assert Kt % BLOCK == 0
    KB = Kt // BLOCK
    xb = xt.reshape(KB, BLOCK, C)
    scale = _safe_scale(xb.abs().amax(dim=1), pow2)       # [KB, C]
    codes = _cast_e4m3(xb / scale[:, None, :]).reshape(Kt, C)
    return codes.numpy(), scale.contiguous().numpy()


def ue8m0_words(e: np.ndarray) -> np.ndarray:
    """Exponent bytes e [..., KB, MN] -> packed UE8M0 words int32 [..., ceil(KB/4), MN]:
    byte i of word k4 holds block 4 k4 + i (little end first), unused bytes 0."""
    e = np.asarray(e).astype(np.uint32)
    KB = e.shape[-2]
    K4 = (KB + 3) // 4
    w = np.zeros(e.shape[:-2] + (K4, e.shape[-1]), np.uint32)
    for kb in range(KB):
        w[..., kb // 4, :] |= e[..., kb, :] << np.uint32(8 * (kb % 4))
    return w.view(np.int32)


def exponent_bytes(sf: np.ndarray) -> np.ndarray:
    """8-bit exponent fields of fp32 scales (the UE8M0 code of a power of two)."""
    return (np.ascontiguousarray(sf, np.float32).view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)


def pow2_scales(e: np.ndarray) -> np.ndarray:
    """UE8M0 codes -> the fp32 scales 2^(e - 127) (e in [1, 254])."""
    return np.ldexp(np.float32(1), (np.asarray(e, np.int64) - 127).astype(np.int32)).astype(np.float32)


# --------------------------------------------------------------------------
# Workload containers
# --------------------------------------------------------------------------

@dataclasses.dataclass
class DenseInputs:
    a: np.ndarray      # uint8 [M, K]
    sfa: np.ndarray    # fp32 [K/128, M]
    b: np.ndarray      # uint8 [N, K]
    sfb: np.ndarray    # fp32 [ceil(N/128), K/128]
    M: int
    N: int
    K: int
    c: Optional[np.ndarray] = None   # fp32 values of C (bf16-representable), [M, N]


@dataclasses.dataclass
class ContiguousInputs:
    a: np.ndarray          # uint8 [M_tot, K]
    sfa: np.ndarray        # fp32 [K/128, M_tot]
    b: np.ndarray          # uint8 [G, N, K]
    sfb: np.ndarray        # fp32 [G, ceil(N/128), K/128]
    m_indices: np.ndarray  # int32 [M_tot], expert id or -1
    counts: np.ndarray     # int64 [G], valid rows per expert
    M_tot: int
    N: int
    K: int
    G: int


@dataclasses.dataclass
class MaskedInputs:
    a: np.ndarray          # uint8 [G, M_max, K]
    sfa: np.ndarray        # fp32 [G, K/128, M_max]
    b: np.ndarray          # uint8 [G, N, K]
    sfb: np.ndarray        # fp32 [G, ceil(N/128), K/128]
    masked_m: np.ndarray   # int32 [G]
    G: int
    M_max: int
    N: int
    K: int


@dataclasses.dataclass
class KGroupedInputs:
    a: np.ndarray          # uint8 [K_tot, M]
    sfa: np.ndarray        # fp32 [K_tot/128, M]
    b: np.ndarray          # uint8 [K_tot, N]
    sfb: np.ndarray        # fp32 [K_tot/128, N]
    k_sizes: np.ndarray    # int32 [G], multiples of 128
    valid_tokens: np.ndarray  # int64 [G]
    c: Optional[np.ndarray]   # fp32 [G, M, N]
    G: int
    M: int
    N: int
    K_tot: int


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclasses.dataclass
class DenseUe8m0Inputs:
    a: np.ndarray      # uint8 [M, K]
    sfa: np.ndarray    # int32 [ceil(K/512), M], packed UE8M0 words
    b: np.ndarray      # uint8 [N, K]
    sfb: np.ndarray    # int32 [ceil(K/512), N], one exponent per row of B
    sfa_f32: np.ndarray   # the same A scales as fp32 [K/128, M]
    sfb_f32: np.ndarray   # fp32 [ceil(N/128), K/128] (block scales) or None
    M: int
    N: int
    K: int


# --------------------------------------------------------------------------
# Dense NT (workloads 1 and 2)
# --------------------------------------------------------------------------

DENSE_SMALL = (128, 256, 512)
DENSE_SWEEP = [(m, n, k) for m in (64, 128, 4096)
               for (n, k) in ((2112, 7168), (24576, 1536), (7168, 16384),
                              (4096, 7168), (7168, 2048))]


def gen_dense(M: int, N: int, K: int, seed: int = 0, with_c: bool = False) -> DenseInputs:
    """A[M,K], B[N,K] ~ N(0,1) fp32, quantised 1x128 / 128x128.

    with_c adds a bf16-representable C ~ N(0,1) drawn after B (not part of
    the named workloads; used to exercise D = C + A @ B^T)."""
    rng = _rng(seed)
    a32 = _normal(rng, (M, K))
    b32 = _normal(rng, (N, K))
    a, sfa = quantize_rows(a32)
    b, sfb = quantize_blocks(b32)
    c = None
    if with_c:
        c = torch.from_numpy(_normal(rng, (M, N))).to(torch.bfloat16).float().numpy()
    return DenseInputs(a, sfa, b, sfb, M, N, K, c)


def _sparse_rows(a: np.ndarray, sfa: np.ndarray, rows, rng: np.random.Generator,
                 pow2: bool = False) -> None:
    """Fill rows `rows` of a zero [R, K] code matrix (and its [K/128, R] scales)
    with N(0,1) values quantised per row."""
    rows = np.asarray(sorted(set(int(r) for r in rows)), np.int64)
    a[rows], sfa[:, rows] = quantize_rows(_normal(rng, (len(rows), a.shape[1])), pow2)


def gen_dense_sparse(M: int, N: int, K: int, a_rows, b_blocks, seed: int = 0,
                     pow2: bool = False) -> DenseInputs:
    """Dense inputs at sizes where a full random operand would be slow to build
    (an operand of up to 2 GiB): A is zero except the rows a_rows and B zero
    except the 128-row blocks b_blocks, whose values are N(0,1) quantised as in
    gen_dense (scales rounded up to powers of two with pow2); every other
    scale is 1.  Outputs outside the live rows of A or the live blocks of B
    are exactly zero."""
    rng = _rng(seed)
    a = np.zeros((M, K), np.uint8)
    sfa = np.ones((K // BLOCK, M), np.float32)
    _sparse_rows(a, sfa, a_rows, rng, pow2)
    NB = (N + BLOCK - 1) // BLOCK
    b = np.zeros((N, K), np.uint8)
    sfb = np.ones((NB, K // BLOCK), np.float32)
    for blk in sorted(set(int(x) for x in b_blocks)):
        r0, r1 = BLOCK * blk, min(N, BLOCK * blk + BLOCK)
        codes, sf = quantize_blocks(_normal(rng, (r1 - r0, K)), pow2)
        b[r0:r1], sfb[blk] = codes, sf[0]
    return DenseInputs(a, sfa, b, sfb, M, N, K)


def gen_contiguous_sparse(m_indices: np.ndarray, N: int, K: int, G: int, a_rows,
                          seed: int = 0) -> ContiguousInputs:
    """The contiguous M-grouped workload with an A of up to 2 GiB: A is zero
    except the rows a_rows (scale 1 elsewhere); every expert's B is N(0,1)
    quantised per 128x128 block.  m_indices gives the segments (-1 padding)."""
    rng = _rng(seed)
    mi = np.ascontiguousarray(m_indices, np.int32)
    M_tot = len(mi)
    a = np.zeros((M_tot, K), np.uint8)
    sfa = np.ones((K // BLOCK, M_tot), np.float32)
    _sparse_rows(a, sfa, a_rows, rng)
    parts = [quantize_blocks(_normal(rng, (N, K))) for _ in range(G)]
    b = np.stack([q[0] for q in parts])
    sfb = np.stack([q[1] for q in parts])
    counts = np.array([int(np.count_nonzero(mi == e)) for e in range(G)], np.int64)
    return ContiguousInputs(a, sfa, b, sfb, mi, counts, M_tot, N, K, G)


def gen_masked_sparse(G: int, M_max: int, N: int, K: int, masked_m, a_rows,
                      seed: int = 0) -> MaskedInputs:
    """The masked M-grouped workload with an A of up to 2 GiB per group: A[g]
    is zero except the rows a_rows[g] (scale 1 elsewhere); every group's B is
    N(0,1) quantised per 128x128 block."""
    rng = _rng(seed)
    a = np.zeros((G, M_max, K), np.uint8)
    sfa = np.ones((G, K // BLOCK, M_max), np.float32)
    for g in range(G):
        _sparse_rows(a[g], sfa[g], a_rows[g], rng)
    parts = [quantize_blocks(_normal(rng, (N, K))) for _ in range(G)]
    b = np.stack([q[0] for q in parts])
    sfb = np.stack([q[1] for q in parts])
    return MaskedInputs(a, sfa, b, sfb, np.ascontiguousarray(masked_m, np.int32), G, M_max, N, K)


def gen_dense_ue8m0(M: int, N: int, K: int, seed: int = 0) -> DenseUe8m0Inputs:
    """The dense workload with power-of-two scales: A[M,K], B[N,K] ~ N(0,1),
    quantised 1x128 / 128x128 with each scale rounded up to a power of two,
    then packed into UE8M0 words (B's block exponents given to each row)."""
    rng = _rng(seed)
    a32 = _normal(rng, (M, K))
    b32 = _normal(rng, (N, K))
    a, sfa = quantize_rows(a32, pow2=True)
    b, sfb = quantize_blocks(b32, pow2=True)
    eb = np.repeat(exponent_bytes(sfb).T, BLOCK, axis=1)[:, :N]        # [KB, N]
    return DenseUe8m0Inputs(a, ue8m0_words(exponent_bytes(sfa)), b, ue8m0_words(eb),
                            sfa, sfb, M, N, K)


# --------------------------------------------------------------------------
# M-grouped contiguous (workload 3): Zipf(1.1) top-6 routing
# --------------------------------------------------------------------------

def zipf_probs(G: int, s: float = 1.1) -> np.ndarray:
    p = (np.arange(1, G + 1, dtype=np.float64)) ** (-s)
    return p / p.sum()


def route_topk_zipf(rng: np.random.Generator, tokens: int, G: int, topk: int,
                    s: float = 1.1) -> np.ndarray:
    """Per-expert token counts for `tokens` tokens each choosing `topk`
    distinct experts, expert e drawn with weight (e+1)^-s (Gumbel top-k)."""
    logp = np.log(zipf_probs(G, s))
    g = rng.gumbel(size=(tokens, G))
    choice = np.argsort(-(logp[None, :] + g), axis=1)[:, :topk]
    return np.bincount(choice.ravel(), minlength=G).astype(np.int64)


def contiguous_layout(counts: np.ndarray, align: int = BLOCK):
    """Segments in expert order, each padded at its tail to `align` rows.
    Returns (m_indices int32 [M_tot], row offset of each segment)."""
    G = len(counts)
    padded = ((counts + align - 1) // align) * align
    M_tot = int(padded.sum())
    m_idx = np.full(M_tot, -1, dtype=np.int32)
    offs = np.zeros(G + 1, dtype=np.int64)
    offs[1:] = np.cumsum(padded)
    for e in range(G):
        m_idx[offs[e]: offs[e] + counts[e]] = e
    return m_idx, offs


def gen_contiguous(G: int = 32, N: int = 4096, K: int = 4096, tokens: int = 8192,
                   topk: int = 6, seed: int = 0, counts: Optional[np.ndarray] = None,
                   zipf_s: float = 1.1, pow2: bool = False) -> ContiguousInputs:
    """Workload 3 (or a smaller variant).  `counts` overrides the routing;
    pow2 rounds every scale up to a power of two (see to_ue8m0)."""
    rng = _rng(seed)
    if counts is None:
        counts = route_topk_zipf(rng, tokens, G, topk, zipf_s)
    counts = np.asarray(counts, dtype=np.int64)
    m_idx, offs = contiguous_layout(counts)
    M_tot = len(m_idx)
    a32 = np.zeros((M_tot, K), dtype=np.float32)
    valid = _normal(rng, (int(counts.sum()), K))
    r = 0
    for e in range(G):
        c = int(counts[e])
        a32[offs[e]: offs[e] + c] = valid[r: r + c]
        r += c
    del valid
    a, sfa = quantize_rows(a32, pow2)
    del a32
    NB = (N + BLOCK - 1) // BLOCK
    b = np.empty((G, N, K), dtype=np.uint8)
    sfb = np.empty((G, NB, K // BLOCK), dtype=np.float32)
    for e in range(G):
        b[e], sfb[e] = quantize_blocks(_normal(rng, (N, K)), pow2)
    return ContiguousInputs(a, sfa, b, sfb, m_idx, counts, M_tot, N, K, G)


# --------------------------------------------------------------------------
# M-grouped masked (workload 4)
# --------------------------------------------------------------------------

def gen_masked(G: int = 32, M_max: int = 256, N: int = 4096, K: int = 2048,
               seed: int = 0, masked_m: Optional[np.ndarray] = None,
               pow2: bool = False) -> MaskedInputs:
    """masked_m ~ U{0..M_max} per group; A fully drawn (rows past masked_m are
    junk the kernel must never let into D)."""
    rng = _rng(seed)
    if masked_m is None:
        masked_m = rng.integers(0, M_max + 1, G)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    a = np.empty((G, M_max, K), dtype=np.uint8)
    sfa = np.empty((G, K // BLOCK, M_max), dtype=np.float32)
    for g in range(G):
        a[g], sfa[g] = quantize_rows(_normal(rng, (M_max, K)), pow2)
    NB = (N + BLOCK - 1) // BLOCK
    b = np.empty((G, N, K), dtype=np.uint8)
    sfb = np.empty((G, NB, K // BLOCK), dtype=np.float32)
    for g in range(G):
        b[g], sfb[g] = quantize_blocks(_normal(rng, (N, K)), pow2)
    return MaskedInputs(a, sfa, b, sfb, masked_m, G, M_max, N, K)


def to_ue8m0(sfa: np.ndarray, sfb: np.ndarray, N: int):
    """Power-of-two fp32 scales of an NT workload -> packed UE8M0 words:
    sfa [..., KB, rows] -> [..., ceil(KB/4), rows]; sfb [..., ceil(N/128), KB]
    (block scales) -> [..., ceil(KB/4), N], each row of a block taking the
    block's exponent."""
    ea = exponent_bytes(sfa)
    eb = np.repeat(np.swapaxes(exponent_bytes(sfb), -1, -2), BLOCK, axis=-1)[..., :N]
    return ue8m0_words(ea), ue8m0_words(eb)


# --------------------------------------------------------------------------
# K-grouped TN (workload 5)
# --------------------------------------------------------------------------

def gen_k_grouped(G: int = 32, M: int = 2048, N: int = 4096, K_tot: int = 49152,
                  seed: int = 0, k_sizes: Optional[np.ndarray] = None,
                  c_std: float = 0.01, with_c: bool = True,
                  zipf_s: float = 1.1, pow2: bool = False) -> KGroupedInputs:
    """Per-group K = 128 * multinomial(K_tot/128, Zipf(1.1)); inside a group of
    K_g > 0 the first K_g - U{0..127} tokens are N(0,1), the tail is zero (the
    padding).  C ~ N(0, c_std) fp32 [G, M, N]."""
    rng = _rng(seed)
    if k_sizes is None:
        blocks = rng.multinomial(K_tot // BLOCK, zipf_probs(G, zipf_s))
        k_sizes = blocks * BLOCK
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    assert int(k_sizes.sum()) == K_tot and np.all(k_sizes % BLOCK == 0)
    pad = np.where(k_sizes > 0, rng.integers(0, BLOCK, G), 0)
    valid = k_sizes - pad
    a32 = _normal(rng, (K_tot, M))
    b32 = _normal(rng, (K_tot, N))
    off = 0
    for g in range(G):
        a32[off + valid[g]: off + k_sizes[g]] = 0
        b32[off + valid[g]: off + k_sizes[g]] = 0
        off += int(k_sizes[g])
    a, sfa = quantize_cols(a32, pow2)
    del a32
    b, sfb = quantize_cols(b32, pow2)
    del b32
    c = _normal(rng, (G, M, N), c_std) if with_c else None
    return KGroupedInputs(a, sfa, b, sfb, k_sizes.astype(np.int32), valid, c,
                          G, M, N, K_tot)


def gen_k_grouped_sparse(k_sizes, M: int, N: int, live_tokens, seed: int = 0,
                         c_std: float = 0.01) -> KGroupedInputs:
    """The K-grouped workload with operands of up to 2 GiB: A [K_tot, M] and
    B [K_tot, N] are zero except the token rows live_tokens, which are N(0,1)
    quantised per column per 128-token block as in gen_k_grouped (scale 1 in
    blocks without live tokens).  C ~ N(0, c_std) fp32 [G, M, N]."""
    rng = _rng(seed)
    ks = np.asarray(k_sizes, np.int64)
    assert np.all(ks % BLOCK == 0)
    K_tot, G = int(ks.sum()), len(ks)
    a = np.zeros((K_tot, M), np.uint8)
    sfa = np.ones((K_tot // BLOCK, M), np.float32)
    b = np.zeros((K_tot, N), np.uint8)
    sfb = np.ones((K_tot // BLOCK, N), np.float32)
    live = np.asarray(sorted(set(int(t) for t in live_tokens)), np.int64)
    for blk in np.unique(live // BLOCK):
        rows = live[live // BLOCK == blk] - BLOCK * blk
        for codes, sf, cols in ((a, sfa, M), (b, sfb, N)):
            x = np.zeros((BLOCK, cols), np.float32)
            x[rows] = _normal(rng, (len(rows), cols))
            q, s_ = quantize_cols(x)
            codes[BLOCK * blk: BLOCK * blk + BLOCK] = q
            sf[blk] = s_[0]
    c = _normal(rng, (G, M, N), c_std)
    return KGroupedInputs(a, sfa, b, sfb, ks.astype(np.int32), ks.copy(), c, G, M, N, K_tot)


def gen_config(i: int, seed: int = 0):
    """The five named workloads by index 1..5 (2 returns the 15-shape list)."""
    if i == 1:
        return gen_dense(*DENSE_SMALL, seed=seed)
    if i == 2:
        return [gen_dense(m, n, k, seed=seed) for (m, n, k) in DENSE_SWEEP]
    if i == 3:
        return gen_contiguous(seed=seed)
    if i == 4:
        return gen_masked(seed=seed)
    if i == 5:
        return gen_k_grouped(seed=seed)
    raise ValueError(i)


# --------------------------------------------------------------------------
# Unquantised operands for the casting kernels
# --------------------------------------------------------------------------

def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp32 array rounded (RNE) to bf16-representable values, kept as fp32."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def gen_activations(shape, seed: int = 0, bf16: bool = True) -> np.ndarray:
    """Activation-like values: N(0,1) times a per-row magnitude exp(N(0, 1.5)),
    one outlier (x 30) per row, a few exact zeros and negative zeros, and in
    the last row a block of bf16 subnormals (its amax is subnormal).  Returned
    as fp32; with bf16, every value is bf16-representable."""
    rng = _rng(seed)
    x = _normal(rng, shape)
    rows = int(np.prod(shape[:-1]))
    K = shape[-1]
    flat = x.reshape(rows, K)
    flat *= np.exp(rng.normal(0, 1.5, size=(rows, 1))).astype(np.float32)
    out_col = rng.integers(0, K, size=rows)
    flat[np.arange(rows), out_col] *= np.float32(30)
    flat[:, 3] = 0.0
    flat[:, 7] = -0.0
    if K >= 128 and rows > 1:
        flat[-1, :128] = (rng.integers(-120, 121, size=128) * 2.0 ** -133).astype(np.float32)
    return to_bf16_values(x) if bf16 else x


# --------------------------------------------------------------------------
# Other layouts (NN / TN / TT) and the M-grouped contiguous NN form
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LayoutInputs:
    layout: str        # "nn", "tn" or "tt"
    a: np.ndarray      # uint8, stored [M, K] ("n") or [K, M] ("t")
    sfa: np.ndarray    # fp32 [K/128, M]
    b: np.ndarray      # uint8, stored [K, N] ("n") or [N, K] ("t")
    sfb: np.ndarray    # fp32 [K/128, N]
    M: int
    N: int
    K: int
    c: Optional[np.ndarray] = None


def gen_layout(layout: str, M: int, N: int, K: int, seed: int = 0,
               with_c: bool = False) -> LayoutInputs:
    """A(m,k), B(k,n) ~ N(0,1) fp32, each quantised with one scale per output
    row / column per 128-K block (1 x 128 along K), then stored in the
    layout's orientation (a transpose of the codes; the scales are MN-major
    either way)."""
    assert layout in ("nn", "tn", "tt")
    rng = _rng(seed)
    a32 = _normal(rng, (M, K))
    bt32 = _normal(rng, (N, K))          # B^T: row n holds B(:, n)
    a, sfa = quantize_rows(a32)
    bt, sfb = quantize_rows(bt32)
    if layout[0] == "t":
        a = np.ascontiguousarray(a.T)
    if layout[1] == "n":
        bt = np.ascontiguousarray(bt.T)
    c = None
    if with_c:
        c = torch.from_numpy(_normal(rng, (M, N))).to(torch.bfloat16).float().numpy()
    return LayoutInputs(layout, a, sfa, bt, sfb, M, N, K, c)


def gen_layout_sparse(layout: str, M: int, N: int, K: int, a_rows, seed: int = 0) -> LayoutInputs:
    """gen_layout's workload with an A of up to 2 GiB: A(m, k) is zero except
    the rows m in a_rows (N(0,1) quantised per row per 128-K block; scale 1
    elsewhere), written straight into the layout's orientation; B is N(0,1)
    quantised as in gen_layout."""
    assert layout in ("nn", "tn", "tt")
    rng = _rng(seed)
    rows = np.asarray(sorted(set(int(r) for r in a_rows)), np.int64)
    codes, sf_live = quantize_rows(_normal(rng, (len(rows), K)))
    sfa = np.ones((K // BLOCK, M), np.float32)
    sfa[:, rows] = sf_live
    if layout[0] == "n":
        a = np.zeros((M, K), np.uint8)
        a[rows] = codes
    else:
        a = np.zeros((K, M), np.uint8)
        a[:, rows] = codes.T
    bt, sfb = quantize_rows(_normal(rng, (N, K)))
    if layout[1] == "n":
        bt = np.ascontiguousarray(bt.T)
    return LayoutInputs(layout, a, sfa, bt, sfb, M, N, K, None)


@dataclasses.dataclass
class NNContiguousInputs:
    a: np.ndarray          # uint8 [M_tot, K]
    sfa: np.ndarray        # fp32 [K/128, M_tot]
    b: np.ndarray          # uint8 [G, K, N]
    sfb: np.ndarray        # fp32 [G, K/128, N]
    m_indices: np.ndarray  # int32 [M_tot]
    counts: np.ndarray
    M_tot: int
    N: int
    K: int
    G: int


def gen_nn_contiguous(G: int = 32, N: int = 4096, K: int = 4096, tokens: int = 8192,
                      topk: int = 6, seed: int = 0, counts: Optional[np.ndarray] = None,
                      zipf_s: float = 1.1) -> NNContiguousInputs:
    """The contiguous MoE workload with each expert's B stored [K, N] and
    quantised per column n per 128-K block."""
    rng = _rng(seed)
    if counts is None:
        counts = route_topk_zipf(rng, tokens, G, topk, zipf_s)
    counts = np.asarray(counts, dtype=np.int64)
    m_idx, offs = contiguous_layout(counts)
    M_tot = len(m_idx)
    a32 = np.zeros((M_tot, K), dtype=np.float32)
    valid = _normal(rng, (int(counts.sum()), K))
    r = 0
    for e in range(G):
        c = int(counts[e])
        a32[offs[e]: offs[e] + c] = valid[r: r + c]
        r += c
    del valid
    a, sfa = quantize_rows(a32)
    del a32
    b = np.empty((G, K, N), dtype=np.uint8)
    sfb = np.empty((G, K // BLOCK, N), dtype=np.float32)
    for e in range(G):
        bt, sfb[e] = quantize_rows(_normal(rng, (N, K)))
        b[e] = bt.T
    return NNContiguousInputs(a, sfa, b, sfb, m_idx, counts, M_tot, N, K, G)


# --------------------------------------------------------------------------
# MQA logits (the indexer kernel)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class MqaInputs:
    q: np.ndarray        # uint8 [S, H, D] e4m3 (no scale)
    kv: np.ndarray       # uint8 [S_kv, D] e4m3
    kv_sf: np.ndarray    # fp32 [S_kv], one scale per kv token
    weights: np.ndarray  # fp32 [S, H]
    ks: np.ndarray       # int32 [S], first kv index of query i's range
    ke: np.ndarray       # int32 [S], one past the last
    S: int
    S_kv: int
    H: int
    D: int


def causal_ranges(seq_lens, S_kv: Optional[int] = None):
    """Packed sequences of the given lengths, each query attending to its own
    sequence's tokens up to and including itself: (ks, ke) int32 [sum(lens)].
    With S_kv > sum(lens), the kv side holds a shared prefix of S_kv - sum(lens)
    tokens ahead of the packed sequences that every query also sees."""
    lens = [int(x) for x in seq_lens]
    S = sum(lens)
    prefix = 0 if S_kv is None else S_kv - S
    ks, ke = np.empty(S, np.int32), np.empty(S, np.int32)
    i = 0
    for L in lens:
        for t in range(L):
            ks[i] = 0 if prefix else prefix + (i - t)
            ke[i] = prefix + i + 1
            i += 1
    return ks, ke


def gen_mqa(S: int, S_kv: int, H: int = 64, D: int = 128, seed: int = 0,
            seq_lens=None) -> MqaInputs:
    """q ~ N(0,1) cast to e4m3 (RNE, clamped to +-448; q carries no scale);
    kv ~ N(0,1) quantised per token (scale = amax / 448 over its D values);
    weights ~ N(0,1); causal ranges over packed sequences (one sequence of
    length S by default, S_kv - S shared prefix tokens)."""
    rng = _rng(seed)
    q = _cast_e4m3(torch.from_numpy(_normal(rng, (S, H, D)))).numpy()
    kvc, sf = quantize_rows(_normal(rng, (S_kv, D)))
    w = _normal(rng, (S, H))
    ks, ke = causal_ranges([S] if seq_lens is None else seq_lens, S_kv)
    return MqaInputs(q, kvc, np.ascontiguousarray(sf.reshape(-1)[:S_kv]) if D == BLOCK
                     else None, w, ks, ke, S, S_kv, H, D)


def gen_mqa_sparse(S: int, S_kv: int, H: int, live_queries, seed: int = 0) -> MqaInputs:
    """MQA inputs with a q of many GiB: q is zero except the queries
    live_queries (N(0,1) cast to e4m3 as in gen_mqa, with N(0,1) weights; the
    other weights are 1); kv as in gen_mqa.  Ranges vary with i: ks = i mod
    1024, ke = ks + 1 + (i mod 1021), clamped to [0, S_kv] by the kernel."""
    rng = _rng(seed)
    D = BLOCK
    live = np.asarray(sorted(set(int(i) for i in live_queries)), np.int64)
    q = np.zeros((S, H, D), np.uint8)
    q[live] = _cast_e4m3(torch.from_numpy(_normal(rng, (len(live), H, D)))).numpy()
    kvc, sf = quantize_rows(_normal(rng, (S_kv, D)))
    w = np.ones((S, H), np.float32)
    w[live] = _normal(rng, (len(live), H))
    i = np.arange(S, dtype=np.int64)
    ks = (i % 1024).astype(np.int32)
    ke = (ks + 1 + i % 1021).astype(np.int32)
    return MqaInputs(q, kvc, np.ascontiguousarray(sf.reshape(-1)), w, ks, ke, S, S_kv, H, D)


def k_grouped_ue8m0_words(sf: np.ndarray, k_sizes) -> np.ndarray:
    """Power-of-two fp32 scales [K_tot/128, MN] of a K-grouped operand ->
    packed UE8M0 words, each group's blocks on their own ceil(KB_g / 4) rows."""
    e = exponent_bytes(sf)
    parts, kb = [], 0
    for k in k_sizes:
        nkb = int(k) // BLOCK
        if nkb:
            parts.append(ue8m0_words(e[kb:kb + nkb]))
        kb += nkb
    MN = sf.shape[1]
    return np.concatenate(parts) if parts else np.zeros((0, MN), np.int32)
