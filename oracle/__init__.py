"""fp64 CPU oracle for the fine-grained FP8 e4m3 GEMM -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The GPU library never imports, links or calls it, and
the two share no code.  The arithmetic lives in oracle.c (plain C, built with
gcc, -ffp-contract=off); this wrapper only marshals numpy arrays.

The GEMM functions return float64 arrays.  Rows with no reference value
(padding rows of the contiguous layout, rows at or past masked_m) come back as
NaN.  The casting functions (cast_rows, cast_blocks, e4m3_encode) return the
e4m3 codes and fp32 scales they define, bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None
_override = None


def compile_source(src: str, out: str) -> str:
    """gcc + OpenMP build of one oracle source file into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (next to this file)."""
    if force or not os.path.exists(LIB_PATH):
        compile_source(SRC_PATH, LIB_PATH)
    return LIB_PATH


class use_library:
    """Context manager: route the wrappers to another build of the oracle
    (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _override
        self.prev = _override
        _override = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_e4m3_decode.argtypes = [P, P, I]
    lib.oracle_e4m3_decode.restype = None
    lib.oracle_gemm_nt.argtypes = [P, P, P, P, P, I, I, I, P, I, P]
    lib.oracle_gemm_nt.restype = ctypes.c_int
    lib.oracle_m_grouped_contiguous.argtypes = [P, P, P, P, P, I, I, I, I, P, I, P]
    lib.oracle_m_grouped_contiguous.restype = ctypes.c_int
    lib.oracle_m_grouped_masked.argtypes = [P, P, P, P, P, I, I, I, I, P, P, I, P]
    lib.oracle_m_grouped_masked.restype = ctypes.c_int
    lib.oracle_k_grouped_tn.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, I, P]
    lib.oracle_k_grouped_tn.restype = ctypes.c_int
    lib.oracle_e4m3_encode.argtypes = [P, P, I]
    lib.oracle_e4m3_encode.restype = None
    lib.oracle_cast_rows.argtypes = [P, I, I, I, ctypes.c_int, P, P]
    lib.oracle_cast_rows.restype = ctypes.c_int
    lib.oracle_cast_blocks.argtypes = [P, I, I, I, ctypes.c_int, P, P]
    lib.oracle_cast_blocks.restype = ctypes.c_int
    lib.oracle_gemm_nt_ue8m0.argtypes = [P, P, P, P, P, I, I, I, P, I, P]
    lib.oracle_gemm_nt_ue8m0.restype = ctypes.c_int
    lib.oracle_pack_ue8m0.argtypes = [P, ctypes.c_int, I, I, P]
    lib.oracle_pack_ue8m0.restype = ctypes.c_int
    lib.oracle_gemm_layout.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P, I, I, I, P, I, P]
    lib.oracle_gemm_layout.restype = ctypes.c_int
    lib.oracle_mqa_logits.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_int, P, I, P]
    lib.oracle_mqa_logits.restype = ctypes.c_int
    lib.oracle_k_grouped_tn_ue8m0.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, I, P]
    lib.oracle_k_grouped_tn_ue8m0.restype = ctypes.c_int
    lib.oracle_pack_ue8m0_k_grouped.argtypes = [P, P, I, I, P]
    lib.oracle_pack_ue8m0_k_grouped.restype = ctypes.c_int
    return lib


def _c(x, dtype):
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(x):
    return None if x is None else x.ctypes.data


def num_threads() -> int:
    """OpenMP threads the oracle will use (OMP_NUM_THREADS, else all cores)."""
    v = os.environ.get("OMP_NUM_THREADS")
    if v and v.isdigit():
        return int(v)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode(_ptr(c), _ptr(out), c.size)
    return out


def gemm_nt(a, sfa, b, sfb, c=None, rows=None) -> np.ndarray:
    """D[rows] of D = C + A @ B^T.  a [M,K] u8, sfa [K/128,M], b [N,K] u8,
    sfb [ceil(N/128),K/128], c [M,N] (any float dtype) or None."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and sfa.shape == (K // 128, M)
    assert sfb.shape == ((N + 127) // 128, K // 128)
    cc = None if c is None else _c(c, np.float32)
    if cc is not None:
        assert cc.shape == (M, N)
    r = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    rc = _load().oracle_gemm_nt(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(cc),
                                M, N, K, _ptr(r), len(r), _ptr(out))
    if rc:
        raise ValueError("oracle_gemm_nt: bad arguments")
    return out


def m_grouped_contiguous(a, sfa, b, sfb, m_indices, rows=None) -> np.ndarray:
    """D[rows] of the contiguous M-grouped GEMM.  b [G,N,K], sfb [G,NB,KB]."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32)
    mi = _c(m_indices, np.int32)
    M_tot, K = a.shape
    G, N, _ = b.shape
    assert sfa.shape == (K // 128, M_tot) and mi.shape == (M_tot,)
    r = np.arange(M_tot, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    rc = _load().oracle_m_grouped_contiguous(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(mi),
                                             M_tot, N, K, G, _ptr(r), len(r), _ptr(out))
    if rc:
        raise ValueError("oracle_m_grouped_contiguous: bad arguments")
    return out


def m_grouped_masked(a, sfa, b, sfb, masked_m, groups=None, rows=None) -> np.ndarray:
    """Selected (group, row) outputs of the masked M-grouped GEMM; with no
    selection, the full [G, M_max, N] array.  a [G,M_max,K], sfa [G,KB,M_max]."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32)
    mm = _c(masked_m, np.int32)
    G, M_max, K = a.shape
    N = b.shape[1]
    full = groups is None
    if full:
        groups = np.repeat(np.arange(G), M_max)
        rows = np.tile(np.arange(M_max), G)
    g = _c(groups, np.int64); r = _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    rc = _load().oracle_m_grouped_masked(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(mm),
                                         G, M_max, N, K, _ptr(g), _ptr(r), len(r), _ptr(out))
    if rc:
        raise ValueError("oracle_m_grouped_masked: bad arguments")
    return out.reshape(G, M_max, N) if full else out


def k_grouped_tn(a, sfa, b, sfb, k_sizes, c=None, groups=None, rows=None) -> np.ndarray:
    """Selected (group, m) rows of D[g] = C[g] + A_g^T @ B_g; with no
    selection, the full [G, M, N].  a [K_tot,M], b [K_tot,N], sf [K_tot/128, M|N]."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32)
    ks = _c(k_sizes, np.int32)
    K_tot, M = a.shape
    N = b.shape[1]
    G = len(ks)
    cc = None if c is None else _c(c, np.float32)
    full = groups is None
    if full:
        groups = np.repeat(np.arange(G), M)
        rows = np.tile(np.arange(M), G)
    g = _c(groups, np.int64); r = _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    rc = _load().oracle_k_grouped_tn(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(ks), _ptr(cc),
                                     G, M, N, K_tot, _ptr(g), _ptr(r), len(r), _ptr(out))
    if rc:
        raise ValueError("oracle_k_grouped_tn: bad arguments")
    return out.reshape(G, M, N) if full else out


def e4m3_encode(values) -> np.ndarray:
    """Nearest e4m3 codes (ties to even mantissa, |y| >= 448 -> +-448)."""
    y = _c(values, np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode(_ptr(y), _ptr(out), y.size)
    return out


def cast_rows(x, pow2: bool = False):
    """1 x 128 casting of activations x [R, K] or [G, R, K] (any float dtype
    exact in fp32).  Returns (codes uint8 like x, sf fp32 [K/128, R] or
    [G, K/128, R])."""
    xx = np.asarray(x)
    batched = xx.ndim == 3
    x3 = _c(xx if batched else xx[None], np.float32)
    G, R, K = x3.shape
    codes = np.empty((G, R, K), dtype=np.uint8)
    sf = np.empty((G, K // 128, R), dtype=np.float32)
    if _load().oracle_cast_rows(_ptr(x3), G, R, K, int(pow2), _ptr(codes), _ptr(sf)):
        raise ValueError("oracle_cast_rows: bad arguments")
    return (codes, sf) if batched else (codes[0], sf[0])


def cast_blocks(w, pow2: bool = False):
    """128 x 128 casting of weights w [N, K] or [G, N, K].  Returns (codes,
    sf fp32 [ceil(N/128), K/128] or [G, ceil(N/128), K/128])."""
    ww = np.asarray(w)
    batched = ww.ndim == 3
    w3 = _c(ww if batched else ww[None], np.float32)
    G, N, K = w3.shape
    codes = np.empty((G, N, K), dtype=np.uint8)
    sf = np.empty((G, (N + 127) // 128, K // 128), dtype=np.float32)
    if _load().oracle_cast_blocks(_ptr(w3), G, N, K, int(pow2), _ptr(codes), _ptr(sf)):
        raise ValueError("oracle_cast_blocks: bad arguments")
    return (codes, sf) if batched else (codes[0], sf[0])


def gemm_nt_ue8m0(a, sfa_packed, b, sfb_packed, c=None, rows=None) -> np.ndarray:
    """D[rows] of D = C + A @ B^T with packed UE8M0 per-row scales:
    sfa_packed int32 [ceil(K/512), M], sfb_packed int32 [ceil(K/512), N]."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sfa_packed, np.int32); sb = _c(sfb_packed, np.int32)
    M, K = a.shape
    N = b.shape[0]
    K4 = (K // 128 + 3) // 4
    assert b.shape[1] == K and sa.shape == (K4, M) and sb.shape == (K4, N)
    cc = None if c is None else _c(c, np.float32)
    r = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    if _load().oracle_gemm_nt_ue8m0(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(cc), M, N, K,
                                    _ptr(r), len(r), _ptr(out)):
        raise ValueError("oracle_gemm_nt_ue8m0: bad arguments")
    return out


def pack_ue8m0(sf, per_block: bool, MN: int, K: int) -> np.ndarray:
    """Power-of-two fp32 scales -> packed UE8M0 int32 [ceil(K/512), MN].
    per_block=False: sf [K/128, MN]; True: sf [ceil(MN/128), K/128]."""
    s = _c(sf, np.float32)
    out = np.empty(((K // 128 + 3) // 4, MN), dtype=np.int32)
    if _load().oracle_pack_ue8m0(_ptr(s), int(per_block), MN, K, _ptr(out)):
        raise ValueError("oracle_pack_ue8m0: bad arguments or a scale that is not a power of two")
    return out


def gemm_layout(layout: str, a, sfa, b, sfb, c=None, rows=None) -> np.ndarray:
    """D[rows] of the GEMM in layout "nn", "tn", "tt" (or "nt" with per-row B
    scales): A stored [M, K] ("n") or [K, M] ("t"), B stored [K, N] ("n") or
    [N, K] ("t"); sfa fp32 [K/128, M], sfb fp32 [K/128, N]; c fp32 [M, N]."""
    assert layout in ("nn", "tn", "tt", "nt")
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sfa, np.float32); sb = _c(sfb, np.float32)
    a_mk, b_nk = layout[0] == "n", layout[1] == "t"
    M, K = a.shape if a_mk else a.shape[::-1]
    N = b.shape[0] if b_nk else b.shape[1]
    assert (b.shape[1] if b_nk else b.shape[0]) == K
    assert sa.shape == (K // 128, M) and sb.shape == (K // 128, N)
    cc = None if c is None else _c(c, np.float32)
    r = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    if _load().oracle_gemm_layout(_ptr(a), int(a_mk), _ptr(sa), _ptr(b), int(b_nk), _ptr(sb),
                                  _ptr(cc), M, N, K, _ptr(r), len(r), _ptr(out)):
        raise ValueError("oracle_gemm_layout: bad arguments")
    return out


def m_grouped_nn_contiguous(a, sfa, b, sfb, m_indices, rows=None) -> np.ndarray:
    """M-grouped contiguous NN: D[r] = A[r] @ B[e_r] with e_r = m_indices[r];
    A [M_tot, K], sfa [K/128, M_tot], B [G, K, N], sfb [G, K/128, N].  Rows
    whose index is outside [0, G) have no reference (NaN).  Each expert's
    rows are the NN definition with that expert's B."""
    mi = np.asarray(m_indices)
    G, _, N = b.shape
    r = np.arange(len(mi), dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    out = np.full((len(r), N), np.nan)
    for e in range(G):
        sel = np.nonzero(mi[r] == e)[0]
        if len(sel):
            out[sel] = gemm_layout("nn", a, sfa, b[e], sfb[e], rows=r[sel])
    return out


def mqa_logits(q, kv, kv_sf, weights, ks, ke, clean: bool = True, rows=None) -> np.ndarray:
    """out[rows] of the MQA logits: q uint8 [S, H, D], kv uint8 [S_kv, D],
    kv_sf fp32 [S_kv], weights fp32 [S, H], ks / ke int32 [S]; fp64
    [len(rows), S_kv] with -inf (clean) or NaN outside each row's range."""
    q = _c(q, np.uint8); kv = _c(kv, np.uint8)
    sf = _c(kv_sf, np.float32); w = _c(weights, np.float32)
    ks = _c(ks, np.int32); ke = _c(ke, np.int32)
    S, H, D = q.shape
    S_kv = kv.shape[0]
    assert kv.shape == (S_kv, D) and sf.shape == (S_kv,) and w.shape == (S, H)
    assert ks.shape == (S,) and ke.shape == (S,)
    r = np.arange(S, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((len(r), S_kv), dtype=np.float64)
    if _load().oracle_mqa_logits(_ptr(q), _ptr(kv), _ptr(sf), _ptr(w), _ptr(ks), _ptr(ke), S, S_kv,
                                 H, D, int(clean), _ptr(r), len(r), _ptr(out)):
        raise ValueError("oracle_mqa_logits: bad arguments")
    return out


def k_grouped_word_rows(k_sizes) -> int:
    """Packed UE8M0 word rows of a K-grouped operand: sum_g ceil(K_g / 512)."""
    return int(sum((int(k) // 128 + 3) // 4 for k in k_sizes))


def k_grouped_tn_ue8m0(a, sfa_packed, b, sfb_packed, k_sizes, c=None, groups=None,
                       rows=None) -> np.ndarray:
    """The K-grouped TN form with per-group packed UE8M0 scales
    (sfa_packed [W, M], sfb_packed [W, N], W = k_grouped_word_rows(k_sizes))."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sfa_packed, np.int32); sb = _c(sfb_packed, np.int32)
    ks = _c(k_sizes, np.int32)
    K_tot, M = a.shape
    N = b.shape[1]
    G = len(ks)
    W = k_grouped_word_rows(ks)
    assert sa.shape == (W, M) and sb.shape == (W, N)
    cc = None if c is None else _c(c, np.float32)
    full = groups is None
    if full:
        groups = np.repeat(np.arange(G), M)
        rows = np.tile(np.arange(M), G)
    g = _c(groups, np.int64); r = _c(rows, np.int64)
    out = np.empty((len(r), N), dtype=np.float64)
    if _load().oracle_k_grouped_tn_ue8m0(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(ks), _ptr(cc),
                                         G, M, N, K_tot, _ptr(g), _ptr(r), len(r), _ptr(out)):
        raise ValueError("oracle_k_grouped_tn_ue8m0: bad arguments")
    return out.reshape(G, M, N) if full else out


def pack_ue8m0_k_grouped(sf, k_sizes) -> np.ndarray:
    """fp32 power-of-two scales [K_tot/128, MN] -> per-group packed words [W, MN]."""
    s = _c(sf, np.float32)
    ks = _c(k_sizes, np.int32)
    MN = s.shape[1]
    out = np.zeros((k_grouped_word_rows(ks), MN), dtype=np.int32)
    if _load().oracle_pack_ue8m0_k_grouped(_ptr(s), _ptr(ks), len(ks), MN, _ptr(out)):
        raise ValueError("oracle_pack_ue8m0_k_grouped: bad arguments or a non-power-of-two scale")
    return out
