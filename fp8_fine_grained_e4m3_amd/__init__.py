"""Python binding of libdg.so, the MI355X (gfx950) fine-grained FP8 e4m3 GEMM.

Argument marshalling only: every step of every GEMM, and of the FP8 casting
that prepares its operands, runs in the HIP kernels behind the C ABI declared
in include/dg.h.  PyTorch supplies device memory and
the current stream.  There is no fallback path: if libdg.so is missing or a
call fails, an exception is raised.

FP8 operands are passed as (data, scale) pairs, data being uint8 (raw e4m3
bytes) or torch.float8_e4m3fn, scales fp32 (the operand convention of the
"DeepGEMM" README, yuguo-Jack fork, section "Interfaces").  For the three NT
forms the scales may instead be packed UE8M0 words (int32, four power-of-two
exponents per word, the README's newer-path format): the dtype of the scale
tensors picks the C entry point.  The caller allocates the output and passes
it in.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP = 0, 1, 2, 3
DG_BF16, DG_F32 = 1, 2

# Every symbol include/dg.h declares (the CPU tests check the library exports them).
EXPORTED = (
    "dg_fp8_gemm_nt",
    "dg_m_grouped_fp8_gemm_nt_contiguous",
    "dg_m_grouped_fp8_gemm_nt_masked",
    "dg_k_grouped_fp8_gemm_tn_contiguous",
    "dg_last_error",
    "dg_get_num_cus",
    "dg_set_num_cus",
    "dg_get_mk_alignment_for_contiguous_layout",
    "dg_kernel_config_name",
    "dg_per_token_cast_to_fp8",
    "dg_per_block_cast_to_fp8",
    "dg_fp8_gemm_nt_ue8m0",
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0",
    "dg_pack_ue8m0_scales",
    "dg_fp8_gemm_nn",
    "dg_fp8_gemm_tn",
    "dg_fp8_gemm_tt",
    "dg_m_grouped_fp8_gemm_nn_contiguous",
    "dg_fp8_mqa_logits",
    "dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0",
    "dg_pack_ue8m0_scales_k_grouped",
    "dg_fp8_gemm_nt_workspace_bytes",
    "dg_fp8_gemm_nt_noalloc",
)
DG_CAST_POW2_SCALE = 1

_lib = None


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dg status {status}: {message}")
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libdg.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m fp8_fine_grained_e4m3_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.dg_fp8_gemm_nt.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P, I64, P]
    lib.dg_fp8_gemm_nt_noalloc.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
    lib.dg_fp8_gemm_nt_noalloc.restype = I
    lib.dg_fp8_gemm_nt_workspace_bytes.argtypes = [I64, I64, I64]
    lib.dg_fp8_gemm_nt_workspace_bytes.restype = I64
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.dg_k_grouped_fp8_gemm_tn_contiguous.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, P]
    for name in EXPORTED[:4]:
        getattr(lib, name).restype = I
    lib.dg_last_error.argtypes = []
    lib.dg_last_error.restype = ctypes.c_char_p
    lib.dg_get_num_cus.argtypes = []
    lib.dg_get_num_cus.restype = I
    lib.dg_set_num_cus.argtypes = [I]
    lib.dg_set_num_cus.restype = I
    lib.dg_get_mk_alignment_for_contiguous_layout.argtypes = []
    lib.dg_get_mk_alignment_for_contiguous_layout.restype = I
    lib.dg_kernel_config_name.argtypes = [I, I64, I64, I64, I]
    lib.dg_kernel_config_name.restype = ctypes.c_char_p
    for name in ("dg_per_token_cast_to_fp8", "dg_per_block_cast_to_fp8"):
        getattr(lib, name).argtypes = [P, I, P, P, I64, I64, I64, I, P]
        getattr(lib, name).restype = I
    lib.dg_fp8_gemm_nt_ue8m0.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P, I64, P]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0.argtypes = [P, P, P, P, P, P, I64, I64, I64,
                                                              I64, P]
    lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.dg_pack_ue8m0_scales.argtypes = [P, I, P, I64, I64, I64, P]
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
        getattr(lib, name).argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
        getattr(lib, name).restype = I
    lib.dg_m_grouped_fp8_gemm_nn_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.dg_m_grouped_fp8_gemm_nn_contiguous.restype = I
    lib.dg_fp8_mqa_logits.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I, P]
    lib.dg_fp8_mqa_logits.restype = I
    lib.dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0.argtypes = [P, P, P, P, P, P, P, I64, I64, I64,
                                                              I64, P]
    lib.dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0.restype = I
    lib.dg_pack_ue8m0_scales_k_grouped.argtypes = [P, P, P, I64, I64, I64, P]
    lib.dg_pack_ue8m0_scales_k_grouped.restype = I
    for name in ("dg_fp8_gemm_nt_ue8m0", "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
                 "dg_m_grouped_fp8_gemm_nt_masked_ue8m0", "dg_pack_ue8m0_scales"):
        getattr(lib, name).restype = I
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != DG_OK:
        raise DGError(status, load_library().dg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _fp8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    return _dev(t, name)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    return _dev(t, name)


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    return _dev(t, name)


def _scales(sa: torch.Tensor, sb: torch.Tensor):
    """Both fp32 (-> False) or both packed UE8M0 int32 words (-> True)."""
    if sa.dtype == torch.int32 and sb.dtype == torch.int32:
        return _dev(sa, "SFA"), _dev(sb, "SFB"), True
    return _f32(sa, "SFA"), _f32(sb, "SFB"), False


def _k4(K: int) -> int:
    """Packed UE8M0 words per row: ceil(K / 512)."""
    return (K // 128 + 3) // 4


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def get_fp8_gemm_nt_workspace_bytes(M: int, N: int, K: int) -> int:
    """Split-K workspace bytes a dense NT call of this shape needs (0: none)."""
    return int(load_library().dg_fp8_gemm_nt_workspace_bytes(M, N, K))


def make_fp8_gemm_nt_workspace(M: int, N: int, K: int, device=None) -> Optional[torch.Tensor]:
    """A zero-filled workspace for dense NT calls of this shape (None when the
    shape needs none).  Stream-ordered calls may reuse it: every call leaves
    its counters zero again."""
    n = get_fp8_gemm_nt_workspace_bytes(M, N, K)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


def fp8_gemm_nt(a: Tuple[torch.Tensor, torch.Tensor], b: Tuple[torch.Tensor, torch.Tensor],
                d: torch.Tensor, c: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d[M,N] = c + a @ b^T.  a = (A [M,K], SFA [K/128, M]), b = (B [N,K],
    SFB [ceil(N/128), K/128]); d bf16 or fp32; c None or like d (may be d).
    Packed UE8M0 scales (int32): SFA [ceil(K/512), M], SFB [ceil(K/512), N].
    workspace: a uint8 device buffer of at least
    get_fp8_gemm_nt_workspace_bytes(M, N, K) bytes whose counters are zero
    (make_fp8_gemm_nt_workspace); when None and the shape splits K, a
    zero-filled one is allocated for this call from torch's allocator."""
    A, B = _fp8(a[0], "A"), _fp8(b[0], "B")
    SA, SB, ue8m0 = _scales(a[1], b[1])
    d = _dev(d, "d")
    if d.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("d must be bfloat16 or float32")
    if c is not None:
        c = _dev(c, "c")
        if c.dtype != d.dtype or c.shape != d.shape:
            raise ValueError("c must match d in dtype and shape")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(d.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)} d {tuple(d.shape)}")
    want = (((_k4(K), M), (_k4(K), N)) if ue8m0
            else ((K // 128, M), ((N + 127) // 128, K // 128)))
    if (tuple(SA.shape), tuple(SB.shape)) != want:
        raise ValueError(f"scale shapes: SFA {tuple(SA.shape)} SFB {tuple(SB.shape)}, want {want}")
    fn = "dg_fp8_gemm_nt_ue8m0" if ue8m0 else "dg_fp8_gemm_nt"
    with torch.cuda.device(d.device):
        need = get_fp8_gemm_nt_workspace_bytes(M, N, K)
        if workspace is None and need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=d.device)
        ws_bytes = 0
        if workspace is not None:
            workspace = _dev(workspace, "workspace")
            if workspace.dtype != torch.uint8:
                raise TypeError("workspace must be uint8")
            ws_bytes = workspace.numel()
        _check(getattr(load_library(), fn)(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(c), _ptr(d),
            DG_F32 if d.dtype == torch.float32 else DG_BF16, M, N, K,
            _ptr(workspace), ws_bytes, _stream(d)))
    return d


def fp8_gemm_nt_noalloc(a: Tuple[torch.Tensor, torch.Tensor], b: Tuple[torch.Tensor, torch.Tensor],
                        d: torch.Tensor, c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8_gemm_nt (fp32 scales) with the split-K workspace taken from the
    library's static per-GPU scratch: nothing is allocated on any call.
    Calls that may overlap on one GPU race on that scratch."""
    A, B = _fp8(a[0], "A"), _fp8(b[0], "B")
    SA, SB = _f32(a[1], "SFA"), _f32(b[1], "SFB")
    d = _dev(d, "d")
    if d.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("d must be bfloat16 or float32")
    if c is not None:
        c = _dev(c, "c")
        if c.dtype != d.dtype or c.shape != d.shape:
            raise ValueError("c must match d in dtype and shape")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(d.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)} d {tuple(d.shape)}")
    want = ((K // 128, M), ((N + 127) // 128, K // 128))
    if (tuple(SA.shape), tuple(SB.shape)) != want:
        raise ValueError(f"scale shapes: SFA {tuple(SA.shape)} SFB {tuple(SB.shape)}, want {want}")
    with torch.cuda.device(d.device):
        _check(load_library().dg_fp8_gemm_nt_noalloc(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(c), _ptr(d),
            DG_F32 if d.dtype == torch.float32 else DG_BF16, M, N, K, _stream(d)))
    return d


def m_grouped_fp8_gemm_nt_contiguous(a: Tuple[torch.Tensor, torch.Tensor],
                                     b: Tuple[torch.Tensor, torch.Tensor],
                                     d: torch.Tensor, m_indices: torch.Tensor) -> torch.Tensor:
    """d[r] = a[r] @ b[m_indices[r]]^T; a = (A [M_tot,K], SFA [K/128, M_tot]),
    b = (B [G,N,K], SFB [G, ceil(N/128), K/128]); d bf16 [M_tot, N].
    Packed UE8M0 scales (int32): SFA [ceil(K/512), M_tot], SFB [G, ceil(K/512), N]."""
    A, B = _fp8(a[0], "A"), _fp8(b[0], "B")
    SA, SB, ue8m0 = _scales(a[1], b[1])
    d, mi = _dev(d, "d"), _i32(m_indices, "m_indices")
    if d.dtype != torch.bfloat16:
        raise TypeError("d must be bfloat16")
    M_tot, K = A.shape
    G, N, Kb = B.shape
    if Kb != K or tuple(d.shape) != (M_tot, N) or tuple(mi.shape) != (M_tot,):
        raise ValueError("shape mismatch")
    want = (((_k4(K), M_tot), (G, _k4(K), N)) if ue8m0
            else ((K // 128, M_tot), (G, (N + 127) // 128, K // 128)))
    if (tuple(SA.shape), tuple(SB.shape)) != want:
        raise ValueError(f"scale shapes: SFA {tuple(SA.shape)} SFB {tuple(SB.shape)}, want {want}")
    fn = ("dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0" if ue8m0
          else "dg_m_grouped_fp8_gemm_nt_contiguous")
    with torch.cuda.device(d.device):
        _check(getattr(load_library(), fn)(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(mi), _ptr(d), M_tot, N, K, G, _stream(d)))
    return d


def m_grouped_fp8_gemm_nt_masked(a: Tuple[torch.Tensor, torch.Tensor],
                                 b: Tuple[torch.Tensor, torch.Tensor],
                                 d: torch.Tensor, masked_m: torch.Tensor) -> torch.Tensor:
    """d[g, r] = a[g, r] @ b[g]^T for r < masked_m[g]; other rows untouched.
    a = (A [G,M_max,K], SFA [G, K/128, M_max]), b = (B [G,N,K], SFB [G,NB,KB]).
    Packed UE8M0 scales (int32): SFA [G, ceil(K/512), M_max], SFB [G, ceil(K/512), N]."""
    A, B = _fp8(a[0], "A"), _fp8(b[0], "B")
    SA, SB, ue8m0 = _scales(a[1], b[1])
    d, mm = _dev(d, "d"), _i32(masked_m, "masked_m")
    if d.dtype != torch.bfloat16:
        raise TypeError("d must be bfloat16")
    G, M_max, K = A.shape
    N = B.shape[1]
    if tuple(B.shape) != (G, N, K) or tuple(d.shape) != (G, M_max, N) or tuple(mm.shape) != (G,):
        raise ValueError("shape mismatch")
    want = (((G, _k4(K), M_max), (G, _k4(K), N)) if ue8m0
            else ((G, K // 128, M_max), (G, (N + 127) // 128, K // 128)))
    if (tuple(SA.shape), tuple(SB.shape)) != want:
        raise ValueError(f"scale shapes: SFA {tuple(SA.shape)} SFB {tuple(SB.shape)}, want {want}")
    fn = "dg_m_grouped_fp8_gemm_nt_masked_ue8m0" if ue8m0 else "dg_m_grouped_fp8_gemm_nt_masked"
    with torch.cuda.device(d.device):
        _check(getattr(load_library(), fn)(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(mm), _ptr(d), G, M_max, N, K, _stream(d)))
    return d


def k_grouped_fp8_gemm_tn_contiguous(a: Tuple[torch.Tensor, torch.Tensor],
                                     b: Tuple[torch.Tensor, torch.Tensor],
                                     d: torch.Tensor, k_sizes: Sequence[int],
                                     c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d[g] = c[g] + a_g^T @ b_g over group g's K rows.  a = (A [K_tot, M],
    SFA [K_tot/128, M]), b = (B [K_tot, N], SFB [K_tot/128, N]); k_sizes is a
    host sequence; d (and c) fp32 [G, M, N].  Packed UE8M0 scales (int32):
    SFA [W, M], SFB [W, N], each group on its own ceil(K_g / 512) word rows."""
    A, B = _fp8(a[0], "A"), _fp8(b[0], "B")
    SA, SB, ue8m0 = _scales(a[1], b[1])
    d = _f32(d, "d")
    if c is not None:
        c = _f32(c, "c")
        if c.shape != d.shape:
            raise ValueError("c must match d")
    ks = np.ascontiguousarray(np.asarray(k_sizes, dtype=np.int64))
    if ks.ndim != 1 or np.any(ks > np.iinfo(np.int32).max) or np.any(ks < np.iinfo(np.int32).min):
        raise ValueError("k_sizes must be a 1-D sequence of int32 values")
    ks = ks.astype(np.int32)
    K_tot, M = A.shape
    N = B.shape[1]
    G = len(ks)
    if B.shape[0] != K_tot or tuple(d.shape) != (G, M, N):
        raise ValueError("shape mismatch")
    rows = _k_grouped_words(ks) if ue8m0 else K_tot // 128
    if tuple(SA.shape) != (rows, M) or tuple(SB.shape) != (rows, N):
        raise ValueError("scale shape mismatch")
    fn = ("dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0" if ue8m0
          else "dg_k_grouped_fp8_gemm_tn_contiguous")
    with torch.cuda.device(d.device):
        _check(getattr(load_library(), fn)(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), ks.ctypes.data_as(ctypes.c_void_p), _ptr(c),
            _ptr(d), G, M, N, K_tot, _stream(d)))
    return d


def get_num_cus() -> int:
    return load_library().dg_get_num_cus()


def set_num_cus(n: int) -> None:
    _check(load_library().dg_set_num_cus(int(n)))


def get_mk_alignment_for_contiguous_layout() -> int:
    return load_library().dg_get_mk_alignment_for_contiguous_layout()


FORM_DENSE, FORM_CONTIGUOUS, FORM_MASKED, FORM_K_GROUPED = 0, 1, 2, 3
FORM_NN, FORM_TN, FORM_TT, FORM_NN_CONTIGUOUS = 4, 5, 6, 7


def kernel_config_name(form: int, rows: int, N: int, K: int, out_f32: bool = False) -> str:
    """Kernel instance (tile configuration) a call with these sizes launches."""
    return load_library().dg_kernel_config_name(form, rows, N, K, int(out_f32)).decode()


def to_mn_major_sf(sf: torch.Tensor) -> torch.Tensor:
    """[rows, K/128] per-row scales -> the MN-major [K/128, rows] layout the
    A-side scale factors use (a transpose + copy; layout only)."""
    return sf.transpose(-1, -2).contiguous()


def _cast(fn: str, x: torch.Tensor, block_scale: bool, pow2_scale: bool,
          out: Optional[Tuple[torch.Tensor, torch.Tensor]]):
    x = _dev(x, "x")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    if x.dim() not in (2, 3):
        raise ValueError("x must be [rows, K] or [G, rows, K]")
    batched = x.dim() == 3
    G, R, K = x.shape if batched else (1,) + tuple(x.shape)
    if K % 128:
        raise ValueError(f"K={K} is not a multiple of 128")
    sf_shape = (G, (R + 127) // 128, K // 128) if block_scale else (G, K // 128, R)
    if not batched:
        sf_shape = sf_shape[1:]
    if out is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        sf = torch.empty(sf_shape, dtype=torch.float32, device=x.device)
    else:
        codes, sf = _fp8(out[0], "codes"), _f32(out[1], "sf")
        if tuple(codes.shape) != tuple(x.shape) or tuple(sf.shape) != sf_shape:
            raise ValueError(f"out shapes: codes {tuple(codes.shape)} sf {tuple(sf.shape)}, "
                             f"want {tuple(x.shape)} and {sf_shape}")
    with torch.cuda.device(x.device):
        _check(getattr(load_library(), fn)(
            _ptr(x), DG_F32 if x.dtype == torch.float32 else DG_BF16, _ptr(codes), _ptr(sf),
            G, R, K, DG_CAST_POW2_SCALE if pow2_scale else 0, _stream(x)))
    return codes, sf


def per_token_cast_to_fp8(x: torch.Tensor, pow2_scale: bool = False,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """1 x 128 casting of activations x [R, K] or [G, R, K] (bf16 or fp32).
    Returns (codes uint8 like x, sf fp32 [K/128, R] or [G, K/128, R]): the A
    operand and its MN-major scales for the GEMM calls above."""
    return _cast("dg_per_token_cast_to_fp8", x, False, pow2_scale, out)


def per_block_cast_to_fp8(w: torch.Tensor, pow2_scale: bool = False,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """128 x 128 casting of weights w [N, K] or [G, N, K] (bf16 or fp32).
    Returns (codes uint8 like w, sf fp32 [ceil(N/128), K/128] or
    [G, ceil(N/128), K/128]): the B operand and its scales."""
    return _cast("dg_per_block_cast_to_fp8", w, True, pow2_scale, out)


def pack_ue8m0_scales(sf: torch.Tensor, mn: Optional[int] = None,
                      per_block: bool = False) -> torch.Tensor:
    """fp32 power-of-two scales -> packed UE8M0 int32 words [.., ceil(K/512), MN].

    per_block False: sf [K/128, MN] or [G, K/128, MN] (A-side, MN-major);
    per_block True: sf [ceil(MN/128), K/128] or [G, ..] (128 x 128 weight
    blocks, each given to its rows; pass mn = N).  Byte i of word k4 holds
    the exponent of K block 4 k4 + i (the layout the *_ue8m0 GEMMs take)."""
    sf = _f32(sf, "sf")
    if sf.dim() not in (2, 3):
        raise ValueError("sf must be 2-D or 3-D")
    batched = sf.dim() == 3
    sf3 = sf if batched else sf.unsqueeze(0)
    G = sf3.shape[0]
    if per_block:
        if mn is None:
            raise ValueError("per_block packing needs mn (the row count N)")
        KB = sf3.shape[2]
        if sf3.shape[1] != (mn + 127) // 128:
            raise ValueError(f"sf {tuple(sf.shape)} does not cover {mn} rows")
    else:
        KB, MN = sf3.shape[1], sf3.shape[2]
        if mn is not None and mn != MN:
            raise ValueError(f"mn={mn} but sf has {MN} rows")
        mn = MN
    out = torch.empty((G, (KB + 3) // 4, mn), dtype=torch.int32, device=sf.device)
    with torch.cuda.device(sf.device):
        _check(load_library().dg_pack_ue8m0_scales(_ptr(sf3), int(per_block), _ptr(out), G, mn,
                                                   KB * 128, _stream(sf)))
    return out if batched else out[0]


def _gemm_layout(layout: str, a, b, d, c):
    """Dense NN / TN / TT: A stored [M, K] ("n") or [K, M] ("t"); B stored
    [K, N] ("n") or [N, K] ("t"); SFA fp32 [K/128, M], SFB fp32 [K/128, N]."""
    A, SA = _fp8(a[0], "A"), _f32(a[1], "SFA")
    B, SB = _fp8(b[0], "B"), _f32(b[1], "SFB")
    d = _dev(d, "d")
    if d.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("d must be bfloat16 or float32")
    if c is not None:
        c = _dev(c, "c")
        if c.dtype != d.dtype or c.shape != d.shape:
            raise ValueError("c must match d in dtype and shape")
    M, K = A.shape if layout[0] == "n" else A.shape[::-1]
    N, Kb = B.shape if layout[1] == "t" else B.shape[::-1]
    if Kb != K or tuple(d.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)} d {tuple(d.shape)}")
    if tuple(SA.shape) != (K // 128, M) or tuple(SB.shape) != (K // 128, N):
        raise ValueError(f"scale shapes: SFA {tuple(SA.shape)} SFB {tuple(SB.shape)}, "
                         f"want {(K // 128, M)} and {(K // 128, N)}")
    with torch.cuda.device(d.device):
        _check(getattr(load_library(), f"dg_fp8_gemm_{layout}")(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(c), _ptr(d),
            DG_F32 if d.dtype == torch.float32 else DG_BF16, M, N, K, _stream(d)))
    return d


def fp8_gemm_nn(a, b, d, c=None):
    """d[M,N] = c + A @ B; a = (A [M,K], SFA [K/128, M]), b = (B [K,N], SFB [K/128, N])."""
    return _gemm_layout("nn", a, b, d, c)


def fp8_gemm_tn(a, b, d, c=None):
    """d[M,N] = c + A^T @ B; a = (A [K,M], SFA [K/128, M]), b = (B [K,N], SFB [K/128, N])."""
    return _gemm_layout("tn", a, b, d, c)


def fp8_gemm_tt(a, b, d, c=None):
    """d[M,N] = c + A^T @ B^T; a = (A [K,M], SFA [K/128, M]), b = (B [N,K], SFB [K/128, N])."""
    return _gemm_layout("tt", a, b, d, c)


def m_grouped_fp8_gemm_nn_contiguous(a, b, d: torch.Tensor, m_indices: torch.Tensor) -> torch.Tensor:
    """d[r] = a[r] @ b[m_indices[r]]; a = (A [M_tot,K], SFA [K/128, M_tot]),
    b = (B [G,K,N], SFB [G, K/128, N]); d bf16 [M_tot, N]."""
    A, SA = _fp8(a[0], "A"), _f32(a[1], "SFA")
    B, SB = _fp8(b[0], "B"), _f32(b[1], "SFB")
    d, mi = _dev(d, "d"), _i32(m_indices, "m_indices")
    if d.dtype != torch.bfloat16:
        raise TypeError("d must be bfloat16")
    M_tot, K = A.shape
    G, Kb, N = B.shape
    if Kb != K or tuple(d.shape) != (M_tot, N) or tuple(mi.shape) != (M_tot,):
        raise ValueError("shape mismatch")
    if tuple(SA.shape) != (K // 128, M_tot) or tuple(SB.shape) != (G, K // 128, N):
        raise ValueError("scale shape mismatch")
    with torch.cuda.device(d.device):
        _check(load_library().dg_m_grouped_fp8_gemm_nn_contiguous(
            _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(mi), _ptr(d), M_tot, N, K, G, _stream(d)))
    return d


def fp8_mqa_logits(q: torch.Tensor, kv: Tuple[torch.Tensor, torch.Tensor], weights: torch.Tensor,
                   cu_seq_len_k_start: torch.Tensor, cu_seq_len_k_end: torch.Tensor,
                   clean_logits: bool = True, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """logits[i, j] = sum_h relu(q[i, h] . kv[j] * sf[j]) * weights[i, h] for j in
    [start[i], end[i]) (-inf elsewhere when clean_logits).  q e4m3 [S, H, 128],
    kv = (e4m3 [S_kv, 128], fp32 [S_kv]), weights fp32 [S, H], ranges int32 [S];
    returns fp32 [S, S_kv] (or fills `out`)."""
    Q = _fp8(q, "q")
    KV, SF = _fp8(kv[0], "kv"), _f32(kv[1], "kv_sf")
    W = _f32(weights, "weights")
    ks, ke = _i32(cu_seq_len_k_start, "cu_seq_len_k_start"), _i32(cu_seq_len_k_end, "cu_seq_len_k_end")
    if Q.dim() != 3:
        raise ValueError("q must be [seq_len, num_heads, head_dim]")
    S, H, D = Q.shape
    S_kv = KV.shape[0]
    if tuple(KV.shape) != (S_kv, D) or tuple(SF.shape) != (S_kv,) or tuple(W.shape) != (S, H):
        raise ValueError("shape mismatch")
    if tuple(ks.shape) != (S,) or tuple(ke.shape) != (S,):
        raise ValueError("range shape mismatch")
    if out is None:
        out = torch.empty(S, S_kv, dtype=torch.float32, device=Q.device)
    else:
        out = _f32(out, "out")
        if tuple(out.shape) != (S, S_kv):
            raise ValueError("out shape mismatch")
    with torch.cuda.device(Q.device):
        _check(load_library().dg_fp8_mqa_logits(
            _ptr(Q), _ptr(KV), _ptr(SF), _ptr(W), _ptr(ks), _ptr(ke), _ptr(out), S, S_kv, H, D,
            int(bool(clean_logits)), _stream(out)))
    return out


def _k_grouped_words(k_sizes) -> int:
    return int(sum((int(k) // 128 + 3) // 4 for k in k_sizes))


def pack_ue8m0_scales_k_grouped(sf: torch.Tensor, k_sizes: Sequence[int]) -> torch.Tensor:
    """fp32 power-of-two scales [K_tot/128, MN] of a K-grouped operand ->
    packed UE8M0 words [sum_g ceil(K_g / 512), MN], each group on its own rows."""
    sf = _f32(sf, "sf")
    ks = np.ascontiguousarray(np.asarray(k_sizes, dtype=np.int32))
    KB, MN = sf.shape
    out = torch.empty((_k_grouped_words(ks), MN), dtype=torch.int32, device=sf.device)
    with torch.cuda.device(sf.device):
        _check(load_library().dg_pack_ue8m0_scales_k_grouped(
            _ptr(sf), ks.ctypes.data_as(ctypes.c_void_p), _ptr(out), len(ks), MN, KB * 128,
            _stream(sf)))
    return out
