"""dg_fp8_gemm_nt_noalloc, the dense NT entry point for callers that cannot
allocate (code under graph capture, tight serving loops, harnesses that forbid
hipMalloc): its split-K workspace is the library's static per-GPU scratch.

Called through the C ABI and compared, bit for bit, with dg_fp8_gemm_nt run
with a caller-owned workspace, over consecutive calls: a split shape, then a
smaller split shape (the scratch keeps the first call's partials; its
counters must have been left zero), then a shape that does not split, then
the first shape again, with bf16 and fp32 outputs and an in-place C.  Each
call's own result is also checked against the oracle for the first shape.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp8_fine_grained_e4m3_amd as dg
import oracle
from tests import gen
from tests.parity import announce, check_close, dev, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield


def noalloc(lib, ops, d, c=None):
    (a, sa), (b, sb) = ops
    M, K = a.shape
    N = b.shape[0]
    st = lib.dg_fp8_gemm_nt_noalloc(
        ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(sa.data_ptr()),
        ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(sb.data_ptr()),
        None if c is None else ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(d.data_ptr()),
        dg.DG_F32 if d.dtype == torch.float32 else dg.DG_BF16, M, N, K,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == dg.DG_OK, lib.dg_last_error().decode()


def test_noalloc_equals_the_workspace_entry_point_over_consecutive_calls():
    lib = dg.load_library()
    shapes = [(128, 7168, 16384), (64, 2112, 7168), (4096, 2112, 7168), (128, 7168, 16384)]
    need = [dg.get_fp8_gemm_nt_workspace_bytes(*s) for s in shapes]
    assert need[0] > need[1] > 0 and need[2] == 0
    xs = {s: gen.gen_dense(*s, seed=500 + i) for i, s in enumerate(shapes[:3])}
    for i, s in enumerate(shapes):
        M, N, K = s
        announce(f"noalloc call {i}: {M}x{N}x{K}")
        x = xs[s]
        ops = ((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)))
        for out_dtype in (torch.bfloat16, torch.float32):
            want = torch.empty(M, N, dtype=out_dtype, device="cuda")
            dg.fp8_gemm_nt(*ops, want, workspace=dg.make_fp8_gemm_nt_workspace(M, N, K))
            got = torch.empty(M, N, dtype=out_dtype, device="cuda")
            noalloc(lib, ops, got)
            torch.cuda.synchronize()
            assert torch.equal(got, want), f"call {i} {s} {out_dtype}"
        if i == 0:
            check_close(to64(got), oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb), "noalloc vs oracle")
    # in-place C (bf16), a split shape
    M, N, K = shapes[1]
    x = xs[shapes[1]]
    ops = ((dev(x.a), dev(x.sfa)), (dev(x.b), dev(x.sfb)))
    c0 = torch.from_numpy(np.random.default_rng(7).standard_normal((M, N)).astype(np.float32))
    want = c0.to(torch.bfloat16).cuda()
    dg.fp8_gemm_nt(*ops, want, c=want)
    got = c0.to(torch.bfloat16).cuda()
    noalloc(lib, ops, got, c=got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "in-place C"


def test_noalloc_rejects_like_the_workspace_entry_point():
    lib = dg.load_library()
    p = ctypes.c_void_p(0x10000)
    st = lib.dg_fp8_gemm_nt_noalloc(p, p, ctypes.c_void_p(0x20000), p, None,
                                    ctypes.c_void_p(0x30000), dg.DG_BF16, 64, 2112, 500, None)
    assert st == dg.DG_ERR_INVALID_ARG and b"K=500" in lib.dg_last_error()
