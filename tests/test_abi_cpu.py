"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before any HIP call.

No GPU is needed: invalid arguments never reach the device (validation runs
first), so fake, never-dereferenced device addresses are enough.  Nothing here
launches a kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import fp8_fine_grained_e4m3_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")

P16 = ctypes.c_void_p(0x10000)      # fake 16-byte-aligned device addresses
P16b = ctypes.c_void_p(0x20000)
P16c = ctypes.c_void_p(0x30000)
BAD = ctypes.c_void_p(0x10008)      # 8-byte aligned only
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return dg.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dg_status|const char\*|int|int64_t)\s+(dg_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_four_gemms_and_utilities():
    syms = declared_symbols()
    for name in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous",
                 "dg_m_grouped_fp8_gemm_nt_masked", "dg_k_grouped_fp8_gemm_tn_contiguous"):
        assert name in syms
    assert set(syms) == set(dg.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {dg.LIB_PATH}").read()
    for name in declared_symbols():
        assert re.search(rf"\bT {name}\b", nm), name


def test_alignment_getter(lib):
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128


def err(lib):
    return lib.dg_last_error().decode()


def nt(lib, a=P16, sfa=P16, b=P16b, sfb=P16, c=NULL, d=P16c, dt=dg.DG_BF16, M=128, N=256, K=512,
       ws=NULL, ws_bytes=0):
    return lib.dg_fp8_gemm_nt(a, sfa, b, sfb, c, d, dt, M, N, K, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(K=500), "K=500"),
    (dict(N=250), "N=250"),
    (dict(M=-1), "negative"),
    (dict(dt=7), "d_dtype"),
    (dict(a=NULL), "a is NULL"),
    (dict(b=BAD), "b is not 16-byte"),
    (dict(d=NULL), "d is NULL"),
    (dict(sfa=NULL), "sfa is NULL"),
    (dict(sfb=ctypes.c_void_p(0x10004)), "sfb is not 16-byte"),
    (dict(c=ctypes.c_void_p(0x30000 + 64)), "overlaps"),
    (dict(M=1 << 22, K=1024), "2^31"),
])
def test_dense_rejects(lib, kw, needle):
    st = nt(lib, **kw)
    assert st == dg.DG_ERR_INVALID_ARG
    assert needle in err(lib)


def test_dense_zero_size_is_a_noop(lib):
    assert nt(lib, M=0) == dg.DG_OK
    assert nt(lib, N=0, a=NULL) == dg.DG_OK
    assert err(lib) == ""


def test_contiguous_rejects(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert f(P16, P16, P16b, P16, P16, P16c, 200, 256, 512, 4, None) == dg.DG_ERR_INVALID_ARG
    assert "multiple of 128" in err(lib)
    assert f(P16, P16, P16b, P16, P16, P16c, 256, 256, 512, 0, None) == dg.DG_ERR_INVALID_ARG
    assert "G=0" in err(lib)
    assert f(P16, P16, P16b, P16, NULL, P16c, 256, 256, 512, 4, None) == dg.DG_ERR_INVALID_ARG
    assert "m_indices is NULL" in err(lib)
    assert f(P16, P16, P16b, P16, P16, P16c, 0, 256, 512, 4, None) == dg.DG_OK


def test_masked_rejects(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert f(P16, P16, P16b, P16, NULL, P16c, 4, 256, 256, 512, None) == dg.DG_ERR_INVALID_ARG
    assert "masked_m is NULL" in err(lib)
    assert f(P16, P16, P16b, P16, P16, P16c, 4, 256, 250, 512, None) == dg.DG_ERR_INVALID_ARG
    assert f(P16, P16, P16b, P16, P16, P16c, 0, 256, 256, 512, None) == dg.DG_OK
    # a group count whose tile count would overflow is rejected before any product
    assert f(P16, P16, P16b, P16, P16, P16c, 2**40, 256, 256, 512, None) == dg.DG_ERR_INVALID_ARG
    assert "G too large" in err(lib)
    assert f(P16, P16, P16b, P16, P16, P16c, 2**20, 2**14, 2**14, 128, None) == dg.DG_ERR_INVALID_ARG
    assert "too many tiles" in err(lib)


def test_k_grouped_rejects(lib):
    f = lib.dg_k_grouped_fp8_gemm_tn_contiguous

    def call(ks, M=256, N=256, K_tot=None, c=NULL, d=P16c, G=None):
        ks = np.asarray(ks, np.int32)
        K_tot = int(ks.sum()) if K_tot is None else K_tot
        G = len(ks) if G is None else G
        return f(P16, P16, P16b, P16, ks.ctypes.data_as(ctypes.c_void_p), c, d, G, M, N, K_tot,
                 None)

    assert call([128, 100]) == dg.DG_ERR_INVALID_ARG and "multiple of 128" in err(lib)
    assert call([128, 256], K_tot=512) == dg.DG_ERR_INVALID_ARG and "K_tot" in err(lib)
    assert call([128], M=200) == dg.DG_ERR_INVALID_ARG
    assert call([128] * 257) == dg.DG_ERR_INVALID_ARG and "G=257" in err(lib)
    assert call([128], c=ctypes.c_void_p(0x30000 + 16)) == dg.DG_ERR_INVALID_ARG
    assert call([128, 0], M=0) == dg.DG_OK


def test_cast_rejects(lib):
    for f in (lib.dg_per_token_cast_to_fp8, lib.dg_per_block_cast_to_fp8):
        def call(x=P16, dt=dg.DG_BF16, codes=P16b, sf=P16c, G=1, R=64, K=256, flags=0):
            return f(x, dt, codes, sf, G, R, K, flags, None)
        assert call(K=200) == dg.DG_ERR_INVALID_ARG and "K=200" in err(lib)
        assert call(R=-1) == dg.DG_ERR_INVALID_ARG and "negative" in err(lib)
        assert call(dt=9) == dg.DG_ERR_INVALID_ARG and "dtype" in err(lib)
        assert call(flags=2) == dg.DG_ERR_INVALID_ARG and "flags" in err(lib)
        assert call(x=BAD) == dg.DG_ERR_INVALID_ARG and "16-byte" in err(lib)
        assert call(codes=NULL) == dg.DG_ERR_INVALID_ARG and "codes is NULL" in err(lib)
        assert call(codes=ctypes.c_void_p(0x10000 + 64 * 256)) == dg.DG_ERR_INVALID_ARG
        assert "overlap" in err(lib)
        assert call(R=1 << 24, K=1024) == dg.DG_ERR_INVALID_ARG and "2^31" in err(lib)
        assert call(R=0, x=NULL) == dg.DG_OK and call(G=0, x=NULL) == dg.DG_OK
        assert call(K=0, x=NULL) == dg.DG_OK


def test_valid_call_without_gpu_fails_cleanly(lib):
    """With valid arguments the library asks HIP for the device; with no GPU
    that fails with a HIP or unsupported-device status, never a crash."""
    st = nt(lib)
    assert st in (dg.DG_ERR_HIP, dg.DG_ERR_UNSUPPORTED, dg.DG_OK)
    if st != dg.DG_OK:
        assert err(lib)


def test_python_binding_rejects_host_tensors():
    import torch
    a = torch.zeros(128, 512, dtype=torch.uint8)
    sa = torch.ones(4, 128)
    b = torch.zeros(256, 512, dtype=torch.uint8)
    sb = torch.ones(2, 4)
    d = torch.empty(128, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        dg.fp8_gemm_nt((a, sa), (b, sb), d)


def test_no_oracle_in_product_path():
    """The GPU package neither imports nor links the oracle."""
    pkg = os.path.join(ROOT, "fp8_fine_grained_e4m3_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn
    nm = os.popen(f"nm -D {dg.LIB_PATH}").read()
    assert "oracle" not in nm


def test_ue8m0_entry_points_reject(lib):
    def f(*args):
        return lib.dg_fp8_gemm_nt_ue8m0(*args[:-1], NULL, 0, args[-1])
    assert f(P16, P16, P16b, P16, NULL, P16c, dg.DG_BF16, 128, 256, 500, None) == dg.DG_ERR_INVALID_ARG
    assert "K=500" in err(lib)
    assert f(P16, NULL, P16b, P16, NULL, P16c, dg.DG_BF16, 128, 256, 512, None) == dg.DG_ERR_INVALID_ARG
    assert "sfa is NULL" in err(lib)
    assert f(P16, P16, P16b, P16, NULL, P16c, 9, 128, 256, 512, None) == dg.DG_ERR_INVALID_ARG
    assert f(P16, P16, P16b, P16, NULL, P16c, dg.DG_BF16, 0, 256, 512, None) == dg.DG_OK
    g = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0
    assert g(P16, P16, P16b, P16, P16, P16c, 200, 256, 512, 4, None) == dg.DG_ERR_INVALID_ARG
    assert "multiple of 128" in err(lib)
    h = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0
    assert h(P16, P16, P16b, P16, NULL, P16c, 4, 256, 256, 512, None) == dg.DG_ERR_INVALID_ARG
    assert "masked_m is NULL" in err(lib)


def test_pack_ue8m0_rejects(lib):
    f = lib.dg_pack_ue8m0_scales

    def call(sf=P16, per_block=0, packed=P16b, G=1, MN=256, K=512):
        return f(sf, per_block, packed, G, MN, K, None)

    assert call(K=200) == dg.DG_ERR_INVALID_ARG and "K=200" in err(lib)
    assert call(per_block=2) == dg.DG_ERR_INVALID_ARG and "per_block" in err(lib)
    assert call(sf=NULL) == dg.DG_ERR_INVALID_ARG and "sf is NULL" in err(lib)
    assert call(packed=ctypes.c_void_p(0x10002)) == dg.DG_ERR_INVALID_ARG
    assert call(packed=ctypes.c_void_p(0x10000 + 64)) == dg.DG_ERR_INVALID_ARG
    assert "overlap" in err(lib)
    assert call(MN=0, sf=NULL) == dg.DG_OK and call(K=0, sf=NULL) == dg.DG_OK


def test_layout_entry_points_reject(lib):
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
        f = getattr(lib, name)

        def call(a=P16, b=P16b, sfa=P16, sfb=P16, c=NULL, d=P16c, dt=dg.DG_BF16, M=128, N=256, K=512):
            return f(a, sfa, b, sfb, c, d, dt, M, N, K, None)

        assert call(K=300) == dg.DG_ERR_INVALID_ARG and "K=300" in err(lib)
        assert call(N=100) == dg.DG_ERR_INVALID_ARG and "N=100" in err(lib)
        assert call(dt=5) == dg.DG_ERR_INVALID_ARG and "d_dtype" in err(lib)
        assert call(sfb=BAD) == dg.DG_ERR_INVALID_ARG and "sfb" in err(lib)
        assert call(c=ctypes.c_void_p(0x30000 + 32)) == dg.DG_ERR_INVALID_ARG
        assert call(M=0, a=NULL) == dg.DG_OK
        st = call(M=100)       # M % 16 only matters when A is stored [K, M]
        if name == "dg_fp8_gemm_nn":
            assert st != dg.DG_ERR_INVALID_ARG
        else:
            assert st == dg.DG_ERR_INVALID_ARG and "M=100" in err(lib)
    g = lib.dg_m_grouped_fp8_gemm_nn_contiguous
    assert g(P16, P16, P16b, P16, P16, P16c, 200, 256, 512, 4, None) == dg.DG_ERR_INVALID_ARG
    assert "multiple of 128" in err(lib)
    assert g(P16, P16, P16b, P16, NULL, P16c, 256, 256, 512, 4, None) == dg.DG_ERR_INVALID_ARG
    assert g(P16, P16, P16b, P16, P16, P16c, 0, 256, 512, 4, None) == dg.DG_OK


def test_layout_config_names(lib):
    assert dg.kernel_config_name(dg.FORM_NN, 4096, 4096, 4096) == "nn_dense_bf16_256x256"
    assert dg.kernel_config_name(dg.FORM_TN, 256, 256, 512, True) == "tn_dense_f32_256x256"
    assert dg.kernel_config_name(dg.FORM_TT, 256, 256, 512) == "tt_dense_bf16_256x256"
    assert dg.kernel_config_name(dg.FORM_NN_CONTIGUOUS, 256, 256, 512) == "nn_contiguous_bf16_256x256"
    assert dg.kernel_config_name(dg.FORM_K_GROUPED, 256, 256, 512) == "tn_kgrouped_f32_256x256"


def test_mqa_logits_rejects(lib):
    f = lib.dg_fp8_mqa_logits

    def call(q=P16, kv=P16b, sf=P16, w=P16c, ks=P16, ke=P16, out=P16c, S=64, S_kv=256, H=64,
             D=128, clean=1):
        return f(q, kv, sf, w, ks, ke, out, S, S_kv, H, D, clean, None)

    assert call(D=64) == dg.DG_ERR_INVALID_ARG and "head_dim" in err(lib)
    assert call(H=48) == dg.DG_ERR_INVALID_ARG and "num_heads" in err(lib)
    assert call(clean=2) == dg.DG_ERR_INVALID_ARG and "clean_logits" in err(lib)
    assert call(q=BAD) == dg.DG_ERR_INVALID_ARG and "q is not 16-byte" in err(lib)
    assert call(ke=NULL) == dg.DG_ERR_INVALID_ARG and "ke is NULL" in err(lib)
    assert call(S=-1) == dg.DG_ERR_INVALID_ARG
    assert call(S=1048561) == dg.DG_ERR_INVALID_ARG and "seq_len" in err(lib)
    assert call(S_kv=2**31 - 4096) == dg.DG_ERR_INVALID_ARG and "seq_len_kv" in err(lib)
    assert call(S=0, q=NULL) == dg.DG_OK and call(S_kv=0, kv=NULL) == dg.DG_OK


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No fallback: with libdg.so absent, loading raises instead of running
    anything else."""
    monkeypatch.setattr(dg, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        dg.load_library(str(tmp_path / "libdg.so"))
    monkeypatch.setattr(dg, "LIB_PATH", str(tmp_path / "libdg.so"))
    with pytest.raises(ImportError):
        dg.load_library()



# ---- dense split-K workspace: caller-owned, queried by shape ---------------------

DECODE_SHAPES = [(m, n, k) for m in (1, 16, 64, 65, 128) for (n, k) in
                 ((2112, 7168), (24576, 1536), (7168, 16384), (4096, 7168), (7168, 2048))]


def test_workspace_query_is_a_pure_function_of_the_shape(lib):
    """No device is needed to size the workspace, large problems need none,
    decode-size problems do, and no shape needs more than the documented
    32 MiB + 1 KiB."""
    q = lib.dg_fp8_gemm_nt_workspace_bytes
    assert q(4096, 7168, 16384) == 0 and q(4096, 2112, 7168) == 0
    assert q(64, 7168, 16384) > 0 and q(128, 2112, 7168) > 0
    assert q(0, 256, 512) == 0 and q(64, 250, 512) == 0 and q(64, 256, 500) == 0
    assert q(64, 7168, 512) == 0          # too few K blocks to split
    worst = 0
    for M in (1, 16, 64, 65, 128, 129, 200, 256, 300, 512, 1024):
        for N in (16, 256, 1024, 2112, 4096, 7168, 24576):
            for K in (1024, 2048, 7168, 16384):
                worst = max(worst, q(M, N, K))
    assert 0 < worst <= 32 * 2**20 + 1024
    assert all(q(*s) == dg.get_fp8_gemm_nt_workspace_bytes(*s) for s in DECODE_SHAPES)


def test_split_shape_needs_the_caller_workspace(lib):
    M, N, K = 64, 7168, 16384
    need = lib.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    assert need > 0
    a, b, d, ws = (ctypes.c_void_p(x) for x in (0x1000000, 0x10000000, 0x40000000, 0x50000000))
    sfa = sfb = ctypes.c_void_p(0x60000000)
    assert nt(lib, a=a, sfa=sfa, b=b, sfb=sfb, d=d, M=M, N=N, K=K) == dg.DG_ERR_INVALID_ARG
    assert "needs a workspace" in err(lib)
    assert nt(lib, a=a, sfa=sfa, b=b, sfb=sfb, d=d, M=M, N=N, K=K, ws=ws,
              ws_bytes=need - 16) == dg.DG_ERR_INVALID_ARG
    assert "needed" in err(lib)
    assert nt(lib, a=a, sfa=sfa, b=b, sfb=sfb, d=d, M=M, N=N, K=K, ws=ctypes.c_void_p(0x50000008),
              ws_bytes=need) == dg.DG_ERR_INVALID_ARG
    assert "workspace is not 16-byte" in err(lib)
    # overlapping the output (d spans M * N * 2 bytes from 0x40000000)
    assert nt(lib, a=a, sfa=sfa, b=b, sfb=sfb, d=d, M=M, N=N, K=K, ws=ctypes.c_void_p(0x40000000 + 256),
              ws_bytes=need) == dg.DG_ERR_INVALID_ARG
    assert "overlaps" in err(lib)
    # with an adequate workspace validation passes; without a GPU the device query fails cleanly
    st = nt(lib, a=a, sfa=sfa, b=b, sfb=sfb, d=d, M=M, N=N, K=K, ws=ws, ws_bytes=need)
    assert st in (dg.DG_ERR_HIP, dg.DG_ERR_UNSUPPORTED, dg.DG_OK)


def test_library_sources_never_allocate_or_synchronise():
    """Every GEMM entry point enqueues its kernel and returns: no HIP
    allocation, free, memset, blocking copy or synchronisation is reachable
    from the library's sources."""
    csrc = os.path.join(ROOT, "fp8_fine_grained_e4m3_amd", "csrc")
    banned = re.compile(r"\bhip(Malloc\w*|Free\w*|HostMalloc|HostRegister|MallocAsync|Memset\w*|"
                        r"Memcpy\w*|StreamSynchronize|DeviceSynchronize|EventSynchronize)\s*\(")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".cpp", ".h")):
            text = open(os.path.join(csrc, fn)).read()
            hits = banned.findall(text)
            assert not hits, (fn, hits)
