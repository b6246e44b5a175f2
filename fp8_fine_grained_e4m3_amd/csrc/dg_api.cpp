// C-ABI layer: argument validation (before any HIP call), device checks,
// CU-count cap, error reporting, and dispatch to the kernels.
#include "../../include/dg.h"
#include "dg_internal.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

dg_status fail(dg_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

dg_status ok() {
    g_last_error.clear();
    return DG_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// c must be NULL, equal to d, or not overlap [d, d + bytes).
bool alias_ok(const void* c, const void* d, int64_t bytes) {
    if (c == nullptr || c == d) return true;
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(c), d0 = reinterpret_cast<uintptr_t>(d);
    return c0 + (uintptr_t)bytes <= d0 || d0 + (uintptr_t)bytes <= c0;
}

#define REQUIRE(cond, ...)                                   \
    do {                                                     \
        if (!(cond)) return fail(DG_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p, align)                                                         \
    do {                                                                              \
        if ((p) == nullptr) return fail(DG_ERR_INVALID_ARG, "%s is NULL", #p);        \
        if (!aligned((p), (align)))                                                   \
            return fail(DG_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, (int)(align)); \
    } while (0)

constexpr int64_t kOffsetLimit = INT_MAX;   // kernels index one matrix with 32-bit offsets

// ---- device state -------------------------------------------------------------

constexpr int kMaxDevices = 64;
struct DeviceInfo {
    bool probed = false;
    bool gfx950 = false;
    int cus = 0;
    char arch[64] = {0};
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mutex;
std::atomic<int> g_cu_cap{0};   // 0 = use every CU; process-wide, set from any thread

dg_status current_device(int& dev, DeviceInfo& info) {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceInfo& d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(DG_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
        d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        d.probed = true;
    }
    info = d;
    if (!info.gfx950)
        return fail(DG_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                    info.arch);
    return DG_OK;
}

int cu_cap_for(const DeviceInfo& info) {
    const int cap = g_cu_cap.load(std::memory_order_relaxed);
    return (cap > 0 && cap < info.cus) ? cap : info.cus;
}

bool print_configs() {
    // read once; the initialisation of a function-local static is thread-safe
    static const bool v = [] {
        const char* s = getenv("DG_PRINT_CONFIGS");
        return s != nullptr && s[0] == '1';
    }();
    return v;
}

dg_status run_tn(const dg::TnProblem& p, void* stream) {
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    if (print_configs()) fprintf(stderr, "[dg] %s\n", dg::describe_tn_config(p));
    hipError_t e = dg::launch_tn(p, cu_cap_for(info), reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

dg_status run_nt(dg::NtProblem p, void* stream) {
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    if (print_configs()) fprintf(stderr, "[dg] %s\n", dg::describe_nt_config(p));
    hipError_t e = dg::launch_nt(p, cu_cap_for(info), reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

// [p0, p0 + n0) and [p1, p1 + n1) do not overlap
bool disjoint(const void* p0, int64_t n0, const void* p1, int64_t n1) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p0), a1 = reinterpret_cast<uintptr_t>(p1);
    return a0 + (uintptr_t)n0 <= a1 || a1 + (uintptr_t)n1 <= a0;
}

// The three NT forms take either fp32 scales or packed UE8M0 words; both are
// 4-byte elements, passed through as raw pointers.
// noalloc: the split-K workspace is the library's static scratch instead of
// the caller's (workspace / workspace_bytes are ignored).
dg_status gemm_nt(const uint8_t* a, const void* sfa_, const uint8_t* b, const void* sfb_,
                  const void* c, void* d, dg_dtype d_dtype, int64_t M, int64_t N, int64_t K,
                  void* workspace, int64_t workspace_bytes, bool ue8m0, void* stream,
                  bool noalloc = false) {
    const float* sfa = static_cast<const float*>(sfa_);
    const float* sfb = static_cast<const float*>(sfb_);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
            (long long)N, (long long)K);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    REQUIRE(d_dtype == DG_BF16 || d_dtype == DG_F32, "d_dtype must be DG_BF16 or DG_F32");
    if (M == 0 || N == 0) return ok();
    REQUIRE_PTR(d, 16);
    if (c) REQUIRE_PTR(c, 16);
    if (K > 0) {   // with K == 0 the operands are empty: D = C (or 0)
        REQUIRE_PTR(a, 16);
        REQUIRE_PTR(b, 16);
        REQUIRE_PTR(sfa, 16);
        REQUIRE_PTR(sfb, 16);
    }
    REQUIRE(M <= kOffsetLimit / (K > 0 ? K : 1) && N <= kOffsetLimit / (K > 0 ? K : 1),
            "M*K and N*K must stay below 2^31");
    REQUIRE(M <= INT_MAX && N <= INT_MAX, "size too large");
    // work units: 64 x 64 tiles (the smallest) times up to 8 K splits
    REQUIRE(((M + 63) / 64) * ((N + 63) / 64) <= INT_MAX / 8, "too many tiles");
    const int64_t dbytes = M * N * (d_dtype == DG_F32 ? 4 : 2);
    REQUIRE(alias_ok(c, d, dbytes), "c overlaps d without being equal to it");
    const int64_t need = dg::nt_dense_workspace_bytes(M, N, K);
    if (noalloc) {
        if (need > dg::nt_noalloc_scratch_bytes())
            return fail(DG_ERR_UNSUPPORTED,
                        "this shape needs %lld bytes of split-K scratch; the static scratch "
                        "holds %lld", (long long)need, (long long)dg::nt_noalloc_scratch_bytes());
        workspace = nullptr;
        workspace_bytes = 0;
    }
    REQUIRE(workspace_bytes >= 0, "workspace_bytes=%lld is negative", (long long)workspace_bytes);
    if (need > 0 && !noalloc) {
        REQUIRE(workspace != nullptr,
                "this shape splits K and needs a workspace of %lld bytes "
                "(dg_fp8_gemm_nt_workspace_bytes); workspace is NULL", (long long)need);
        REQUIRE_PTR(workspace, 16);
        REQUIRE(workspace_bytes >= need, "workspace_bytes=%lld < %lld needed for this shape",
                (long long)workspace_bytes, (long long)need);
        const int64_t KB = K / 128, sf_w = ue8m0 ? (KB + 3) / 4 : KB;
        const int64_t sfb_n = ue8m0 ? sf_w * N : ((N + 127) / 128) * KB;
        REQUIRE(disjoint(workspace, need, d, dbytes) && (c == nullptr || disjoint(workspace, need, c, dbytes)) &&
                    disjoint(workspace, need, a, M * K) && disjoint(workspace, need, b, N * K) &&
                    disjoint(workspace, need, sfa, 4 * sf_w * M) && disjoint(workspace, need, sfb, 4 * sfb_n),
                "workspace overlaps an operand or the output");
    }
    dg::NtProblem p{};
    p.form = dg::kDense;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.c = c; p.d = d;
    p.rows = M; p.N = N; p.K = K; p.G = 1;
    p.out_f32 = d_dtype == DG_F32;
    p.ue8m0 = ue8m0;
    if (noalloc && need > 0) {
        // after host validation: the device check, then this device's scratch
        int dev = 0;
        DeviceInfo info;
        dg_status st = current_device(dev, info);
        if (st != DG_OK) return st;
        hipError_t e = dg::nt_noalloc_scratch(&workspace);
        if (e != hipSuccess)
            return fail(DG_ERR_HIP, "static scratch lookup: %s", hipGetErrorString(e));
        workspace_bytes = dg::nt_noalloc_scratch_bytes();
    }
    p.workspace = need > 0 ? workspace : nullptr;
    p.workspace_bytes = need > 0 ? workspace_bytes : 0;
    return run_nt(p, stream);
}

dg_status gemm_nt_contiguous(const uint8_t* a, const void* sfa_, const uint8_t* b,
                             const void* sfb_, const int32_t* m_indices, void* d, int64_t M_tot,
                             int64_t N, int64_t K, int64_t G, bool ue8m0, void* stream) {
    const float* sfa = static_cast<const float*>(sfa_);
    const float* sfb = static_cast<const float*>(sfb_);
    REQUIRE(M_tot >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(G >= 1, "G=%lld must be >= 1", (long long)G);
    REQUIRE(M_tot % 128 == 0, "M_tot=%lld is not a multiple of 128 (the contiguous-layout alignment)",
            (long long)M_tot);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    if (M_tot == 0 || N == 0) return ok();
    REQUIRE_PTR(a, 16);
    REQUIRE_PTR(b, 16);
    REQUIRE_PTR(d, 16);
    REQUIRE_PTR(sfa, 16);
    REQUIRE_PTR(sfb, 16);
    REQUIRE_PTR(m_indices, 16);
    REQUIRE(M_tot <= kOffsetLimit / (K > 0 ? K : 1) && N <= kOffsetLimit / (K > 0 ? K : 1),
            "M_tot*K and N*K must stay below 2^31");
    REQUIRE(G <= INT_MAX, "G too large");
    dg::NtProblem p{};
    p.form = dg::kContiguous;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.c = nullptr; p.d = d;
    p.m_indices = m_indices;
    p.rows = M_tot; p.N = N; p.K = K; p.G = G;
    p.out_f32 = false;
    p.ue8m0 = ue8m0;
    return run_nt(p, stream);
}

dg_status gemm_nt_masked(const uint8_t* a, const void* sfa_, const uint8_t* b, const void* sfb_,
                         const int32_t* masked_m, void* d, int64_t G, int64_t M_max, int64_t N,
                         int64_t K, bool ue8m0, void* stream) {
    const float* sfa = static_cast<const float*>(sfa_);
    const float* sfb = static_cast<const float*>(sfb_);
    REQUIRE(G >= 0 && M_max >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    if (G == 0 || M_max == 0 || N == 0) return ok();
    REQUIRE_PTR(a, 16);
    REQUIRE_PTR(b, 16);
    REQUIRE_PTR(d, 16);
    REQUIRE_PTR(sfa, 16);
    REQUIRE_PTR(sfb, 16);
    REQUIRE_PTR(masked_m, 16);
    REQUIRE(M_max <= kOffsetLimit / (K > 0 ? K : 1) && N <= kOffsetLimit / (K > 0 ? K : 1),
            "M_max*K and N*K must stay below 2^31");
    // bound for the smallest tile (64 x 64) any configuration uses (G first, so
    // the product below cannot overflow)
    REQUIRE(G <= INT_MAX, "G too large");
    REQUIRE(G * ((M_max + 63) / 64) * ((N + 63) / 64) <= INT_MAX, "too many tiles");
    dg::NtProblem p{};
    p.form = dg::kMasked;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.c = nullptr; p.d = d;
    p.masked_m = masked_m;
    p.rows = M_max; p.N = N; p.K = K; p.G = G;
    p.out_f32 = false;
    p.ue8m0 = ue8m0;
    return run_nt(p, stream);
}

}  // namespace

extern "C" {

dg_status dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype, int64_t M, int64_t N,
                         int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
    return gemm_nt(a, sfa, b, sfb, c, d, d_dtype, M, N, K, workspace, workspace_bytes, false,
                   stream);
}

dg_status dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b,
                                 const float* sfb, const void* c, void* d, dg_dtype d_dtype,
                                 int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_nt(a, sfa, b, sfb, c, d, d_dtype, M, N, K, nullptr, 0, false, stream, true);
}

int64_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || N % 16 != 0) return 0;
    if (M > kOffsetLimit / K || N > kOffsetLimit / K) return 0;
    return dg::nt_dense_workspace_bytes(M, N, K);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* m_indices, void* d, int64_t M_tot,
                                              int64_t N, int64_t K, int64_t G, void* stream) {
    return gemm_nt_contiguous(a, sfa, b, sfb, m_indices, d, M_tot, N, K, G, false, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                          const float* sfb, const int32_t* masked_m, void* d,
                                          int64_t G, int64_t M_max, int64_t N, int64_t K,
                                          void* stream) {
    return gemm_nt_masked(a, sfa, b, sfb, masked_m, d, G, M_max, N, K, false, stream);
}

dg_status dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                               const int32_t* sfb, const void* c, void* d, dg_dtype d_dtype,
                               int64_t M, int64_t N, int64_t K, void* workspace,
                               int64_t workspace_bytes, void* stream) {
    return gemm_nt(a, sfa, b, sfb, c, d, d_dtype, M, N, K, workspace, workspace_bytes, true,
                   stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                    const uint8_t* b, const int32_t* sfb,
                                                    const int32_t* m_indices, void* d,
                                                    int64_t M_tot, int64_t N, int64_t K,
                                                    int64_t G, void* stream) {
    return gemm_nt_contiguous(a, sfa, b, sfb, m_indices, d, M_tot, N, K, G, true, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                const uint8_t* b, const int32_t* sfb,
                                                const int32_t* masked_m, void* d, int64_t G,
                                                int64_t M_max, int64_t N, int64_t K,
                                                void* stream) {
    return gemm_nt_masked(a, sfa, b, sfb, masked_m, d, G, M_max, N, K, true, stream);
}

dg_status dg_pack_ue8m0_scales(const float* sf, int per_block, int32_t* packed, int64_t G,
                               int64_t MN, int64_t K, void* stream) {
    REQUIRE(G >= 0 && MN >= 0 && K >= 0, "negative size (G=%lld MN=%lld K=%lld)", (long long)G,
            (long long)MN, (long long)K);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(per_block == 0 || per_block == 1, "per_block must be 0 or 1");
    if (G == 0 || MN == 0 || K == 0) return ok();
    REQUIRE_PTR(sf, 16);
    REQUIRE_PTR(packed, 16);
    const int64_t kb = K / 128, k4 = (kb + 3) / 4;
    REQUIRE(MN <= INT_MAX && G <= kOffsetLimit / k4 && G * k4 <= kOffsetLimit / MN,
            "G*ceil(K/512)*MN must stay below 2^31");
    const int64_t sf_count = per_block ? G * ((MN + 127) / 128) * kb : G * kb * MN;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(sf), p0 = reinterpret_cast<uintptr_t>(packed);
    REQUIRE(s0 + (uintptr_t)(sf_count * 4) <= p0 || p0 + (uintptr_t)(G * k4 * MN * 4) <= s0,
            "sf and packed must not overlap");
    dg::PackProblem p{};
    p.sf = sf; p.per_block = per_block != 0; p.packed = packed;
    p.G = G; p.MN = MN; p.KB = kb;
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    hipError_t e = dg::launch_pack_ue8m0(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

static dg_status k_grouped_tn(const uint8_t* a, const void* sfa, const uint8_t* b,
                              const void* sfb, const int32_t* k_sizes_host, const float* c,
                              float* d, int64_t G, int64_t M, int64_t N, int64_t K_tot,
                              bool ue8m0, void* stream);

dg_status dg_k_grouped_fp8_gemm_tn_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* k_sizes_host, const float* c,
                                              float* d, int64_t G, int64_t M, int64_t N,
                                              int64_t K_tot, void* stream) {
    return k_grouped_tn(a, sfa, b, sfb, k_sizes_host, c, d, G, M, N, K_tot, false, stream);
}

dg_status dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                    const uint8_t* b, const int32_t* sfb,
                                                    const int32_t* k_sizes_host, const float* c,
                                                    float* d, int64_t G, int64_t M, int64_t N,
                                                    int64_t K_tot, void* stream) {
    return k_grouped_tn(a, sfa, b, sfb, k_sizes_host, c, d, G, M, N, K_tot, true, stream);
}

dg_status dg_pack_ue8m0_scales_k_grouped(const float* sf, const int32_t* k_sizes_host,
                                         int32_t* packed, int64_t G, int64_t MN, int64_t K_tot,
                                         void* stream) {
    REQUIRE(G >= 1 && G <= dg::kMaxTnGroups, "G=%lld must be in [1, %d]", (long long)G,
            dg::kMaxTnGroups);
    REQUIRE(MN >= 0 && K_tot >= 0, "negative size");
    REQUIRE(k_sizes_host != nullptr, "k_sizes_host is NULL");
    int64_t total = 0, words = 0;
    for (int64_t g = 0; g < G; ++g) {
        const int64_t kg = k_sizes_host[g];
        REQUIRE(kg >= 0 && kg % 128 == 0, "k_sizes_host[%lld]=%lld must be >= 0 and a multiple of 128",
                (long long)g, (long long)kg);
        total += kg;
        words += (kg / 128 + 3) / 4;
    }
    REQUIRE(total == K_tot, "sum of k_sizes_host (%lld) != K_tot (%lld)", (long long)total,
            (long long)K_tot);
    if (MN == 0 || words == 0) return ok();
    REQUIRE_PTR(sf, 16);
    REQUIRE_PTR(packed, 16);
    // the kernel's 32-bit column index runs up to one 256-thread block past MN
    REQUIRE(MN <= INT_MAX - 256, "MN=%lld too large", (long long)MN);
    REQUIRE(words <= 65535, "too many packed word rows");
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(sf), p0 = reinterpret_cast<uintptr_t>(packed);
    REQUIRE(s0 + (uintptr_t)((K_tot / 128) * MN * 4) <= p0 || p0 + (uintptr_t)(words * MN * 4) <= s0,
            "sf and packed must not overlap");
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    hipError_t e = dg::launch_pack_ue8m0_k_grouped(sf, k_sizes_host, G, MN, packed,
                                                   reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

static dg_status k_grouped_tn(const uint8_t* a, const void* sfa_, const uint8_t* b,
                              const void* sfb_, const int32_t* k_sizes_host, const float* c,
                              float* d, int64_t G, int64_t M, int64_t N, int64_t K_tot,
                              bool ue8m0, void* stream) {
    const float* sfa = static_cast<const float*>(sfa_);
    const float* sfb = static_cast<const float*>(sfb_);
    REQUIRE(M >= 0 && N >= 0 && K_tot >= 0, "negative size");
    REQUIRE(G >= 1 && G <= dg::kMaxTnGroups, "G=%lld must be in [1, %d]", (long long)G,
            dg::kMaxTnGroups);
    REQUIRE(M % 16 == 0, "M=%lld is not a multiple of 16", (long long)M);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    REQUIRE(k_sizes_host != nullptr, "k_sizes_host is NULL");
    int64_t total = 0;
    for (int64_t g = 0; g < G; ++g) {
        const int64_t kg = k_sizes_host[g];
        REQUIRE(kg >= 0 && kg % 128 == 0, "k_sizes_host[%lld]=%lld must be >= 0 and a multiple of 128",
                (long long)g, (long long)kg);
        total += kg;
    }
    REQUIRE(total == K_tot, "sum of k_sizes_host (%lld) != K_tot (%lld)", (long long)total,
            (long long)K_tot);
    if (M == 0 || N == 0) return ok();
    REQUIRE_PTR(d, 16);
    if (c) REQUIRE_PTR(c, 16);
    if (K_tot > 0) {
        REQUIRE_PTR(a, 16);
        REQUIRE_PTR(b, 16);
        REQUIRE_PTR(sfa, 16);
        REQUIRE_PTR(sfb, 16);
    }
    REQUIRE(K_tot <= kOffsetLimit / M && K_tot <= kOffsetLimit / N,
            "K_tot*M and K_tot*N must stay below 2^31");
    REQUIRE(G * ((M + 127) / 128) * ((N + 127) / 128) <= INT_MAX, "too many tiles");
    REQUIRE(alias_ok(c, d, G * M * N * 4), "c overlaps d without being equal to it");
    dg::TnProblem p{};
    p.form = dg::kKGrouped;
    p.a_mk = false; p.b_nk = false; p.out_f32 = true; p.ue8m0 = ue8m0;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.k_sizes_host = k_sizes_host;
    p.c = c; p.d = d; p.G = G; p.M = M; p.N = N; p.K_tot = K_tot;
    return run_tn(p, stream);
}

// Dense NN / TN / TT: A stored [M, K] (a_mk) or [K, M]; B stored [N, K] (b_nk)
// or [K, N]; sfa [K/128, M], sfb [K/128, N]; C like D (may equal it).
static dg_status gemm_layout(const uint8_t* a, bool a_mk, const float* sfa, const uint8_t* b,
                             bool b_nk, const float* sfb, const void* c, void* d,
                             dg_dtype d_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
            (long long)N, (long long)K);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    REQUIRE(a_mk || M % 16 == 0, "M=%lld is not a multiple of 16 (A stored [K, M])", (long long)M);
    REQUIRE(d_dtype == DG_BF16 || d_dtype == DG_F32, "d_dtype must be DG_BF16 or DG_F32");
    if (M == 0 || N == 0) return ok();
    REQUIRE_PTR(d, 16);
    if (c) REQUIRE_PTR(c, 16);
    if (K > 0) {
        REQUIRE_PTR(a, 16);
        REQUIRE_PTR(b, 16);
        REQUIRE_PTR(sfa, 16);
        REQUIRE_PTR(sfb, 16);
    }
    REQUIRE(M <= kOffsetLimit / (K > 0 ? K : 1) && N <= kOffsetLimit / (K > 0 ? K : 1),
            "M*K and N*K must stay below 2^31");
    REQUIRE(((M + 127) / 128) * ((N + 127) / 128) <= INT_MAX, "too many tiles");
    REQUIRE(alias_ok(c, d, M * N * (d_dtype == DG_F32 ? 4 : 2)),
            "c overlaps d without being equal to it");
    dg::TnProblem p{};
    p.form = dg::kDenseLayout;
    p.a_mk = a_mk; p.b_nk = b_nk; p.out_f32 = d_dtype == DG_F32;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.c = c; p.d = d;
    p.G = 1; p.M = M; p.N = N; p.K_tot = K;
    return run_tn(p, stream);
}

dg_status dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype, int64_t M, int64_t N,
                         int64_t K, void* stream) {
    return gemm_layout(a, true, sfa, b, false, sfb, c, d, d_dtype, M, N, K, stream);
}

dg_status dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype, int64_t M, int64_t N,
                         int64_t K, void* stream) {
    return gemm_layout(a, false, sfa, b, false, sfb, c, d, d_dtype, M, N, K, stream);
}

dg_status dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype, int64_t M, int64_t N,
                         int64_t K, void* stream) {
    return gemm_layout(a, false, sfa, b, true, sfb, c, d, d_dtype, M, N, K, stream);
}

dg_status dg_m_grouped_fp8_gemm_nn_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* m_indices, void* d, int64_t M_tot,
                                              int64_t N, int64_t K, int64_t G, void* stream) {
    REQUIRE(M_tot >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(G >= 1, "G=%lld must be >= 1", (long long)G);
    REQUIRE(M_tot % 128 == 0, "M_tot=%lld is not a multiple of 128 (the contiguous-layout alignment)",
            (long long)M_tot);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(N % 16 == 0, "N=%lld is not a multiple of 16", (long long)N);
    if (M_tot == 0 || N == 0) return ok();
    REQUIRE_PTR(a, 16);
    REQUIRE_PTR(b, 16);
    REQUIRE_PTR(d, 16);
    REQUIRE_PTR(sfa, 16);
    REQUIRE_PTR(sfb, 16);
    REQUIRE_PTR(m_indices, 16);
    REQUIRE(M_tot <= kOffsetLimit / (K > 0 ? K : 1) && N <= kOffsetLimit / (K > 0 ? K : 1),
            "M_tot*K and K*N must stay below 2^31");
    REQUIRE(G <= INT_MAX && (M_tot / 128) * ((N + 255) / 256) <= INT_MAX, "too many tiles");
    dg::TnProblem p{};
    p.form = dg::kMGroupedNN;
    p.a_mk = true; p.b_nk = false; p.out_f32 = false;
    p.a = a; p.sfa = sfa; p.b = b; p.sfb = sfb; p.m_indices = m_indices; p.c = nullptr; p.d = d;
    p.G = G; p.M = M_tot; p.N = N; p.K_tot = K;
    return run_tn(p, stream);
}

static dg_status run_cast(const void* x, dg_dtype dtype, uint8_t* codes, float* sf, int64_t G,
                          int64_t R, int64_t K, int flags, bool block_scale, void* stream) {
    REQUIRE(G >= 0 && R >= 0 && K >= 0, "negative size (G=%lld rows=%lld K=%lld)", (long long)G,
            (long long)R, (long long)K);
    REQUIRE(K % 128 == 0, "K=%lld is not a multiple of 128", (long long)K);
    REQUIRE(dtype == DG_BF16 || dtype == DG_F32, "input dtype must be DG_BF16 or DG_F32");
    REQUIRE(flags == 0 || flags == DG_CAST_POW2_SCALE, "flags must be 0 or DG_CAST_POW2_SCALE");
    if (G == 0 || R == 0 || K == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(codes, 16);
    REQUIRE_PTR(sf, 16);
    REQUIRE(R <= kOffsetLimit && K <= kOffsetLimit, "size too large");
    REQUIRE(G <= kOffsetLimit && R <= kOffsetLimit / K, "rows*K must stay below 2^31");
    const int64_t n = G * R * K;   // < 2^62
    const int64_t in_bytes = n * (dtype == DG_F32 ? 4 : 2);
    const int64_t kb = K / 128;
    const int64_t sf_count = block_scale ? G * ((R + 127) / 128) * kb : G * kb * R;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), c0 = reinterpret_cast<uintptr_t>(codes),
                    s0 = reinterpret_cast<uintptr_t>(sf);
    auto disjoint = [](uintptr_t a, int64_t na, uintptr_t b, int64_t nb) {
        return a + (uintptr_t)na <= b || b + (uintptr_t)nb <= a;
    };
    REQUIRE(disjoint(x0, in_bytes, c0, n) && disjoint(x0, in_bytes, s0, sf_count * 4) &&
                disjoint(c0, n, s0, sf_count * 4),
            "input, codes and sf must not overlap");
    dg::CastProblem p{};
    p.x = x; p.in_f32 = dtype == DG_F32; p.block_scale = block_scale;
    p.pow2 = flags == DG_CAST_POW2_SCALE;
    p.codes = codes; p.sf = sf; p.G = G; p.R = R; p.K = K;
    REQUIRE(dg::cast_grid(p) <= INT_MAX, "too many blocks");
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    hipError_t e = dg::launch_cast(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

dg_status dg_per_token_cast_to_fp8(const void* x, dg_dtype x_dtype, uint8_t* codes, float* sf,
                                   int64_t G, int64_t R, int64_t K, int flags, void* stream) {
    return run_cast(x, x_dtype, codes, sf, G, R, K, flags, false, stream);
}

dg_status dg_per_block_cast_to_fp8(const void* w, dg_dtype w_dtype, uint8_t* codes, float* sf,
                                   int64_t G, int64_t N, int64_t K, int flags, void* stream) {
    return run_cast(w, w_dtype, codes, sf, G, N, K, flags, true, stream);
}

dg_status dg_fp8_mqa_logits(const uint8_t* q, const uint8_t* kv, const float* kv_sf,
                            const float* weights, const int32_t* ks, const int32_t* ke,
                            float* logits, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                            int clean_logits, void* stream) {
    REQUIRE(S >= 0 && S_kv >= 0, "negative size (seq_len=%lld seq_len_kv=%lld)", (long long)S,
            (long long)S_kv);
    REQUIRE(D == 128, "head_dim=%lld: only 128 is supported (one MFMA K step)", (long long)D);
    REQUIRE(H == 16 || H == 32 || H == 64, "num_heads=%lld must be 16, 32 or 64", (long long)H);
    REQUIRE(clean_logits == 0 || clean_logits == 1, "clean_logits must be 0 or 1");
    if (S == 0 || S_kv == 0) return ok();
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(kv, 16);
    REQUIRE_PTR(weights, 16);
    REQUIRE_PTR(logits, 16);
    REQUIRE_PTR(kv_sf, 16);
    REQUIRE_PTR(ks, 16);
    REQUIRE_PTR(ke, 16);
    // token indices are 32-bit and run up to one workgroup (256 tokens) past S_kv
    REQUIRE(S <= 65535LL * 16 && S_kv <= INT_MAX - 4096,
            "seq_len must be <= 1048560 and seq_len_kv <= 2^31 - 4097");
    dg::MqaProblem p{};
    p.q = q; p.kv = kv; p.kv_sf = kv_sf; p.weights = weights; p.ks = ks; p.ke = ke;
    p.logits = logits; p.S = S; p.S_kv = S_kv; p.H = H; p.clean = clean_logits != 0;
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    hipError_t e = dg::launch_mqa(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

const char* dg_last_error(void) { return g_last_error.c_str(); }

int dg_get_num_cus(void) {
    int dev = 0;
    DeviceInfo info;
    if (current_device(dev, info) != DG_OK && !info.probed) return 0;
    return cu_cap_for(info);
}

dg_status dg_set_num_cus(int n) {
    if (n == 0) {
        g_cu_cap.store(0, std::memory_order_relaxed);
        return ok();
    }
    int dev = 0;
    DeviceInfo info;
    dg_status st = current_device(dev, info);
    if (st != DG_OK) return st;
    if (n < 0 || n > info.cus)
        return fail(DG_ERR_INVALID_ARG, "num_cus=%d must be in [1, %d] (or 0 for all)", n, info.cus);
    g_cu_cap.store(n, std::memory_order_relaxed);
    return ok();
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

const char* dg_kernel_config_name(int form, int64_t rows, int64_t N, int64_t K, int out_f32) {
    if (form >= 0 && form <= 2) {
        dg::NtProblem p{};
        p.form = static_cast<dg::NtForm>(form);
        p.rows = rows; p.N = N; p.K = K; p.G = 1;
        p.out_f32 = form == 0 && out_f32 != 0;
        return dg::nt_config_name(p);
    }
    if (form >= 3 && form <= 7) {
        dg::TnProblem p{};
        p.M = rows; p.N = N; p.K_tot = K; p.G = 1;
        p.out_f32 = out_f32 != 0;
        p.form = form == 3 ? dg::kKGrouped : (form == 7 ? dg::kMGroupedNN : dg::kDenseLayout);
        p.a_mk = form == 4;           // 4 NN, 5 TN, 6 TT
        p.b_nk = form == 6;
        return dg::tn_config_name(p);
    }
    return "";
}

}  // extern "C"
