// Internal interface between the C-ABI layer (dg_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Which M-axis scheduling the NT kernel uses.
enum NtForm : int { kDense = 0, kContiguous = 1, kMasked = 2 };

struct NtProblem {
    NtForm form;
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    const void* c;            // dense only, same dtype as d, may be NULL
    void* d;
    const int32_t* m_indices; // contiguous
    const int32_t* masked_m;  // masked
    int64_t rows;             // dense: M, contiguous: M_tot, masked: M_max
    int64_t N, K, G;
    bool out_f32;
    // false: fp32 scales, sfa [KB, rows] (masked: per group), sfb [G, ceil(N/128), KB].
    // true: packed UE8M0 words (int32; byte i of word k4 = exponent of K block
    // 4 k4 + i), sfa [K4, rows] (masked: [G, K4, M_max]), sfb [G, K4, N],
    // K4 = ceil(KB / 4).
    bool ue8m0;
    // Dense only: caller-owned split-K workspace (nt_dense_workspace_bytes;
    // NULL / 0 when that is 0).
    void* workspace;
    int64_t workspace_bytes;
};

// Bytes of split-K workspace a dense NT problem needs (0: K is not split).
// A function of the shape alone: no device query, no HIP call.
int64_t nt_dense_workspace_bytes(int64_t M, int64_t N, int64_t K);

// The library's static split-K scratch (for callers that cannot allocate):
// its capacity in bytes (host constant) and its device address on the current
// device (looked up once per device; a HIP call).
int64_t nt_noalloc_scratch_bytes();
hipError_t nt_noalloc_scratch(void** ptr);

// MN-major kernel family: the K-grouped TN form, the dense NN / TN / TT
// layouts and the M-grouped contiguous NN form.  Both operands carry one fp32
// scale per output row (m) / column (n) per 128-K block: sfa [KB, M],
// sfb [KB, N] (grouped NN: sfb [G, KB, N]).
enum TnForm : int { kKGrouped = 0, kDenseLayout = 1, kMGroupedNN = 2 };

struct TnProblem {
    TnForm form;
    bool a_mk;      // A stored [M, K] (K contiguous), else [K, M]
    bool b_nk;      // B stored [N, K] (K contiguous), else [K, N] (grouped NN: [G, K, N])
    bool out_f32;   // D (and C) fp32, else bf16
    bool ue8m0;     // K-grouped: packed UE8M0 scales, each group on its own word rows
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    const int32_t* k_sizes_host;   // K-grouped
    const int32_t* m_indices;      // M-grouped NN
    const void* c;
    void* d;
    int64_t G, M, N, K_tot;        // dense / grouped NN: G = experts (1 dense), K_tot = K
};

constexpr int kMaxTnGroups = 256;

// FP8 casting: x [G, R, K] (bf16 bits or fp32) -> codes [G, R, K] and either
// per-token scales sf [G, K/128, R] or per-block scales sf [G, ceil(R/128), K/128].
struct CastProblem {
    const void* x;
    bool in_f32;
    bool block_scale;   // false: 1 x 128 (per token), true: 128 x 128 (per block)
    bool pow2;          // round each scale up to a power of two
    uint8_t* codes;
    float* sf;
    int64_t G, R, K;
};

// fp32 power-of-two scales -> packed UE8M0 words packed [G, ceil(KB/4), MN]:
// per_block false: sf [G, KB, MN] (one scale per row and K block, MN-major);
// true: sf [G, ceil(MN/128), KB] (one per 128 x 128 block, given to each of
// its rows).
struct PackProblem {
    const float* sf;
    bool per_block;
    int32_t* packed;
    int64_t G, MN, KB;
};
hipError_t launch_pack_ue8m0(const PackProblem& p, hipStream_t stream);
// K-grouped: sf [K_tot/128, MN] -> packed [sum_g ceil(KB_g / 4), MN], each
// group's blocks on their own word rows.
hipError_t launch_pack_ue8m0_k_grouped(const float* sf, const int32_t* k_sizes_host, int64_t G,
                                       int64_t MN, int32_t* packed, hipStream_t stream);

// MQA logits: q e4m3 [S, H, 128], kv e4m3 [S_kv, 128], kv_sf [S_kv],
// weights [S, H], ks / ke [S] -> logits fp32 [S, S_kv].
struct MqaProblem {
    const uint8_t* q;
    const uint8_t* kv;
    const float* kv_sf;
    const float* weights;
    const int32_t* ks;
    const int32_t* ke;
    float* logits;
    int64_t S, S_kv, H;
    bool clean;
};
hipError_t launch_mqa(const MqaProblem& p, hipStream_t stream);

// Launch on `stream`; `cu_cap` bounds the persistent grid.  Return the HIP
// status of the launch.  Shapes have already been validated.
hipError_t launch_nt(const NtProblem& p, int cu_cap, hipStream_t stream);
hipError_t launch_tn(const TnProblem& p, int cu_cap, hipStream_t stream);
hipError_t launch_cast(const CastProblem& p, hipStream_t stream);
int64_t cast_grid(const CastProblem& p);   // workgroups launch_cast would start

// Short description of the tile configuration chosen for a problem (for
// DG_PRINT_CONFIGS), and the stable name of the kernel instance it launches.
const char* describe_nt_config(const NtProblem& p);
const char* describe_tn_config(const TnProblem& p);
const char* nt_config_name(const NtProblem& p);
const char* tn_config_name(const TnProblem& p);

}  // namespace dg
