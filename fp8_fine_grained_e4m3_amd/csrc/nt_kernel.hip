// Fine-grained FP8 e4m3 NT GEMM for gfx950: dense, M-grouped contiguous and
// M-grouped masked forms in one kernel template.
//
//   D[m,n] = C[m,n] + sum_kb (sa[kb,m] * sb[n/128,kb]) * P_kb[m,n]
//   P_kb[m,n] = sum over the 128 K of block kb of a[m,k] * b[n,k]
//
// The NT layout, D = C + A @ B^T, the transposed (MN-major) A scales and the
// two grouped layouts follow the "DeepGEMM" README (yuguo-Jack fork), section
// "Interfaces" ("Notices", "Grouped GEMMs (contiguous layout)", "Grouped GEMMs
// (masked layout)").  The per-128-K-block promotion of FP8 partial sums into
// an fp32 accumulator is the two-level accumulation of the news article
// "Deepseek AI Libera Deepgemm: a GEMM FP8 Library ...", section "Details and
// technical benefits"; here the block product runs on the MFMA unit and the
// promotion on the VALU, one fused multiply-add per output per K block.
//
// Work decomposition
//   * A workgroup owns a BM x BN output tile and walks K in 128-wide blocks.
//     The grid is persistent: workgroup w takes tiles w, w + grid, ...
//   * Per K block the A tile [BM x 128] and B tile [BN x 128] are staged into
//     LDS (double-buffered: the global loads of block kb+1 are in flight while
//     block kb is multiplied), rows of 128 bytes with an XOR-swizzled 16-byte
//     chunk order.
//   * Each wave owns a WTM x WTN sub-tile made of 16 x 16 MFMA tiles.  The MFMA
//     takes the B fragment as its row operand and the A fragment as its column
//     operand, so every lane's four results share one m (one A scale) and
//     cover four consecutive n.
//   * Promotion: acc += P * (sa[kb][m] * sb[nb][kb]) in fp32 VGPRs, kb
//     ascending.  bf16 (or fp32) conversion happens once, in the epilogue.
#include "dg_internal.h"
#include "tile_common.h"

#include <stdio.h>

namespace dg {

struct NtArgs {
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    const void* c;
    void* d;
    const int32_t* m_indices;
    const int32_t* masked_m;
    int rows;          // dense: M, contiguous: M_tot, masked: M_max
    int N;
    int K;
    int G;
    int tiles_m;       // per group
    int tiles_n;
    int num_tiles;     // enumerated tiles (masked: G * tiles_m * tiles_n)
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct NtCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WAVES_M;   // wave tile rows (m)
    static constexpr int WTN = BN / WAVES_N;   // wave tile columns (n)
    static constexpr int SM = WTM / 16;        // 16-row MFMA tiles per wave along m
    static constexpr int SN = WTN / 16;        // along n
    static constexpr int A_BYTES = BM * kKBlk;
    static constexpr int B_BYTES = BN * kKBlk;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_LD = A_BYTES / (16 * THREADS);   // 16-byte loads per thread
    static constexpr int B_LD = B_BYTES / (16 * THREADS);
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(A_BYTES % (16 * THREADS) == 0 && B_BYTES % (16 * THREADS) == 0,
                  "tile bytes must split evenly over the workgroup");
    static_assert(BN <= 128 || BN % 128 == 0, "an MFMA tile must not straddle a B scale block");
};

template <class Cfg, int FORM, bool OUT_F32>
__global__ __launch_bounds__(Cfg::THREADS) void nt_fp8_kernel(NtArgs p) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, THREADS = Cfg::THREADS;
    constexpr int SM = Cfg::SM, SN = Cfg::SN, A_LD = Cfg::A_LD, B_LD = Cfg::B_LD;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Cfg::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;
    const int KB = p.K / kKBlk;
    const int NB = (p.N + kKBlk - 1) / kKBlk;
    const int per_group = p.tiles_m * p.tiles_n;

    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        // ---- tile scheduling (uniform over the workgroup) ------------------
        int g = 0, e = 0, local = t;
        if (FORM == kMasked) {
            g = t / per_group;
            local = t - g * per_group;
            e = g;
        }
        const int tm = local % p.tiles_m;
        const int tn = local / p.tiles_m;
        const int r0 = tm * BM;        // first row of the tile, relative to its group
        const int n0 = tn * BN;
        int grp_rows = p.rows;         // rows that exist in memory for this group
        int store_rows = p.rows;       // rows that may be written
        int64_t grp_row0 = 0;          // first row of the group in A / D
        if (FORM == kMasked) {
            int mm = p.masked_m[g];
            mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
            store_rows = mm;
            grp_row0 = (int64_t)g * p.rows;
            if (r0 >= mm) continue;
        } else if (FORM == kContiguous) {
            e = p.m_indices[r0];
            if (e < 0 || e >= p.G) continue;
        }

        const uint8_t* __restrict__ a_t = p.a + grp_row0 * p.K;
        const uint8_t* __restrict__ b_t = p.b + (int64_t)e * p.N * p.K;
        const int sfa_ld = p.rows;
        const float* __restrict__ sfa_t = p.sfa + (FORM == kMasked ? (int64_t)g * KB * p.rows : 0);
        const float* __restrict__ sfb_t = p.sfb + (int64_t)e * NB * KB;

        // per-thread global offsets (rows clamped to what exists) and LDS offsets
        uint32_t ga_off[A_LD], gb_off[B_LD];
        int la_off[A_LD], lb_off[B_LD];
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int ch = tid + i * THREADS;
            const int rr = ch >> 3, cc = ch & 7;
            const int row = min(r0 + rr, grp_rows - 1);
            ga_off[i] = (uint32_t)row * (uint32_t)p.K + cc * 16;
            la_off[i] = lds_chunk_off(rr, cc);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int ch = tid + i * THREADS;
            const int rr = ch >> 3, cc = ch & 7;
            const int row = min(n0 + rr, p.N - 1);
            gb_off[i] = (uint32_t)row * (uint32_t)p.K + cc * 16;
            lb_off[i] = BM * kKBlk + lds_chunk_off(rr, cc);
        }
        // scale indices of this lane's rows and of this wave's 16-column tiles
        int sa_idx[SM];
#pragma unroll
        for (int i = 0; i < SM; ++i)
            sa_idx[i] = min(r0 + wm * Cfg::WTM + 16 * i + (lane & 15), grp_rows - 1);
        int sb_idx[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j)
            sb_idx[j] = min((n0 + wn * Cfg::WTN + 16 * j) / kKBlk, NB - 1) * KB;

        f32x4 acc[SM][SN];
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        i32x4 ra[A_LD], rb[B_LD];
        float sa_cur[SM], sb_cur[SN], sa_nxt[SM], sb_nxt[SN];

        // ---- prologue: block 0 into stage 0 ------------------------------------
        if (KB > 0) {
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                ra[i] = *reinterpret_cast<const i32x4*>(a_t + ga_off[i]);
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                rb[i] = *reinterpret_cast<const i32x4*>(b_t + gb_off[i]);
#pragma unroll
            for (int i = 0; i < SM; ++i) sa_nxt[i] = sfa_t[sa_idx[i]];
#pragma unroll
            for (int j = 0; j < SN; ++j) sb_nxt[j] = sfb_t[sb_idx[j]];
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                *reinterpret_cast<i32x4*>(smem + la_off[i]) = ra[i];
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                *reinterpret_cast<i32x4*>(smem + lb_off[i]) = rb[i];
        }
        __syncthreads();

        // ---- main loop over 128-wide K blocks ------------------------------------
        for (int kb = 0; kb < KB; ++kb) {
            const int cur = kb & 1;
#pragma unroll
            for (int i = 0; i < SM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
            for (int j = 0; j < SN; ++j) sb_cur[j] = sb_nxt[j];
            const bool more = kb + 1 < KB;
            if (more) {
                const uint8_t* an = a_t + (kb + 1) * kKBlk;
                const uint8_t* bn = b_t + (kb + 1) * kKBlk;
#pragma unroll
                for (int i = 0; i < A_LD; ++i)
                    ra[i] = *reinterpret_cast<const i32x4*>(an + ga_off[i]);
#pragma unroll
                for (int i = 0; i < B_LD; ++i)
                    rb[i] = *reinterpret_cast<const i32x4*>(bn + gb_off[i]);
#pragma unroll
                for (int i = 0; i < SM; ++i) sa_nxt[i] = sfa_t[(kb + 1) * sfa_ld + sa_idx[i]];
#pragma unroll
                for (int j = 0; j < SN; ++j) sb_nxt[j] = sfb_t[sb_idx[j] + kb + 1];
            }

            const uint8_t* sA = smem + cur * Cfg::STAGE_BYTES;
            const uint8_t* sB = sA + Cfg::A_BYTES;
            i32x8 bfrag[SN];
#pragma unroll
            for (int j = 0; j < SN; ++j)
                bfrag[j] = lds_fragment(sB, wn * Cfg::WTN + 16 * j, lane);
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const i32x8 afrag = lds_fragment(sA, wm * Cfg::WTM + 16 * i, lane);
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const f32x4 pblk = mfma_e4m3_block(bfrag[j], afrag);
                    const float s = sa_cur[i] * sb_cur[j];
                    acc[i][j].x = __builtin_fmaf(pblk.x, s, acc[i][j].x);
                    acc[i][j].y = __builtin_fmaf(pblk.y, s, acc[i][j].y);
                    acc[i][j].z = __builtin_fmaf(pblk.z, s, acc[i][j].z);
                    acc[i][j].w = __builtin_fmaf(pblk.w, s, acc[i][j].w);
                }
            }

            if (more) {
                uint8_t* nxt = smem + (cur ^ 1) * Cfg::STAGE_BYTES;
#pragma unroll
                for (int i = 0; i < A_LD; ++i)
                    *reinterpret_cast<i32x4*>(nxt + la_off[i]) = ra[i];
#pragma unroll
                for (int i = 0; i < B_LD; ++i)
                    *reinterpret_cast<i32x4*>(nxt + lb_off[i]) = rb[i];
            }
            __syncthreads();
        }

        // ---- epilogue: (+C), convert once, masked store ---------------------------
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int m = r0 + wm * Cfg::WTM + 16 * i + (lane & 15);
            bool row_ok = m < store_rows;
            if (FORM == kContiguous && row_ok) row_ok = p.m_indices[m] == e;
            if (!row_ok) continue;
            const int64_t row_off = (grp_row0 + m) * (int64_t)p.N;
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const int n = n0 + wn * Cfg::WTN + 16 * j + 4 * (lane >> 4);
                if (n >= p.N) continue;
                f32x4 v = acc[i][j];
                if (OUT_F32) {
                    float* dp = reinterpret_cast<float*>(p.d) + row_off + n;
                    if (p.c) {
                        const f32x4 cv = *reinterpret_cast<const f32x4*>(
                            reinterpret_cast<const float*>(p.c) + row_off + n);
                        v += cv;
                    }
                    *reinterpret_cast<f32x4*>(dp) = v;
                } else {
                    uint16_t* dp = reinterpret_cast<uint16_t*>(p.d) + row_off + n;
                    if (p.c) {
                        const i32x2 cv = *reinterpret_cast<const i32x2*>(
                            reinterpret_cast<const uint16_t*>(p.c) + row_off + n);
                        v.x += bf16_bits_to_f32((uint32_t)cv.x & 0xFFFFu);
                        v.y += bf16_bits_to_f32((uint32_t)cv.x >> 16);
                        v.z += bf16_bits_to_f32((uint32_t)cv.y & 0xFFFFu);
                        v.w += bf16_bits_to_f32((uint32_t)cv.y >> 16);
                    }
                    *reinterpret_cast<i32x2*>(dp) = pack_bf16x4(v.x, v.y, v.z, v.w);
                }
            }
        }
        // The next tile's prologue rewrites stage 0; every wave is past its last
        // read of either stage because the K loop ends with a barrier.
    }
}

// ------------------------------------------------------------------------------
// Host side: configuration choice and launch
// ------------------------------------------------------------------------------

namespace {

template <class Cfg, int FORM, bool OUT_F32>
hipError_t launch_cfg(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    NtArgs a;
    a.a = pr.a; a.sfa = pr.sfa; a.b = pr.b; a.sfb = pr.sfb; a.c = pr.c; a.d = pr.d;
    a.m_indices = pr.m_indices; a.masked_m = pr.masked_m;
    a.rows = (int)pr.rows; a.N = (int)pr.N; a.K = (int)pr.K; a.G = (int)pr.G;
    a.tiles_m = (int)((pr.rows + Cfg::BM - 1) / Cfg::BM);
    a.tiles_n = (int)((pr.N + Cfg::BN - 1) / Cfg::BN);
    const int64_t groups = (FORM == kMasked) ? pr.G : 1;
    const int64_t tiles = groups * a.tiles_m * a.tiles_n;
    if (tiles <= 0) return hipSuccess;
    a.num_tiles = (int)tiles;

    static int occupancy = -1;   // workgroups per CU for this instance
    if (occupancy < 0) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &occ, reinterpret_cast<const void*>(&nt_fp8_kernel<Cfg, FORM, OUT_F32>),
                Cfg::THREADS, 0) != hipSuccess || occ < 1)
            occ = 1;
        occupancy = occ;
    }
    const int64_t resident = (int64_t)cu_cap * occupancy;
    const int grid = (int)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL((nt_fp8_kernel<Cfg, FORM, OUT_F32>), dim3(grid), dim3(Cfg::THREADS), 0,
                       stream, a);
    return hipGetLastError();
}

using Cfg128x128 = NtCfg<128, 128, 2, 2>;
using Cfg64x128 = NtCfg<64, 128, 1, 4>;

template <int FORM, bool OUT_F32>
hipError_t dispatch_tiles(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    // Rows per group decide the M tile: small-M (decode-like) problems use
    // 64-row tiles so fewer rows of MFMA work are wasted.
    const bool small_m = (FORM == kMasked) ? pr.rows <= 64 : (FORM == kDense && pr.rows <= 64);
    if (small_m) return launch_cfg<Cfg64x128, FORM, OUT_F32>(pr, cu_cap, stream);
    return launch_cfg<Cfg128x128, FORM, OUT_F32>(pr, cu_cap, stream);
}

}  // namespace

hipError_t launch_nt(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    switch (pr.form) {
    case kDense:
        return pr.out_f32 ? dispatch_tiles<kDense, true>(pr, cu_cap, stream)
                          : dispatch_tiles<kDense, false>(pr, cu_cap, stream);
    case kContiguous:
        return dispatch_tiles<kContiguous, false>(pr, cu_cap, stream);
    case kMasked:
        return dispatch_tiles<kMasked, false>(pr, cu_cap, stream);
    }
    return hipErrorInvalidValue;
}

const char* describe_nt_config(const NtProblem& pr) {
    static thread_local char buf[160];
    const bool small_m = (pr.form == kMasked) ? pr.rows <= 64 : (pr.form == kDense && pr.rows <= 64);
    snprintf(buf, sizeof buf, "nt form=%d rows=%lld N=%lld K=%lld G=%lld tile=%s", (int)pr.form,
             (long long)pr.rows, (long long)pr.N, (long long)pr.K, (long long)pr.G,
             small_m ? "64x128 (1x4 waves)" : "128x128 (2x2 waves)");
    return buf;
}

}  // namespace dg
