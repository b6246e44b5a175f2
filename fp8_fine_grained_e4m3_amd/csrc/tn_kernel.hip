// K-grouped fine-grained FP8 e4m3 TN GEMM for gfx950 (MoE weight gradient).
//
//   D[g][m,n] = C[g][m,n] + sum over group g's K blocks kb of
//               (sa[kb,m] * sb[kb,n]) * sum_{k in kb} a[k,m] * b[k,n]
//
// A is stored [K_total, M] and B [K_total, N] (both MN-major: the "T" and "N"
// of the name), the groups are consecutive segments along K, and M and N are
// fixed ("DeepGEMM" README, yuguo-Jack fork, section "Interfaces", "Grouped
// GEMMs (contiguous layout)": the K-axis-grouped API for the MoE weight
// backward pass).  Both operands carry one fp32 scale per column per 128-wide
// K block, so the promotion multiplies each block product by a per-element
// scale sa[m] * sb[n] (news article "Deepseek AI Libera Deepgemm ...", section
// "Details and technical benefits": two-level accumulation).
//
// The MFMA wants 32 K-consecutive bytes of one row per lane, while memory
// holds M (or N) consecutive bytes of one K row.  Each thread loads an 8 x 8
// byte block (8 K rows x 8 columns, coalesced along the columns), transposes
// it in registers with byte permutes, and writes 8 K-consecutive bytes per
// column into the same swizzled K-major LDS layout the NT kernel uses.  From
// there on the block product, promotion and epilogue mirror the NT kernel,
// with fp32 C read and fp32 D written.
//
// Scheduling: the host passes each group's K-block range and a processing
// order (largest K first, so the longest tiles start first); the persistent
// grid walks (group, m tile, n tile) in that order.  A group with K = 0 still
// produces D[g] = C[g] (or 0).
#include "dg_internal.h"
#include "tile_common.h"

#include <stdio.h>
#include <algorithm>
#include <numeric>

namespace dg {

struct TnArgs {
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    const float* c;
    float* d;
    int M, N, G;
    int tiles_m, tiles_n, num_tiles;
    int32_t order[kMaxTnGroups];      // processing order of the groups
    int32_t kb_start[kMaxTnGroups];   // first 128-K block of group g
    int32_t kb_count[kMaxTnGroups];   // number of 128-K blocks of group g
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TnCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int SM = WTM / 16;
    static constexpr int SN = WTN / 16;
    static constexpr int A_BYTES = BM * kKBlk;
    static constexpr int B_BYTES = BN * kKBlk;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_BLK = (kKBlk / 8) * (BM / 8) / THREADS;   // 8x8 blocks per thread
    static constexpr int B_BLK = (kKBlk / 8) * (BN / 8) / THREADS;
    static_assert(A_BLK * THREADS == (kKBlk / 8) * (BM / 8), "A tile must split evenly");
    static_assert(B_BLK * THREADS == (kKBlk / 8) * (BN / 8), "B tile must split evenly");
};

// 4 x 4 byte transpose: out[j] byte i = in[i] byte j.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3) {
    // __builtin_amdgcn_perm(hi, lo, sel): selector bytes 0..3 pick from lo, 4..7 from hi
    const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0.0 r1.0 r0.1 r1.1
    const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);   // r0.2 r1.2 r0.3 r1.3
    const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    c0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);                  // t0.0 t0.1 t2.0 t2.1
    c1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);                  // t0.2 t0.3 t2.2 t2.3
    c2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    c3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// rows[i] = 8 bytes (columns 0..7) of K row i; out[j] = 8 bytes (K rows 0..7) of column j.
__device__ __forceinline__ void transpose8x8(const i32x2 rows[8], i32x2 out[8]) {
    uint32_t c0, c1, c2, c3;
    // columns 0..3, K 0..3 -> low dwords
    transpose4x4(rows[0].x, rows[1].x, rows[2].x, rows[3].x, c0, c1, c2, c3);
    out[0].x = c0; out[1].x = c1; out[2].x = c2; out[3].x = c3;
    // columns 0..3, K 4..7 -> high dwords
    transpose4x4(rows[4].x, rows[5].x, rows[6].x, rows[7].x, c0, c1, c2, c3);
    out[0].y = c0; out[1].y = c1; out[2].y = c2; out[3].y = c3;
    // columns 4..7
    transpose4x4(rows[0].y, rows[1].y, rows[2].y, rows[3].y, c0, c1, c2, c3);
    out[4].x = c0; out[5].x = c1; out[6].x = c2; out[7].x = c3;
    transpose4x4(rows[4].y, rows[5].y, rows[6].y, rows[7].y, c0, c1, c2, c3);
    out[4].y = c0; out[5].y = c1; out[6].y = c2; out[7].y = c3;
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS) void tn_fp8_kernel(TnArgs p) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, THREADS = Cfg::THREADS;
    constexpr int SM = Cfg::SM, SN = Cfg::SN, A_BLK = Cfg::A_BLK, B_BLK = Cfg::B_BLK;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Cfg::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;
    const int per_group = p.tiles_m * p.tiles_n;

    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const int gi = t / per_group;
        const int local = t - gi * per_group;
        const int g = p.order[gi];
        const int tm = local % p.tiles_m;
        const int tn = local / p.tiles_m;
        const int m0 = tm * BM, n0 = tn * BN;
        const int kb0 = p.kb_start[g];
        const int KBg = p.kb_count[g];

        // Per-thread 8x8 block coordinates; columns clamped so loads stay in bounds.
        uint32_t ga_off[A_BLK], gb_off[B_BLK];
#pragma unroll
        for (int q = 0; q < A_BLK; ++q) {
            const int blk = tid + q * THREADS;
            const int cq = blk % (BM / 8), kq = blk / (BM / 8);
            const int col = min(m0 + cq * 8, p.M - 8);
            ga_off[q] = (uint32_t)(kq * 8) * (uint32_t)p.M + (uint32_t)col;
        }
#pragma unroll
        for (int q = 0; q < B_BLK; ++q) {
            const int blk = tid + q * THREADS;
            const int cq = blk % (BN / 8), kq = blk / (BN / 8);
            const int col = min(n0 + cq * 8, p.N - 8);
            gb_off[q] = (uint32_t)(kq * 8) * (uint32_t)p.N + (uint32_t)col;
        }
        int sa_idx[SM];
#pragma unroll
        for (int i = 0; i < SM; ++i)
            sa_idx[i] = min(m0 + wm * Cfg::WTM + 16 * i + (lane & 15), p.M - 1);
        int sb_idx[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j)
            sb_idx[j] = min(n0 + wn * Cfg::WTN + 16 * j + 4 * (lane >> 4), p.N - 4);

        f32x4 acc[SM][SN];
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        i32x2 ra[A_BLK][8], rb[B_BLK][8];
        float sa_cur[SM], sa_nxt[SM];
        f32x4 sb_cur[SN], sb_nxt[SN];

        auto gload = [&](int kb) {
            const uint8_t* ak = p.a + (int64_t)kb * kKBlk * p.M;
            const uint8_t* bk = p.b + (int64_t)kb * kKBlk * p.N;
#pragma unroll
            for (int q = 0; q < A_BLK; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ra[q][i] = *reinterpret_cast<const i32x2*>(ak + ga_off[q] + i * p.M);
#pragma unroll
            for (int q = 0; q < B_BLK; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rb[q][i] = *reinterpret_cast<const i32x2*>(bk + gb_off[q] + i * p.N);
#pragma unroll
            for (int i = 0; i < SM; ++i) sa_nxt[i] = p.sfa[(int64_t)kb * p.M + sa_idx[i]];
#pragma unroll
            for (int j = 0; j < SN; ++j)
                sb_nxt[j] = *reinterpret_cast<const f32x4*>(p.sfb + (int64_t)kb * p.N + sb_idx[j]);
        };
        auto lstore = [&](int stage) {
            uint8_t* sA = smem + stage * Cfg::STAGE_BYTES;
            uint8_t* sB = sA + Cfg::A_BYTES;
#pragma unroll
            for (int q = 0; q < A_BLK; ++q) {
                i32x2 cols[8];
                transpose8x8(ra[q], cols);
                const int blk = tid + q * THREADS;
                const int cq = blk % (BM / 8), kq = blk / (BM / 8);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<i32x2*>(sA + lds_chunk_off(cq * 8 + j, kq >> 1) +
                                              (kq & 1) * 8) = cols[j];
            }
#pragma unroll
            for (int q = 0; q < B_BLK; ++q) {
                i32x2 cols[8];
                transpose8x8(rb[q], cols);
                const int blk = tid + q * THREADS;
                const int cq = blk % (BN / 8), kq = blk / (BN / 8);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<i32x2*>(sB + lds_chunk_off(cq * 8 + j, kq >> 1) +
                                              (kq & 1) * 8) = cols[j];
            }
        };

        if (KBg > 0) {
            gload(kb0);
            lstore(0);
        }
        __syncthreads();

        for (int it = 0; it < KBg; ++it) {
            const int cur = it & 1;
#pragma unroll
            for (int i = 0; i < SM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
            for (int j = 0; j < SN; ++j) sb_cur[j] = sb_nxt[j];
            const bool more = it + 1 < KBg;
            if (more) gload(kb0 + it + 1);

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
                    const float sa = sa_cur[i];
                    acc[i][j].x = __builtin_fmaf(pblk.x, sa * sb_cur[j].x, acc[i][j].x);
                    acc[i][j].y = __builtin_fmaf(pblk.y, sa * sb_cur[j].y, acc[i][j].y);
                    acc[i][j].z = __builtin_fmaf(pblk.z, sa * sb_cur[j].z, acc[i][j].z);
                    acc[i][j].w = __builtin_fmaf(pblk.w, sa * sb_cur[j].w, acc[i][j].w);
                }
            }
            if (more) lstore(cur ^ 1);
            __syncthreads();
        }

        // epilogue: D[g] = C[g] + acc, fp32, rows/cols inside [M, N]
        const int64_t gbase = (int64_t)g * p.M * p.N;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int m = m0 + wm * Cfg::WTM + 16 * i + (lane & 15);
            if (m >= p.M) continue;
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const int n = n0 + wn * Cfg::WTN + 16 * j + 4 * (lane >> 4);
                if (n >= p.N) continue;
                const int64_t off = gbase + (int64_t)m * p.N + n;
                f32x4 v = acc[i][j];
                if (p.c) v += *reinterpret_cast<const f32x4*>(p.c + off);
                *reinterpret_cast<f32x4*>(p.d + off) = v;
            }
        }
    }
}

namespace {

using TnCfg128 = TnCfg<128, 128, 2, 2>;

template <class Cfg>
hipError_t launch_tn_cfg(const TnProblem& pr, int cu_cap, hipStream_t stream) {
    TnArgs a;
    a.a = pr.a; a.sfa = pr.sfa; a.b = pr.b; a.sfb = pr.sfb; a.c = pr.c; a.d = pr.d;
    a.M = (int)pr.M; a.N = (int)pr.N; a.G = (int)pr.G;
    a.tiles_m = (int)((pr.M + Cfg::BM - 1) / Cfg::BM);
    a.tiles_n = (int)((pr.N + Cfg::BN - 1) / Cfg::BN);
    const int64_t tiles = pr.G * a.tiles_m * a.tiles_n;
    if (tiles <= 0) return hipSuccess;
    a.num_tiles = (int)tiles;
    int32_t start = 0;
    for (int g = 0; g < a.G; ++g) {
        a.kb_start[g] = start;
        a.kb_count[g] = pr.k_sizes_host[g] / kKBlk;
        start += a.kb_count[g];
    }
    // Longest-processing-time order: groups with the most K blocks first.
    std::iota(a.order, a.order + a.G, 0);
    std::stable_sort(a.order, a.order + a.G,
                     [&](int x, int y) { return a.kb_count[x] > a.kb_count[y]; });

    static int occupancy = -1;
    if (occupancy < 0) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &occ, reinterpret_cast<const void*>(&tn_fp8_kernel<Cfg>), Cfg::THREADS, 0) !=
                hipSuccess ||
            occ < 1)
            occ = 1;
        occupancy = occ;
    }
    const int64_t resident = (int64_t)cu_cap * occupancy;
    const int grid = (int)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL((tn_fp8_kernel<Cfg>), dim3(grid), dim3(Cfg::THREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tn(const TnProblem& pr, int cu_cap, hipStream_t stream) {
    return launch_tn_cfg<TnCfg128>(pr, cu_cap, stream);
}

const char* tn_config_name(const TnProblem&) { return "tn_kgrouped_f32_128x128"; }

const char* describe_tn_config(const TnProblem& pr) {
    static thread_local char buf[192];
    snprintf(buf, sizeof buf, "%s G=%lld M=%lld N=%lld K_tot=%lld", tn_config_name(pr),
             (long long)pr.G, (long long)pr.M, (long long)pr.N, (long long)pr.K_tot);
    return buf;
}

}  // namespace dg
