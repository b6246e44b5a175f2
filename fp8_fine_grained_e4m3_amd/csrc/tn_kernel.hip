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
// Staging: per 128-row K block, the A tile [128 k x BM] and the B tile
// [128 k x BN] are copied global -> LDS as they lie in memory (one LDS row per
// K row; 16-byte chunk c of row k at position c ^ f(k)), together with the
// block's scales, by global_load_lds; STAGES - 1 blocks are in flight.
//
// Fragments: the MFMA wants, per lane, 32 K-consecutive bytes of one column
// (one m or one n).  gfx950's transposing LDS read ds_read_b64_tr_b8 produces
// them from the MN-major tile: within each 16-lane group, lane k names 8 bytes
// (chunk C_k) and lane i + 8h (i < 8) receives byte i of C_{2j+h} as its
// byte j.  Lane k of a group names K row kbase + (k >> 1) at column offset
// 8 (k & 1) of a 16-column chunk, so lane r of the group receives column r's
// K values kbase .. kbase + 7; four reads (kbase = 32 g + 8 q for the lane's
// K quarter g, q = 0..3) make the lane's 32 bytes.  The chunk swizzle f(k)
// keeps each 32-lane half of a read on 32 distinct 8-byte bank slots.
//
// The block product runs on the MFMA unit (the B fragment as row operand, A as
// column operand: a lane's 4 results share one m and cover 4 consecutive n),
// the promotion acc += P * (sa[m] * sb[n]) on the VALU, software-pipelined two
// block products behind.  The accumulator starts from C (its loads overlap the
// first copies), so the epilogue is a plain fp32 store, staged through LDS into
// whole-row stores.
//
// Scheduling: the host passes each group's K-block range and a processing
// order (largest K first, so the longest tiles start first); the persistent
// grid walks (group, m tile, n tile) in that order.  A group with K = 0 still
// produces D[g] = C[g] (or 0).
//
// The same kernel serves the dense NN, TN and TT layouts (the README's
// "Notices" lists NT, TN, NN and TT; the first letter is A's, "N" = stored
// [M, K]; the second is B's, "T" = stored [N, K]) as one group spanning all
// of K, and the M-grouped contiguous NN form ("Grouped GEMMs (contiguous
// layout)" names the nt and nn contiguous variants), whose 128-row tiles each
// take the expert of their first row.  An operand stored with K contiguous
// (A_MK, B_NK) is staged like the NT kernel's B tile: one 128-byte LDS row
// per matrix row, 16-byte chunk c at position sigma(c) ^ ((row >> 1) & 7)
// (sigma swaps bits 0 and 1 of c), and read with plain 16-byte LDS loads
// (lane l: row l & 15 of the fragment, K bytes 32 (l >> 4) .. +31), which is
// the same register layout the transposing reads produce.  The position does
// not change between rows 16 apart, so fragment c of a lane is its fragment
// 0 plus the immediate 2048 c; and under gfx950's ds_read_b128 bank rule
// (four 16-lane groups, lane l in group 2 bit5(l) + (bit2 ^ bit3 ^ bit4)(l),
// conflict-free when a group's lanes hit 16 distinct 16-byte slots modulo
// 256 bytes) every group of a fragment read lands on 16 distinct slots.  The scales are per output row / column on both sides in
// every layout, so the promotion is unchanged.
#include "dg_internal.h"
#include "tile_common.h"

#include <limits.h>
#include <stdio.h>
#include <algorithm>
#include <numeric>

namespace dg {

struct TnArgs {
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    const void* c;     // fp32 or bf16 (the output type), may be NULL
    void* d;
    const int32_t* m_indices;   // M-grouped NN
    int M, N, G;
    int K;             // row length of operands stored with K contiguous
    int tiles_m, tiles_n, num_tiles;
    int xcd_bm, xcd_bn;   // XCD blocks of a group's tiles (0: column order)
    int32_t order[kMaxTnGroups];      // processing order of the groups
    int32_t kb_start[kMaxTnGroups];   // first 128-K block of group g
    int32_t kb_count[kMaxTnGroups];   // number of 128-K blocks of group g
    int32_t kw_start[kMaxTnGroups];   // UE8M0: first packed word row of group g
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct TnCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int STAGES = STAGES_;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int SM = WTM / 16;
    static constexpr int SN = WTN / 16;
    static constexpr int A_BYTES = kKBlk * BM;
    static constexpr int B_BYTES = kKBlk * BN;
    static constexpr int SA_OFF = A_BYTES + B_BYTES;
    static constexpr int SB_OFF = SA_OFF + 4 * BM;
    static constexpr int STAGE_BYTES = SB_OFF + 4 * BN;
    static constexpr int A_DMA = A_BYTES / 1024;   // 1 KiB wave copies per stage
    static constexpr int B_DMA = B_BYTES / 1024;
    static constexpr int SA_DMA = BM / 64;         // 256-byte (64-float) wave copies
    static constexpr int SB_DMA = BN / 64;
    static constexpr int DMA_PER_WAVE = (A_DMA + B_DMA) / WAVES;
    static constexpr int VM_PER_STAGE = DMA_PER_WAVE + 1;
    static_assert((A_DMA + B_DMA) % WAVES == 0, "tile copies must split evenly over waves");
    static_assert(SA_DMA + SB_DMA <= WAVES, "at most one scale copy per wave");
    static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "row widths");
    static_assert(WTM % 64 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(STAGES >= 2 && (STAGES - 2) * VM_PER_STAGE <= 63, "vmcnt range");
    // Workgroups resident per CU: bounded by the 160 KiB of LDS and by the
    // two waves per SIMD the kernel is compiled for (8 waves per CU).
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int WG_PER_CU =
        (160 * 1024 / LDS_BYTES) < (8 / WAVES) ? (160 * 1024 / LDS_BYTES) : (8 / WAVES);
    static_assert(WG_PER_CU >= 1, "one workgroup fits a CU");
};

// Swizzle of an MN-major LDS tile with W-byte rows: 16-byte chunk c of K row
// `row` sits at chunk position c ^ tn_swz<W>(row).  A transposing read touches
// rows 32 g + 8 q + 0..7 (g = 0, 1 in one 32-lane half); the low bits spread
// those 8 rows, bit 5 of the row moves the second group to the other half of
// the banks.
// K-contiguous staging: position of chunk c of row `row` (and, sigma being an
// involution, the chunk held at position c).
__device__ __forceinline__ int k_sigma(int c) { return ((c >> 1) & 1) | ((c & 1) << 1) | (c & 4); }
__device__ __forceinline__ int k_pos(int row, int c) { return k_sigma(c) ^ ((row >> 1) & 7); }

template <int W>
__device__ __forceinline__ int tn_swz(int row) {
    if constexpr (W == 128) return ((row >> 1) & 3) | (((row >> 5) & 1) << 2);
    else return (row & 7) | (((row >> 5) & 1) << 3);
}

constexpr int kGroupedBand = 4;   // M-grouped: 256-row tiles per rasterisation band

// UE8M0 (K-grouped form): the scales are packed power-of-two exponents, each
// group's blocks on their own word rows (byte i of word row kw_start[g] + k4
// holds the group's block 4 k4 + i); v_mfma_scale applies them to the block
// product and accumulates, so there is no promotion step.
template <class Cfg, bool A_MK, bool B_NK, bool OUT_F32, bool GROUPED_M, bool UE8M0>
__global__ __launch_bounds__(Cfg::THREADS) void tn_fp8_kernel(TnArgs p) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, SM = Cfg::SM, SN = Cfg::SN;
    static_assert(!GROUPED_M || BM == 2 * kKBlk, "grouped tiles span two 128-row expert blocks");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::STAGES * Cfg::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;
    const int per_group = p.tiles_m * p.tiles_n;
    const uint32_t lds0 = lds_addr(smem);
    const int r16 = lane & 15;

    // Per-lane part of the transposing fragment reads: K row 32 g + (k >> 1)
    // (+ 8 q), column offset 8 (k & 1), for lane (g, k) = (lane >> 4, lane & 15).
    const int tr_row = 32 * (lane >> 4) + (r16 >> 1);
    const int a_lane = tr_row * BM + 8 * (r16 & 1);
    const int b_lane = Cfg::A_BYTES + tr_row * BN + 8 * (r16 & 1);
    const int a_x = tn_swz<BM>(tr_row);
    const int b_x = tn_swz<BN>(tr_row);
    // K-contiguous operands: byte offsets of the lane's two 16-byte chunks in
    // fragment 0 (row r16); fragment c adds 16 * 128 * c
    const int k_c0 = 2 * (lane >> 4);
    const int k_lo = r16 * kKBlk + (k_pos(r16, k_c0) << 4);
    // chunk k_c0 + 1 sits at position k_pos(r16, k_c0) ^ 2 (k_c0 is even, so
    // k_sigma only sets bit 1 for the odd chunk): 32 bytes across, and the
    // row term has no bit 5
    static_assert(kKBlk % 64 == 0, "row term clear of bit 5");

    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        // M-grouped: every tile is listed twice; pass `gi` computes it with the
        // expert of its 128-row block gi (pass 1 only when that expert differs
        // from block 0's), storing only the rows of that expert
        const int gi = t / per_group;
        const int local = t - gi * per_group;
        const int g = GROUPED_M ? 0 : p.order[gi];
        int tm = local % p.tiles_m;
        int tn = local / p.tiles_m;
        if constexpr (!GROUPED_M) {
            // XCD blocks: workgroups are dealt to the 8 XCDs round-robin and a
            // group's tiles start at a multiple of 8, so tile `local` runs on
            // XCD local % 8, which takes one xcd_bm x xcd_bn block of the
            // group's tiles.  The tiles an XCD has in flight then share
            // xcd_bm A panels and xcd_bn B panels in its L2 (in column order
            // a group of 8 M tiles would give each XCD one A panel but every
            // B panel).
            if (p.xcd_bm > 0) {
                const int x = local & 7, j = local >> 3;
                const int bxm = p.tiles_m / p.xcd_bm;
                tm = (x % bxm) * p.xcd_bm + j % p.xcd_bm;
                tn = (x / bxm) * p.xcd_bn + j / p.xcd_bm;
            }
        } else {
            // bands of kGroupedBand M tiles, N advancing after each tile
            // of a band: the tiles in flight share a few A blocks (each read
            // once for all N tiles) and the B panels of the band's experts
            const int band_tiles = kGroupedBand * p.tiles_n;
            const int band = local / band_tiles;
            const int in_band = local - band * band_tiles;
            const int rows_in_band = min(p.tiles_m - band * kGroupedBand, kGroupedBand);
            tm = band * kGroupedBand + in_band % rows_in_band;
            tn = in_band / rows_in_band;
        }
        const int m0 = tm * BM, n0 = tn * BN;
        const int kb0 = GROUPED_M ? 0 : p.kb_start[g];
        const int kw0 = UE8M0 ? p.kw_start[g] : 0;
        const int nkb = GROUPED_M ? p.K / kKBlk : p.kb_count[g];
        const int64_t gbase = (int64_t)g * p.M * p.N;
        // M-grouped: the expert of block gi is the index of its first row
        // (padding blocks are skipped)
        int e = 0;
        if constexpr (GROUPED_M) {
            const int rb = m0 + gi * kKBlk;
            if (rb >= p.M) continue;
            e = p.m_indices[rb];
            if (e < 0 || e >= p.G) continue;
            if (gi == 1 && p.m_indices[m0] == e) continue;   // pass 0 covers it
        }
        const uint8_t* __restrict__ b_e = p.b + (int64_t)e * p.K * p.N;
        const float* __restrict__ sfb_e = p.sfb + (int64_t)e * (p.K / kKBlk) * p.N;
        const int lane_t = opaque(tid) & 63;   // this tile's prologue derives its offsets from it
        // M-grouped: the expert of every row this wave stores in the epilogue
        // (rows wave + 8 j, j = 0 .. 31; lane j holds row j's), requested now so
        // its latency hides under the K loop
        int row_expert = -1;
        if constexpr (GROUPED_M) {
            const int row = m0 + wave + 8 * (lane_t & 31);
            if (row < p.M) row_expert = p.m_indices[row];
        }

        // Copy offsets.  Copy u of A moves 1024 / BM K rows: lane l fills LDS
        // chunk position l % (BM / 16) of row u * (1024 / BM) + l / (BM / 16),
        // i.e. loads the chunk that the swizzle places there.  Chunks past the
        // M (or N) edge re-read the last chunk; their columns are never stored.
        uint32_t goff[Cfg::DMA_PER_WAVE];
#pragma unroll
        for (int q = 0; q < Cfg::DMA_PER_WAVE; ++q) {
            const int u = wave * Cfg::DMA_PER_WAVE + q;
            if (u < Cfg::A_DMA) {
                if constexpr (A_MK) {
                    // 8 matrix rows of 128 K bytes; rows past M re-read the last one
                    const int row = 8 * u + (lane_t >> 3);
                    const int ch = k_sigma((lane_t & 7) ^ ((row >> 1) & 7));   // chunk at position lane & 7
                    goff[q] = (uint32_t)min(m0 + row, p.M - 1) * (uint32_t)p.K + (uint32_t)(ch * 16);
                } else {
                    const int row = u * (1024 / BM) + lane_t / (BM / 16);
                    const int ch = (lane_t % (BM / 16)) ^ tn_swz<BM>(row);
                    goff[q] = (uint32_t)row * (uint32_t)p.M + (uint32_t)min(m0 + 16 * ch, p.M - 16);
                }
            } else {
                const int uu = u - Cfg::A_DMA;
                if constexpr (B_NK) {
                    const int row = 8 * uu + (lane_t >> 3);
                    const int ch = k_sigma((lane_t & 7) ^ ((row >> 1) & 7));
                    goff[q] = (uint32_t)min(n0 + row, p.N - 1) * (uint32_t)p.K + (uint32_t)(ch * 16);
                } else {
                    const int row = uu * (1024 / BN) + lane_t / (BN / 16);
                    const int ch = (lane_t % (BN / 16)) ^ tn_swz<BN>(row);
                    goff[q] = (uint32_t)row * (uint32_t)p.N + (uint32_t)min(n0 + 16 * ch, p.N - 16);
                }
            }
        }
        // Scale copies, one per wave: copies [0, SA_DMA) fill A-scale slots,
        // the next SB_DMA fill B-scale slots, surplus waves repeat one (same
        // bytes to the same place).  A slot wm*WTM + 64 (i / 4) + 4 r + i % 4
        // holds the scale of column wm*WTM + 16 i + r: lane r reads its scales
        // as float4s and each float4 read of 16 lanes covers 256 contiguous
        // bytes (no bank conflicts).
        const int scopy = __builtin_amdgcn_readfirstlane(wave % (Cfg::SA_DMA + Cfg::SB_DMA));
        const bool s_is_a = scopy < Cfg::SA_DMA;
        uint32_t s_off, s_lds;
        if (s_is_a) {
            const int slot = 64 * scopy + lane_t;
            const int wms = slot / Cfg::WTM, u = slot % Cfg::WTM;
            const int col = wms * Cfg::WTM + 16 * (4 * (u / 64) + u % 4) + (u % 64) / 4;
            s_off = 4u * (uint32_t)min(m0 + col, p.M - 1);
            s_lds = Cfg::SA_OFF + 256 * scopy;
        } else {
            const int slot = 64 * (scopy - Cfg::SA_DMA) + lane_t;
            s_off = 4u * (uint32_t)min(n0 + slot, p.N - 1);
            s_lds = Cfg::SB_OFF + 256 * (scopy - Cfg::SA_DMA);
        }
        auto issue_stage = [&](int kb, int stage) {
            const uint32_t dst = lds0 + stage * Cfg::STAGE_BYTES;
            const uint8_t* ak = p.a + (int64_t)kb * kKBlk * (A_MK ? 1 : p.M);
            const uint8_t* bk = b_e + (int64_t)kb * kKBlk * (B_NK ? 1 : p.N);
#pragma unroll
            for (int q = 0; q < Cfg::DMA_PER_WAVE; ++q) {
                const int u = wave * Cfg::DMA_PER_WAVE + q;
                dma16(u < Cfg::A_DMA ? ak : bk, goff[q], dst + u * 1024);
            }
            // fp32: row kb of the scales; UE8M0: the word row holding block kb
            const int64_t srow = UE8M0 ? kw0 + ((kb - kb0) >> 2) : kb;
            const float* sk = s_is_a ? p.sfa + srow * p.M : sfb_e + srow * p.N;
            dma4(sk, s_off, dst + s_lds);
        };

        // The accumulators start from C; its loads overlap the first copies.
        f32x4 acc[SM][SN];
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int m = min(m0 + wm * Cfg::WTM + 16 * i + (lane_t & 15), p.M - 1);
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const int n = min(n0 + wn * Cfg::WTN + 16 * j + 4 * (lane_t >> 4), p.N - 4);
                const int64_t off = gbase + (int64_t)m * p.N + n;
                if (!p.c) {
                    acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                } else if constexpr (OUT_F32) {
                    acc[i][j] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.c) + off);
                } else {
                    const i32x2 cv = *reinterpret_cast<const i32x2*>(static_cast<const uint16_t*>(p.c) + off);
                    acc[i][j] = f32x4{bf16_bits_to_f32((uint32_t)cv.x & 0xFFFFu),
                                      bf16_bits_to_f32((uint32_t)cv.x >> 16),
                                      bf16_bits_to_f32((uint32_t)cv.y & 0xFFFFu),
                                      bf16_bits_to_f32((uint32_t)cv.y >> 16)};
                }
            }
        }

#pragma unroll
        for (int q = 0; q < Cfg::STAGES - 1; ++q)
            if (q < nkb) issue_stage(kb0 + q, q);
        int stage = 0;
        for (int it = 0; it < nkb; ++it) {
            const int ahead = min(Cfg::STAGES - 2, nkb - 1 - it);
            wait_stage_copies<Cfg::STAGES - 2, Cfg::VM_PER_STAGE>(ahead);
            lgkm_drain_barrier();
            if (it + Cfg::STAGES - 1 < nkb) {
                int nst = stage + Cfg::STAGES - 1;
                nst -= nst >= Cfg::STAGES ? Cfg::STAGES : 0;
                issue_stage(kb0 + it + Cfg::STAGES - 1, nst);
            }
            const uint8_t* st = smem + stage * Cfg::STAGE_BYTES;
            stage = stage + 1 == Cfg::STAGES ? 0 : stage + 1;

            // 16 columns x 128 K of the tile whose LDS rows are `row_bytes` wide,
            // columns 16 * chunk .. 16 * chunk + 15.
            auto tr_frag = [&](int lane_off, int chunk, int x, int row_bytes) {
                const uint8_t* base = st + lane_off + ((chunk ^ x) << 4);
                i32x8 r;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)(base + q * 8 * row_bytes));
                    r[2 * q] = v.x;
                    r[2 * q + 1] = v.y;
                }
                return r;
            };
            float sa[SM];
            f32x4 sb[SN];
            int ea[SM], eb[SN];   // UE8M0: the lane's exponents (A column m, B row n of the MFMA)
            if constexpr (UE8M0) {
                const int sh = 8 * (it & 3);
#pragma unroll
                for (int i = 0; i < SM; i += 4) {
                    const i32x4 v = *reinterpret_cast<const i32x4*>(
                        st + Cfg::SA_OFF + 4 * (wm * Cfg::WTM + 64 * (i / 4) + 4 * r16));
                    ea[i] = (v.x >> sh) & 0xFF; ea[i + 1] = (v.y >> sh) & 0xFF;
                    ea[i + 2] = (v.z >> sh) & 0xFF; ea[i + 3] = (v.w >> sh) & 0xFF;
                }
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    eb[j] = (*reinterpret_cast<const int*>(
                                 st + Cfg::SB_OFF + 4 * (wn * Cfg::WTN + 16 * j + r16)) >> sh) & 0xFF;
            } else {
#pragma unroll
                for (int i = 0; i < SM; i += 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(
                        st + Cfg::SA_OFF + 4 * (wm * Cfg::WTM + 64 * (i / 4) + 4 * r16));
                    sa[i] = v.x; sa[i + 1] = v.y; sa[i + 2] = v.z; sa[i + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    sb[j] = *reinterpret_cast<const f32x4*>(
                        st + Cfg::SB_OFF + 4 * (wn * Cfg::WTN + 16 * j + 4 * (lane >> 4)));
            }
            // fragment of 16 columns (tile columns 16 c .. 16 c + 15) of A or B
            auto k_frag = [&](const uint8_t* tile, int c) {
                const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + c * 16 * kKBlk + k_lo);
                const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + c * 16 * kKBlk + (k_lo ^ 32));
                i32x8 r;
                r.s0 = lo.x; r.s1 = lo.y; r.s2 = lo.z; r.s3 = lo.w;
                r.s4 = hi.x; r.s5 = hi.y; r.s6 = hi.z; r.s7 = hi.w;
                return r;
            };
            auto a_frag = [&](int c) {
                if constexpr (A_MK) return k_frag(st, c);
                else return tr_frag(a_lane, c, a_x, BM);
            };
            auto b_frag = [&](int c) {
                if constexpr (B_NK) return k_frag(st + Cfg::A_BYTES, c);
                else return tr_frag(b_lane, c, b_x, BN);
            };
            i32x8 bfrag[SN];
#pragma unroll
            for (int j = 0; j < SN; ++j)
                bfrag[j] = b_frag((wn * Cfg::WTN) / 16 + j);
            i32x8 afrag = a_frag((wm * Cfg::WTM) / 16);
            // Block products t = SN * i + j in order; the promotion of product t
            // runs after product t + 2 is issued (three results in flight).
            auto promote = [&](const f32x4& pr, int i, int j) {
                const float s = sa[i];
                acc[i][j].x = __builtin_fmaf(pr.x, s * sb[j].x, acc[i][j].x);
                acc[i][j].y = __builtin_fmaf(pr.y, s * sb[j].y, acc[i][j].y);
                acc[i][j].z = __builtin_fmaf(pr.z, s * sb[j].z, acc[i][j].z);
                acc[i][j].w = __builtin_fmaf(pr.w, s * sb[j].w, acc[i][j].w);
            };
            f32x4 pbuf[3];
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                i32x8 anext;
                if (i + 1 < SM) anext = a_frag((wm * Cfg::WTM) / 16 + i + 1);
                if constexpr (UE8M0) {
#pragma unroll
                    for (int j = 0; j < SN; ++j) {
                        acc[i][j] = mfma_e4m3_block_ue8m0(bfrag[j], afrag, acc[i][j], eb[j], ea[i]);
                        asm volatile("" : "+v"(acc[i][j]));   // keeps the product in place
                    }
                    if (i + 1 < SM) afrag = anext;
                    __builtin_amdgcn_sched_barrier(0);
                } else {
#pragma unroll
                    for (int j = 0; j < SN; ++j) {
                        const int t = SN * i + j;
                        pbuf[t % 3] = mfma_e4m3_block(bfrag[j], afrag);
                        if (t >= 2) promote(pbuf[(t - 2) % 3], (t - 2) / SN, (t - 2) % SN);
                    }
                    if (i + 1 < SM) afrag = anext;
                    // Issue order: the next A fragment's reads, then each block
                    // product followed by the promotion of the product two back.
                    __builtin_amdgcn_sched_group_barrier(0x100, A_MK ? 2 : 4, 0);   // the A fragment's DS reads
#pragma unroll
                    for (int j = 0; j < SN; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // 8 VALU
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (!UE8M0) {
                constexpr int T = SM * SN;
                promote(pbuf[(T - 2) % 3], (T - 2) / SN, (T - 2) % SN);
                promote(pbuf[(T - 1) % 3], (T - 1) / SN, (T - 1) % SN);
            }
        }
        // every wave is past its last LDS read before the next tile's copies
        lds_barrier();

        if (GROUPED_M || (!OUT_F32 && p.c == nullptr)) {
            // bf16 out without C (M-grouped NN always; the dense layouts when no
            // C is given): every accumulator is rounded to bf16 before staging
            // (the same single rounding as below, so the same bits), and the
            // whole 128 KB tile goes through LDS in one phase.
            // Row r holds 32 16-byte chunks, chunk c at position c ^ (r & 15);
            // a lane's 8-byte write (4 columns of one row) goes to half
            // ((lane >> 4) & 1) ^ ((r >> 3) & 1) of its chunk and the reads swap
            // the halves back.  An 8-byte LDS write is served in groups of 16
            // consecutive lanes that must hit 16 distinct 8-byte slots modulo
            // 128 bytes; a group's 16 consecutive rows differ in r & 7 and in
            // bit 3, which gives the 16 slots.  The row reads take 32 distinct
            // chunks of one row per half-wave.  Each store writes two rows.
            static_assert(BM == 256 && BN == 256 && Cfg::WAVES == 8, "256 x 256 tiles from 8 waves");
            uint8_t* const stg8 = smem;
            const int lane_e = opaque(tid) & 63;
            const int r16_e = lane_e & 15;
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int rl = wm * Cfg::WTM + 16 * i + r16_e;
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const int c = (wn * Cfg::WTN + 16 * j) / 8 + (lane_e >> 5);
                    const int hx = ((lane_e >> 4) & 1) ^ ((rl >> 3) & 1);
                    *reinterpret_cast<i32x2*>(stg8 + rl * 512 + 16 * (c ^ (rl & 15)) + 8 * hx) =
                        pack_bf16x4(acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w);
                }
            }
            lds_barrier();
#pragma unroll 4
            for (int k = 0; k < BM / 16; ++k) {
                const int half = lane_e >> 5;
                const int rl = wave + 16 * k + 8 * half;
                const int c = lane_e & 31;
                i32x4 v = *reinterpret_cast<const i32x4*>(stg8 + rl * 512 + 16 * (c ^ (rl & 15)));
                if ((rl >> 3) & 1) v = i32x4{v.z, v.w, v.x, v.y};   // halves stored swapped
                const int m = m0 + rl;
                const int n = n0 + 8 * c;
                const int e0 = __builtin_amdgcn_readlane(row_expert, 2 * k);
                const int e1 = __builtin_amdgcn_readlane(row_expert, 2 * k + 1);
                if (m >= p.M || n >= p.N || (GROUPED_M && (half ? e1 : e0) != e)) continue;   // padding rows
                const int64_t off = gbase + (int64_t)m * p.N + n;
                __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.d) + off));
            }
            // every wave is done reading the staged rows before the next tile's copies
            lds_barrier();
        } else {
            // Epilogue: D[g] = acc (C already included), fp32, inside [M, N],
            // staged through LDS one wave row (WTM tile rows) at a time so that
            // each store instruction writes one whole row (lane q: 16-byte chunk
            // q).  Chunk c of staged row r sits at position c ^ (r & 15): the 16
            // lanes that write one chunk column hold 16 consecutive rows, so both
            // the writes and the row reads hit 16 distinct 16-byte bank slots.
            // D is written once and never read here: nontemporal stores.
            float* const stg = reinterpret_cast<float*>(smem);
            constexpr int ROW_CHUNKS = BN / 4;
            static_assert(ROW_CHUNKS == 64, "one row per store instruction");
            const int lane_e = opaque(tid) & 63;   // the epilogue's offsets derive from it
            const int r16_e = lane_e & 15;
            static_assert(Cfg::WTM * BN * 4 <= Cfg::STAGES * Cfg::STAGE_BYTES, "a wave row of the tile fits in LDS");
#pragma unroll
            for (int ph = 0; ph < Cfg::WAVES_M; ++ph) {
                if (wm == ph) {
#pragma unroll
                    for (int i = 0; i < SM; ++i) {
                        const int rl = 16 * i + r16_e;
#pragma unroll
                        for (int j = 0; j < SN; ++j) {
                            const int ch = (wn * Cfg::WTN + 16 * j) / 4 + (lane_e >> 4);
                            *reinterpret_cast<f32x4*>(stg + rl * BN + 4 * (ch ^ (rl & 15))) = acc[i][j];
                        }
                    }
                }
                lds_barrier();
#pragma unroll 4
                for (int rl = wave; rl < Cfg::WTM; rl += Cfg::WAVES) {
                    const int m = m0 + ph * Cfg::WTM + rl;
                    const int n = n0 + 4 * lane_e;
                    if (m >= p.M || n >= p.N) continue;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rl * BN + 4 * (lane_e ^ (rl & 15)));
                    const int64_t off = gbase + (int64_t)m * p.N + n;
                    if constexpr (OUT_F32)
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(p.d) + off));
                    else
                        __builtin_nontemporal_store(pack_bf16x4(v.x, v.y, v.z, v.w),
                                                    reinterpret_cast<i32x2*>(static_cast<uint16_t*>(p.d) + off));
                }
                // every wave is done reading the staged rows before they (or the
                // next tile's copies) are overwritten
                lds_barrier();
            }
        }
    }
}

namespace {

using TnCfg256 = TnCfg<256, 256, 2, 4, 2>;

// The XCD blocks of a tiles_m x tiles_n group: 8 equal blocks (one per XCD)
// whose side lengths divide the grid, chosen to need the fewest panels per
// XCD (xcd_bm + xcd_bn); 0, 0 (column order) when the group's tiles do not
// split that way or `enable` is false.
void xcd_blocks(int tiles_m, int tiles_n, bool enable, int* xcd_bm, int* xcd_bn) {
    *xcd_bm = *xcd_bn = 0;
    if (!enable || tiles_m <= 0 || tiles_n <= 0 || (int64_t)tiles_m * tiles_n % 8 != 0) return;
    int best = INT_MAX;
    for (int bxm = 1; bxm <= 8; bxm *= 2) {
        const int bxn = 8 / bxm;
        if (tiles_m % bxm || tiles_n % bxn) continue;
        const int cost = tiles_m / bxm + tiles_n / bxn;
        if (cost < best) {
            best = cost;
            *xcd_bm = tiles_m / bxm;
            *xcd_bn = tiles_n / bxn;
        }
    }
}

template <class Cfg, bool A_MK, bool B_NK, bool OUT_F32, bool GROUPED_M, bool UE8M0 = false>
hipError_t launch_tn_cfg(const TnProblem& pr, int cu_cap, hipStream_t stream) {
    TnArgs a;
    a.a = pr.a; a.sfa = pr.sfa; a.b = pr.b; a.sfb = pr.sfb; a.c = pr.c; a.d = pr.d;
    a.m_indices = pr.m_indices;
    a.M = (int)pr.M; a.N = (int)pr.N; a.G = (int)pr.G;
    a.K = (int)pr.K_tot;
    a.tiles_m = (int)((pr.M + Cfg::BM - 1) / Cfg::BM);
    a.tiles_n = (int)((pr.N + Cfg::BN - 1) / Cfg::BN);
    // K-grouped: every group's tiles; dense: one group spanning K; M-grouped:
    // every tile twice, once per 128-row block's expert (read on the device)
    const int64_t groups = pr.form == kKGrouped ? pr.G : (pr.form == kMGroupedNN ? 2 : 1);
    const int64_t tiles = groups * a.tiles_m * a.tiles_n;
    if (tiles <= 0) return hipSuccess;
    a.num_tiles = (int)tiles;
    xcd_blocks(a.tiles_m, a.tiles_n, pr.form != kMGroupedNN, &a.xcd_bm, &a.xcd_bn);
    if (pr.form == kKGrouped) {
        int32_t start = 0, words = 0;
        for (int g = 0; g < a.G; ++g) {
            a.kb_start[g] = start;
            a.kb_count[g] = pr.k_sizes_host[g] / kKBlk;
            a.kw_start[g] = words;
            start += a.kb_count[g];
            words += (a.kb_count[g] + 3) / 4;
        }
    } else {
        a.kb_start[0] = 0;
        a.kb_count[0] = (int32_t)(pr.K_tot / kKBlk);
        a.kw_start[0] = 0;
    }
    const int n_order = pr.form == kKGrouped ? (int)groups : 1;
    // Longest-processing-time order: groups with the most K blocks first.
    std::iota(a.order, a.order + n_order, 0);
    std::stable_sort(a.order, a.order + n_order,
                     [&](int x, int y) { return a.kb_count[x] > a.kb_count[y]; });

    const int64_t resident = (int64_t)cu_cap * Cfg::WG_PER_CU;
    const int grid = (int)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL((tn_fp8_kernel<Cfg, A_MK, B_NK, OUT_F32, GROUPED_M, UE8M0>), dim3(grid),
                       dim3(Cfg::THREADS), 0, stream, a);
    return hipGetLastError();
}

template <bool A_MK, bool B_NK>
hipError_t launch_dense_layout(const TnProblem& pr, int cu_cap, hipStream_t stream) {
    return pr.out_f32 ? launch_tn_cfg<TnCfg256, A_MK, B_NK, true, false>(pr, cu_cap, stream)
                      : launch_tn_cfg<TnCfg256, A_MK, B_NK, false, false>(pr, cu_cap, stream);
}

}  // namespace

hipError_t launch_tn(const TnProblem& pr, int cu_cap, hipStream_t stream) {
    switch (pr.form) {
    case kKGrouped:
        return pr.ue8m0 ? launch_tn_cfg<TnCfg256, false, false, true, false, true>(pr, cu_cap, stream)
                        : launch_tn_cfg<TnCfg256, false, false, true, false>(pr, cu_cap, stream);
    case kMGroupedNN:
        return launch_tn_cfg<TnCfg256, true, false, false, true>(pr, cu_cap, stream);
    case kDenseLayout:
        if (pr.a_mk && !pr.b_nk) return launch_dense_layout<true, false>(pr, cu_cap, stream);
        if (!pr.a_mk && !pr.b_nk) return launch_dense_layout<false, false>(pr, cu_cap, stream);
        if (!pr.a_mk && pr.b_nk) return launch_dense_layout<false, true>(pr, cu_cap, stream);
        return hipErrorInvalidValue;   // NT is the NT kernel's
    }
    return hipErrorInvalidValue;
}

const char* tn_config_name(const TnProblem& pr) {
    if (pr.form == kKGrouped) return pr.ue8m0 ? "tn_kgrouped_f32_ue8m0_256x256" : "tn_kgrouped_f32_256x256";
    if (pr.form == kMGroupedNN) return "nn_contiguous_bf16_256x256";
    static thread_local char buf[64];
    snprintf(buf, sizeof buf, "%s_dense_%s_256x256",
             pr.a_mk ? (pr.b_nk ? "nt" : "nn") : (pr.b_nk ? "tt" : "tn"),
             pr.out_f32 ? "f32" : "bf16");
    return buf;
}

const char* describe_tn_config(const TnProblem& pr) {
    static thread_local char buf[192];
    snprintf(buf, sizeof buf, "%s G=%lld M=%lld N=%lld K_tot=%lld", tn_config_name(pr),
             (long long)pr.G, (long long)pr.M, (long long)pr.N, (long long)pr.K_tot);
    return buf;
}

}  // namespace dg
