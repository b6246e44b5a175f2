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
//     LDS by direct global -> LDS copies (a ring of STAGES stages: the copies
//     of the next blocks are in flight while block kb is multiplied), rows of
//     128 bytes with an XOR-swizzled 16-byte chunk order.
//   * The epilogue stages the tile through the idle stages and writes D in
//     whole-row stores: dense tiles in fp32 (+ C, then one rounding), the
//     grouped forms' 256 x 256 tiles (bf16, no C) already rounded to bf16.
//   * Each wave owns a WTM x WTN sub-tile made of 16 x 16 MFMA tiles.  The MFMA
//     takes the B fragment as its row operand and the A fragment as its column
//     operand, so every lane's four results share one m (one A scale) and
//     cover four consecutive n.
//   * Promotion: acc += P * (sa[kb][m] * sb[nb][kb]) in fp32 VGPRs, kb
//     ascending.  bf16 (or fp32) conversion happens once, in the epilogue.
#include "dg_internal.h"
#include "tile_common.h"

#include <stdio.h>

#include <mutex>
#include <type_traits>

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
    int band_m;        // grouped rasterisation: bands of band_m M tiles
    int xcd_remap;     // 1: give each XCD a contiguous run of the tile order
    // Contiguous form: the first xcd_units tiles go in XCD blocks (each XCD
    // takes xcd_blk_m M tiles x tiles_n / 2 N tiles per round of the grid);
    // the band order covers the rest, from M tile xcd_m0 on.
    int xcd_blk_m;
    int xcd_units;
    int xcd_m0;
    // Split K (dense only): each output tile is computed as `splits` partial
    // sums over consecutive K-block ranges; see the epilogue.
    int splits;
    // 1: every B row is read by exactly one tile (one M tile per group), so
    // the B copies use the nontemporal cache policy
    int b_nt;
    float* part;       // [tiles][splits][SM * SN * 4][THREADS] fp32 partials
    int32_t* counters; // [tiles], zero between launches
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct NtCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int STAGES = STAGES_;     // LDS stages (STAGES - 1 K blocks in flight)
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WAVES_M;   // wave tile rows (m)
    static constexpr int WTN = BN / WAVES_N;   // wave tile columns (n)
    static constexpr int SM = WTM / 16;        // 16-row MFMA tiles per wave along m
    static constexpr int SN = WTN / 16;        // along n
    static constexpr int A_BYTES = BM * kKBlk;
    static constexpr int B_BYTES = BN * kKBlk;
    static constexpr int SA_BYTES = BM * 4;    // this tile's A scales for the stage's K block
    static constexpr int SB_BYTES = 256 * WAVES;   // one copy of the tile's B scales per wave
    static constexpr int SA_OFF = A_BYTES + B_BYTES;
    static constexpr int SB_OFF = SA_OFF + SA_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int SA_DMA = BM / 64;     // 256-byte (64-float) wave copies per stage
    static constexpr int A_DMA = BM / 8;       // 1 KiB (8-row) wave copies per stage for A
    static constexpr int B_DMA = BN / 8;
    static constexpr int DMA_PER_WAVE = (A_DMA + B_DMA) / WAVES;
    static constexpr int VM_PER_STAGE = DMA_PER_WAVE + 1;   // copies a wave issues per stage
    static_assert(STAGES >= 2 && (STAGES - 2) * VM_PER_STAGE <= 63, "vmcnt range");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert((A_DMA + B_DMA) % WAVES == 0, "stage copies must split evenly over waves");
    static_assert(SA_DMA >= 1 && SA_DMA <= WAVES, "one scale copy per wave at most");
    static_assert(BN % kKBlk == 0 || kKBlk % BN == 0, "tiles align with 128-column B scale blocks");
    static_assert(SM % 4 == 0, "a lane reads its A scales as float4s");
    // Split K is compiled in for tiles whose partial sums fit the batched
    // reduction in registers (up to 16 MFMA tiles per lane).
    static constexpr bool SPLIT_OK = SM * SN <= 16;
    // Early B refill (two stages): when every wave copies only A rows with the
    // A scales, or only B rows with the B scales, the B half of a stage is
    // refilled as soon as its fragments are in registers (one barrier earlier
    // than the A half), so B copies have about two K blocks to land.
    static constexpr bool EARLY_B =
        STAGES == 2 && A_DMA % DMA_PER_WAVE == 0 && SA_DMA * DMA_PER_WAVE == A_DMA;
    static_assert(kKBlk % WTN == 0 && (BN % kKBlk == 0 || kKBlk % BN == 0),
                  "a wave's columns must sit inside one 128-column B scale block");
    // Whole-block prefetch (wave tiles of at most 8 MFMA tiles): with so few
    // products per K block, a row-by-row fragment pipeline leaves the MFMA
    // unit waiting on LDS latency and barriers.  Instead every operand of
    // block kb + 1 is read into a second register set while block kb's
    // products run, one barrier per block.
    static constexpr bool FULL_PREFETCH = SM * SN <= 8;
    // Epilogue staging: wave rows (of WTM tile rows) staged per phase; all of
    // them when the fp32 tile fits in the stages, else one at a time.
    static constexpr int EPI_WAVE_ROWS =
        WAVES_M * WTM * BN * 4 <= STAGES * STAGE_BYTES ? WAVES_M : 1;
    static_assert(WTM * BN * 4 <= STAGES * STAGE_BYTES, "one wave row of the fp32 tile fits in LDS");
    static_assert(BN % 16 == 0 && 64 % (BN / 4) == 0 && (WTM * EPI_WAVE_ROWS) % (64 / (BN / 4)) == 0,
                  "staged rows split evenly into wave instructions");
    static_assert(!(FULL_PREFETCH && EARLY_B), "whole-block prefetch uses the plain stage ring");
    // Workgroups resident per CU: bounded by the 160 KiB of LDS and by the
    // two waves per SIMD every instance is compiled for (8 waves per CU).
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + 256 * WAVES;
    static constexpr int WG_PER_CU =
        (160 * 1024 / LDS_BYTES) < (8 / WAVES) ? (160 * 1024 / LDS_BYTES) : (8 / WAVES);
    static_assert(WG_PER_CU >= 1, "one workgroup fits a CU");
};

// Row and LDS maps.
//  * Lane l (r = l & 15) of a wave owns the SM consecutive rows SM r .. SM r +
//    SM - 1 of its wave tile; MFMA tile i of the lane reads row SM r + (i ^ (r & 1))
//    (odd lanes swap neighbouring rows), so the 16 rows of a fragment cover
//    both parities.  Columns follow the MFMA layout: tile j, lane l owns the
//    four columns 16 j + 4 (l >> 4) + {0, 1, 2, 3}.
//  * LDS holds 128-byte rows (one K block of one row); chunk c of row `row`
//    sits at 16-byte position sigma(c) ^ f(row), with f_A(row) = (row / 2SM) & 7
//    for the A tile, f_B(row) = (row / 2) & 7 for the B tile, and sigma swapping
//    bits 0 and 1 of c.
//  * Bank rule (measured on gfx950): a ds_read_b128 is served in four groups
//    of 16 lanes, lane l in group 2 * bit5(l) + (bit2 ^ bit3 ^ bit4)(l), and a
//    group is conflict-free when its lanes hit 16 distinct 16-byte slots modulo
//    256 bytes.  A group holds each fragment row r once, half of them reading
//    chunk 2q (+1) and half chunk 2q + 2 (+1); sigma makes those two chunks
//    differ in position bit 0 only, so row parity, f and that bit together
//    give 16 distinct slots.  Every fragment address is a per-lane base plus
//    an immediate (i * 128 for A, j * 2048 for B).
//  * A scales: the lane's scale for fragment i sits at float
//    (i / 4) * 64 + 4 r + i % 4 of its wave's block, so each float4 read of a
//    16-lane group covers 256 contiguous bytes.
__device__ __forceinline__ int sigma(int c) { return ((c >> 1) & 1) | ((c & 1) << 1) | (c & 4); }
template <int SM>
__device__ __forceinline__ int pos_a(int row) { return (row / (2 * SM)) & 7; }
__device__ __forceinline__ int pos_b(int row) { return (row >> 1) & 7; }

template <class Cfg, int FORM, bool OUT_F32, bool UE8M0>
__global__ __launch_bounds__(Cfg::THREADS) __attribute__((amdgpu_waves_per_eu(2))) void nt_fp8_kernel(NtArgs p) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    constexpr int SM = Cfg::SM, SN = Cfg::SN;
    // UE8M0: the B-scale words of a stage, one per tile column, fill the
    // 256-byte slots of the waves that do not copy A scales.
    static_assert(!UE8M0 || BN <= 64 * (Cfg::WAVES - Cfg::SA_DMA), "B-scale words fit the slots");
    // stages, then one 256-byte slot per wave that absorbs placeholder copies
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::STAGES * Cfg::STAGE_BYTES +
                                                           256 * Cfg::WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;
    const int KB = p.K / kKBlk;
    const int NB = (p.N + kKBlk - 1) / kKBlk;
    const int K4 = (KB + 3) / 4;   // UE8M0: packed scale words per row
    const int per_group = p.tiles_m * p.tiles_n;

    // Masked groups: only the tiles holding valid rows are enumerated.  Group
    // g has ceil(masked_m[g] / BM) * tiles_n of them; every workgroup reads
    // the counts (device memory, so a captured graph sees the values of each
    // replay) and walks the live tiles round-robin, which balances the work.
    int num_work = p.num_tiles;
    if (FORM == kMasked) {
        num_work = 0;
        for (int gg = 0; gg < p.G; ++gg) {
            const int mm = min(max(p.masked_m[gg], 0), p.rows);
            num_work += ((mm + BM - 1) / BM) * p.tiles_n;
        }
    }

    for (int t = blockIdx.x; t < num_work; t += gridDim.x) {
        // ---- tile scheduling (uniform over the workgroup) ------------------
        int g = 0, e = 0, local = t, half = 0, split = 0;
        int mtiles = 0;   // masked: live M tiles of group g
        if (FORM == kMasked) {
            for (g = 0; g < p.G; ++g) {
                const int mm = min(max(p.masked_m[g], 0), p.rows);
                mtiles = (mm + BM - 1) / BM;
                const int cnt = mtiles * p.tiles_n;
                if (local < cnt) break;
                local -= cnt;
            }
            e = g;
        } else if (FORM == kContiguous) {
            // Tiles of BM = 256 rows span two 128-row expert blocks: the tile is
            // listed twice, pass `half` computing it with the expert of block
            // `half` (pass 1 only when that expert differs from block 0's).
            half = t / per_group;
            local = t - half * per_group;
        }
        // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so
        // with a grid that is a multiple of 8, tile t runs on XCD t % 8.  The
        // remap gives each XCD one contiguous run of the raster order, so the
        // tiles an XCD has in flight together share A and B panels in its L2.
        if (FORM == kDense && p.xcd_remap) {
            const int per = p.num_tiles >> 3, extra = p.num_tiles & 7;
            const int x = t & 7;
            local = x * per + min(x, extra) + (t >> 3);
        }
        if (FORM == kDense) {
            split = local % p.splits;
            local /= p.splits;
        }
        const int tile_id = local;
        int tm, tn;
        if (FORM == kMasked) {
            // Runs of 8 N tiles x all live M tiles: the M tiles that share a
            // B panel are 8 apart in t, hence on one XCD (t % 8) and in flight
            // together, so the panel comes from HBM once.
            const int run = 8 * mtiles;
            const int nfull = p.tiles_n >> 3;
            if (local < nfull * run) {
                const int blk = local / run, r = local - blk * run;
                tm = r >> 3;
                tn = blk * 8 + (r & 7);
            } else {
                const int r = local - nfull * run, w = p.tiles_n - nfull * 8;
                tm = r / w;
                tn = nfull * 8 + r % w;
            }
        } else if (FORM == kContiguous && local < p.xcd_units) {
            // XCD blocks: one round of the grid (gridDim.x units, a multiple
            // of 8) covers 4 * xcd_blk_m M tiles x all N tiles; unit u runs on
            // XCD u % 8, which takes a block of xcd_blk_m M tiles x half the
            // N tiles (4 x 2 blocks).  Fewer panels per XCD than a band of the
            // same size: 12 instead of 18 at 32 tiles per XCD and 16 N tiles.
            const int sb = local / (int)gridDim.x;
            const int u = local - sb * (int)gridDim.x;
            const int x = u & 7, j = u >> 3;
            tm = (sb * 4 + (x & 3)) * p.xcd_blk_m + j % p.xcd_blk_m;
            tn = (x >> 2) * (p.tiles_n >> 1) + j / p.xcd_blk_m;
        } else {
            // Grouped rasterisation: tiles run in bands of band_m M tiles;
            // inside a band N advances after every M tile of the band, so the
            // tiles in flight share a few A row panels and B column panels.
            const int rest = local - p.xcd_units;
            const int band_tiles = p.band_m * p.tiles_n;
            const int band = rest / band_tiles;
            const int in_band = rest - band * band_tiles;
            const int first_m = p.xcd_m0 + band * p.band_m;
            const int rows_in_band = min(p.tiles_m - first_m, p.band_m);
            tm = first_m + in_band % rows_in_band;
            tn = in_band / rows_in_band;
        }
        const int r0 = tm * BM;        // first row of the tile, relative to its group
        const int n0 = tn * BN;
        const int grp_rows = p.rows;   // rows that exist in memory for this group
        int store_rows = p.rows;       // rows that may be written
        int64_t grp_row0 = 0;          // first row of the group in A / D
        if (FORM == kMasked) {
            int mm = p.masked_m[g];
            mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
            store_rows = mm;
            grp_row0 = (int64_t)g * p.rows;
        } else if (FORM == kContiguous) {
            const int rb = r0 + half * kKBlk;   // first row of the block whose expert is used
            if (rb >= p.rows) continue;
            e = p.m_indices[rb];
            if (e < 0 || e >= p.G) continue;
            if (half == 1 && p.m_indices[r0] == e) continue;   // pass 0 already covers it
        }
        // this tile's prologue derives its lane offsets from a fresh copy of
        // the thread index (not hoisted out of the tile loop, so not kept live
        // across the K loop)
        const int lane_t = opaque(tid) & 63;
        // Contiguous groups: the expert of every row this wave stores in the
        // epilogue, requested now so its latency hides under the K loop.  With
        // two rows per store instruction, wave w stores tile rows w + 8 j
        // (j = 0 .. 31); lane j holds that row's expert.
        int row_expert = -1;
        if constexpr (FORM == kContiguous && BN == 256) {
            static_assert(Cfg::WAVES == 8 && BM == 256, "row map of the contiguous epilogue");
            const int row = r0 + wave + 8 * (lane_t & 31);
            if (row < p.rows) row_expert = p.m_indices[row];
        }

        // Contiguous passes: bit b is set when the tile's 128-row block b holds
        // rows of expert e (a block belongs to one expert or is padding).  The
        // other block's rows are not stored in this pass: its A copies shrink to
        // placeholders (as rows past masked_m do) and its waves compute nothing.
        int live_blk = (1 << (BM / kKBlk)) - 1;
        if constexpr (FORM == kContiguous) {
            live_blk = 0;
#pragma unroll
            for (int bb = 0; bb < BM / kKBlk; ++bb) {
                const int rb = r0 + bb * kKBlk;
                if (rb < p.rows && p.m_indices[rb] == e) live_blk |= 1 << bb;
            }
            live_blk = __builtin_amdgcn_readfirstlane(live_blk);
        }

        // K blocks [kb_lo, kb_lo + nkb) of this work unit (all of K unless split)
        const int kb_lo = (int)(((int64_t)split * KB) / p.splits);
        const int nkb = (int)(((int64_t)(split + 1) * KB) / p.splits) - kb_lo;
        const uint8_t* __restrict__ a_t = p.a + grp_row0 * p.K;
        const uint8_t* __restrict__ b_t = p.b + (int64_t)e * p.N * p.K;
        // scale rows per group: KB fp32 scales, or K4 packed UE8M0 words
        const int sf_k = UE8M0 ? K4 : KB;
        const float* __restrict__ sfa_t = p.sfa + (FORM == kMasked ? (int64_t)g * sf_k * p.rows : 0);
        const float* __restrict__ sfb_t =
            p.sfb + (int64_t)e * (UE8M0 ? (int64_t)K4 * p.N : (int64_t)NB * KB);

        // Stage copies: wave copy u (uniform) moves 8 rows x 128 bytes; lane l
        // fetches chunk (l & 7) ^ f(row) of row 8 u' + (l >> 3), so LDS
        // position p of a row holds chunk p ^ f(row).  Rows past the edge re-read
        // the last row (never stored).
        uint32_t goff[Cfg::DMA_PER_WAVE];
#pragma unroll
        for (int q = 0; q < Cfg::DMA_PER_WAVE; ++q) {
            const int u = wave * Cfg::DMA_PER_WAVE + q;
            const bool is_a = u < Cfg::A_DMA;
            const int lrow = 8 * (is_a ? u : u - Cfg::A_DMA) + (lane_t >> 3);
            const int chunk = sigma((lane_t & 7) ^ (is_a ? pos_a<SM>(lrow) : pos_b(lrow)));
            const int row = is_a ? min(r0 + lrow, grp_rows - 1) : min(n0 + lrow, p.N - 1);
            goff[q] = (uint32_t)row * (uint32_t)p.K + (uint32_t)(chunk * 16);
        }
        // Scales.  Every wave issues exactly one scale copy per stage (so all
        // waves count the same number of copies in flight): wave w < SA_DMA
        // copies A-scale slots [64 w, 64 w + 64), slot s holding the scale of
        // tile row s ^ ((s / SM) & 1) (the pair swap of the row map); every
        // other wave copies the B scales of the tile's 128-column blocks into
        // its own 256-byte slot (lanes past the last block repeat it).
        // A-scale slot t of the stage holds the scale of the row that lane
        // r = (u % 64) / 4 of wave-row wm reads as fragment i = 4 (u / 64) + u % 4
        // (u = t % WTM, wm = t / WTM)
        const int sa_slot = 64 * wave + lane_t;
        const int sa_u = sa_slot % Cfg::WTM, sa_r = (sa_u % 64) / 4;
        const int sa_row = (sa_slot / Cfg::WTM) * Cfg::WTM + SM * sa_r +
                           ((4 * (sa_u / 64) + (sa_u % 4)) ^ (sa_r & 1));
        const uint32_t sa_off = 4u * (uint32_t)min(r0 + sa_row, grp_rows - 1);
        const int nb_last = min(NB - 1, (n0 + BN - 1) / kKBlk);   // the tile's last B-scale block
        // UE8M0: wave w >= SA_DMA copies the words of tile columns
        // 64 (w - SA_DMA) + lane (clamped to the last column) into slot w - SA_DMA
        const uint32_t sb_off =
            UE8M0 ? 4u * (uint32_t)min(n0 + 64 * max(wave - Cfg::SA_DMA, 0) + lane_t, p.N - 1)
                  : 4u * (uint32_t)(min(n0 / kKBlk + lane_t, nb_last) * KB);
        const uint32_t lds0 = lds_addr(smem);
        auto issue_stage = [&](int kbr, int stage) {
            const int kb = kb_lo + kbr;
            const uint32_t dst = lds0 + stage * Cfg::STAGE_BYTES;
#pragma unroll
            for (int q = 0; q < Cfg::DMA_PER_WAVE; ++q) {
                const int u = wave * Cfg::DMA_PER_WAVE + q;
                const uint8_t* src = (u < Cfg::A_DMA ? a_t : b_t) + (size_t)kb * kKBlk;
                // Masked groups: A rows at or past masked_m are never stored,
                // so their copy shrinks to a 256-byte placeholder (every wave
                // keeps the same number of copies per stage, which the waits
                // count on); so do the A rows of a contiguous pass's other block.
                if ((FORM == kMasked && u < Cfg::A_DMA && r0 + 8 * u >= store_rows) ||
                    (FORM == kContiguous && u < Cfg::A_DMA && !((live_blk >> ((8 * u) / kKBlk)) & 1)))
                    dma4(src, 0, lds0 + Cfg::STAGES * Cfg::STAGE_BYTES + wave * 256);
                else if (u >= Cfg::A_DMA && p.b_nt)
                    dma16_nt(src, goff[q], dst + u * 1024);
                else
                    dma16(src, goff[q], dst + u * 1024);
            }
            if constexpr (UE8M0) {
                // word kb / 4 of each row holds block kb's exponent in byte kb % 4
                if (wave < Cfg::SA_DMA)
                    dma4(sfa_t + (size_t)(kb >> 2) * grp_rows, sa_off, dst + Cfg::SA_OFF + wave * 256);
                else
                    dma4(sfb_t + (size_t)(kb >> 2) * p.N, sb_off,
                         dst + Cfg::SB_OFF + (wave - Cfg::SA_DMA) * 256);
            } else {
                if (wave < Cfg::SA_DMA)
                    dma4(sfa_t + (size_t)kb * grp_rows, sa_off, dst + Cfg::SA_OFF + wave * 256);
                else
                    dma4(sfb_t + kb, sb_off, dst + Cfg::SB_OFF + wave * 256);
            }
        };

        const int r16 = lane & 15;
        // per-lane LDS byte offsets inside a stage (fragment i / j adds an immediate)
        const int c0 = (lane >> 4) * 2;
        const int pa = pos_a<SM>(wm * Cfg::WTM + SM * r16);
        const int a_even = (wm * Cfg::WTM + SM * r16 + (r16 & 1)) * kKBlk;
        const int a_odd = (wm * Cfg::WTM + SM * r16 - (r16 & 1)) * kKBlk;
        const int a_lo = (sigma(c0) ^ pa) << 4, a_hi = (sigma(c0 + 1) ^ pa) << 4;
        const int pb = pos_b(wn * Cfg::WTN + r16);
        const int b_row = Cfg::A_BYTES + (wn * Cfg::WTN + r16) * kKBlk;
        const int b_lo = b_row + ((sigma(c0) ^ pb) << 4), b_hi = b_row + ((sigma(c0 + 1) ^ pb) << 4);
        const int s_a = Cfg::SA_OFF + 4 * (wm * Cfg::WTM + 4 * r16);
        const int s_b = Cfg::SB_OFF + 256 * (Cfg::WAVES - 1) + 4 * ((wn * Cfg::WTN) / kKBlk);
        const int s_be = Cfg::SB_OFF + 4 * (wn * Cfg::WTN + r16);   // UE8M0: word of B fragment 0

        // Whether this wave's tile rows (WTM rows from r0 + wm * WTM) hold any
        // row the pass stores: masked groups store rows below masked_m;
        // contiguous passes store the rows of expert e, and a wave's rows are
        // one 128-row block (live_blk); dense tiles store rows below M.
        bool wave_live = true;
        {
            const int rw = r0 + wm * Cfg::WTM;
            if (FORM == kMasked) wave_live = rw < store_rows;
            else if (FORM == kContiguous) wave_live = (live_blk >> wm) & 1;
            else wave_live = rw < p.rows;
            wave_live = __builtin_amdgcn_readfirstlane((int)wave_live) != 0;
        }
        static_assert(FORM != kContiguous || Cfg::WTM == kKBlk, "a wave's rows are one expert block");
        f32x4 acc[SM][SN];
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j)
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Stage ring: block kb lives in stage kb % STAGES.  The prologue puts
        // blocks 0 .. STAGES-1 in flight (the last one once block 0 has landed
        // and the barrier has passed); iteration it, once every wave is done
        // reading block it, refills its stage with block it + STAGES.
        const bool a_wave = wave < Cfg::SA_DMA;   // EARLY_B: this wave copies A (else B)
        if constexpr (Cfg::EARLY_B) {
            // blocks 0 (A and B) and 1 (B) in flight; once block 0 has landed,
            // block 1's A
            if (nkb > 0) issue_stage(0, 0);
            if (!a_wave && nkb > 1) issue_stage(1, 1);
            if (!a_wave && nkb > 1) wait_vmcnt<Cfg::VM_PER_STAGE>();
            else wait_vmcnt<0>();
            lgkm_drain_barrier();
            if (a_wave && nkb > 1) issue_stage(1, 1);
        } else {
#pragma unroll
            for (int q = 0; q < Cfg::STAGES - 1; ++q)
                if (q < nkb) issue_stage(q, q);
            wait_stage_copies<Cfg::STAGES - 2, Cfg::VM_PER_STAGE>(min(Cfg::STAGES - 2, nkb - 1));
            lgkm_drain_barrier();
            if (Cfg::STAGES - 1 < nkb) issue_stage(Cfg::STAGES - 1, Cfg::STAGES - 1);
        }

        // Operand reads from one stage: scales, B fragments, A fragment i.
        auto load_scales = [&](const uint8_t* st, float (&sa)[SM], float& sb) {
#pragma unroll
            for (int i = 0; i < SM; i += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + s_a + 4 * 64 * (i / 4));
                sa[i] = v.x; sa[i + 1] = v.y; sa[i + 2] = v.z; sa[i + 3] = v.w;
            }
            sb = *reinterpret_cast<const float*>(st + s_b);
        };
        // UE8M0: the exponent bytes of K block kb (held by the stage `st`) for
        // the lane's SM A rows (same slots as the fp32 A scales) and its SN B
        // fragment rows.
        auto load_exps = [&](const uint8_t* st, int kb, int (&ea)[SM], int (&eb)[SN]) {
            const int sh = 8 * (kb & 3);
#pragma unroll
            for (int i = 0; i < SM; i += 4) {
                const i32x4 v = *reinterpret_cast<const i32x4*>(st + s_a + 4 * 64 * (i / 4));
                ea[i] = (v.x >> sh) & 0xFF; ea[i + 1] = (v.y >> sh) & 0xFF;
                ea[i + 2] = (v.z >> sh) & 0xFF; ea[i + 3] = (v.w >> sh) & 0xFF;
            }
#pragma unroll
            for (int j = 0; j < SN; ++j)
                eb[j] = (*reinterpret_cast<const int*>(st + s_be + 64 * j) >> sh) & 0xFF;
        };
        auto bfrag_at = [&](const uint8_t* st, int j) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(st + b_lo + j * 16 * kKBlk);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(st + b_hi + j * 16 * kKBlk);
            i32x8 r;
            r.s0 = lo.x; r.s1 = lo.y; r.s2 = lo.z; r.s3 = lo.w;
            r.s4 = hi.x; r.s5 = hi.y; r.s6 = hi.z; r.s7 = hi.w;
            return r;
        };
        auto afrag_at = [&](const uint8_t* st, int i) {
            const uint8_t* rowp = st + ((i & 1) ? a_odd : a_even) + i * kKBlk;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + a_lo);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + a_hi);
            i32x8 r;
            r.s0 = lo.x; r.s1 = lo.y; r.s2 = lo.z; r.s3 = lo.w;
            r.s4 = hi.x; r.s5 = hi.y; r.s6 = hi.z; r.s7 = hi.w;
            return r;
        };
        // acc[i][j] += pr * s for one MFMA result.  The empty asm pins the
        // result at this point of the instruction stream: without it the
        // compiler sinks the promotions past the stage-refill branch, where
        // they pile up and the products they wait on spill.
        auto promote1 = [&](int i, int j, const f32x4& pr, float s) {
            acc[i][j].x = __builtin_fmaf(pr.x, s, acc[i][j].x);
            acc[i][j].y = __builtin_fmaf(pr.y, s, acc[i][j].y);
            acc[i][j].z = __builtin_fmaf(pr.z, s, acc[i][j].z);
            acc[i][j].w = __builtin_fmaf(pr.w, s, acc[i][j].w);
            asm volatile("" : "+v"(acc[i][j]));
        };

        if constexpr (Cfg::FULL_PREFETCH) {
            // Block it's operands (cur) were requested during block it-1; the
            // barrier at the top of iteration it also covers block it+1 having
            // landed, so its operands (nxt) are requested before block it's
            // products, which hide their latency.  Products t = i * SN + j run in
            // order; each is promoted two products later (a two-entry ring), so
            // the last two of a block are promoted under the next block's first
            // two, with the scale of the block they came from.
            constexpr int T = SM * SN;
            // products are promoted R products later (four when the block's
            // product count allows; measured the same as two in the sweep)
            constexpr int R = (T % 4 == 0) ? 4 : 2;
            static_assert(T % R == 0, "the product ring divides the block");
            struct Ops {
                i32x8 a[SM];
                i32x8 b[SN];
                float sa[SM];
                float sb;
                int ea[SM];   // UE8M0 exponents
                int eb[SN];
            };
            auto read_ops = [&](const uint8_t* st, int kb, Ops& o) {
                if constexpr (UE8M0) load_exps(st, kb, o.ea, o.eb);
                else load_scales(st, o.sa, o.sb);
#pragma unroll
                for (int j = 0; j < SN; ++j) o.b[j] = bfrag_at(st, j);
#pragma unroll
                for (int i = 0; i < SM; ++i) o.a[i] = afrag_at(st, i);
            };
            Ops cur, nxt;
            read_ops(smem, kb_lo, cur);
            // nothing is pending before block 0: zero products with zero scale
            f32x4 ring[R];
            float ring_s[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                ring[r] = f32x4{0.f, 0.f, 0.f, 0.f};
                ring_s[r] = 0.f;
            }
            int stage = 0;   // stage holding block it
            for (int it = 0; it < nkb; ++it) {
                const int next = stage + 1 == Cfg::STAGES ? 0 : stage + 1;
                // block it+1 has landed for every wave, and every wave's reads of
                // block it (cur) are complete
                wait_stage_copies<Cfg::STAGES - 2, Cfg::VM_PER_STAGE>(
                    max(0, min(Cfg::STAGES - 2, nkb - 2 - it)));
                lgkm_drain_barrier();
                if (it + Cfg::STAGES < nkb) issue_stage(it + Cfg::STAGES, stage);
                if (it + 1 < nkb) read_ops(smem + next * Cfg::STAGE_BYTES, kb_lo + it + 1, nxt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int i = t / SN, j = t % SN;
                    if constexpr (UE8M0) {
                        __builtin_amdgcn_s_setprio(1);
                        acc[i][j] = mfma_e4m3_block_ue8m0(cur.b[j], cur.a[i], acc[i][j], cur.eb[j],
                                                          cur.ea[i]);
                        asm volatile("" : "+v"(acc[i][j]));   // keep the product in place
                        __builtin_amdgcn_s_setprio(0);
                    } else {
                        __builtin_amdgcn_s_setprio(1);
                        const f32x4 pr = mfma_e4m3_block(cur.b[j], cur.a[i]);
                        __builtin_amdgcn_s_setprio(0);
                        const int tp = t >= R ? t - R : T + t - R;   // tile of the pending product
                        promote1(tp / SN, tp % SN, ring[t % R], ring_s[t % R]);
                        ring[t % R] = pr;
                        ring_s[t % R] = cur.sa[i] * cur.sb;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                cur = nxt;
                stage = next;
            }
            if constexpr (!UE8M0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    promote1((T - R + r) / SN, (T - R + r) % SN, ring[(T - R + r) % R],
                             ring_s[(T - R + r) % R]);
            }
        } else {
            // Row pipeline.  Products t = i * SN + j run row by row; A fragment
            // i + 2 is requested at the start of row i (a four-entry ring, two
            // rows of LDS latency hidden), and each product is promoted two
            // products later through a two-entry ring, so a block's last two
            // products are promoted under the next block's first two, with the
            // scale of the block they came from.  The mid-block barrier comes
            // after row SM - 3, once every A read of the block has been issued:
            // past it, rows SM - 2 and SM - 1 request the next block's scales,
            // its first two A fragments and (after the last product that uses
            // each) its B fragments.
            // A wave whose tile rows hold nothing this pass stores (rows past
            // masked_m, another expert's block, rows past M) runs the same
            // copies, waits and barriers as the others but no fragment reads
            // and no products; its accumulators stay zero and are never stored.
            auto row_pipeline = [&](auto live_tag) {
                constexpr bool LIVE = decltype(live_tag)::value;
                constexpr int T = SM * SN;
                static_assert(SM % 4 == 0 && T % 2 == 0, "A ring of four rows, product ring of two");
                i32x8 af[4];
                i32x8 bfr[SN];
                float sa[SM], sb, sa_n[SM], sb_n;
                int ea[SM], eb[SN], ea_n[SM], eb_n[SN];   // UE8M0 exponents
                f32x4 ring[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                float ring_s[2] = {0.f, 0.f};   // nothing pending before block 0
                if constexpr (LIVE) {
                    if constexpr (UE8M0) load_exps(smem, kb_lo, ea, eb);
                    else load_scales(smem, sa, sb);
#pragma unroll
                    for (int j = 0; j < SN; ++j) bfr[j] = bfrag_at(smem, j);
                    af[0] = afrag_at(smem, 0);
                    af[1] = afrag_at(smem, 1);
                }

                // one product step: block product (i, j) (issued at raised wave
                // priority, so a wave with products ready keeps the MFMA unit busy
                // while its SIMD partner waits on LDS) and the promotion of the
                // product two steps back
                // (UE8M0: the MFMA applies the exponents and accumulates itself)
                auto step = [&](int i, int j, float s_row) {
                    if constexpr (!LIVE) {
                        return;
                    } else if constexpr (UE8M0) {
                        __builtin_amdgcn_s_setprio(1);
                        acc[i][j] = mfma_e4m3_block_ue8m0(bfr[j], af[i & 3], acc[i][j], eb[j], ea[i]);
                        // pins the product here: with nothing reading acc until the
                        // epilogue, the compiler would otherwise sink every product of
                        // the block past the LDS reads it is meant to overlap
                        asm volatile("" : "+v"(acc[i][j]));
                        __builtin_amdgcn_s_setprio(0);
                    } else {
                        const int t = i * SN + j;
                        __builtin_amdgcn_s_setprio(1);
                        const f32x4 pr = mfma_e4m3_block(bfr[j], af[i & 3]);
                        __builtin_amdgcn_s_setprio(0);
                        const int tp = t >= 2 ? t - 2 : T + t - 2;   // tile of the pending product
                        promote1(tp / SN, tp % SN, ring[t & 1], ring_s[t & 1]);
                        ring[t & 1] = pr;
                        ring_s[t & 1] = s_row;
                    }
                };

                int stage = 0;   // stage holding block it
                for (int it = 0; it < nkb; ++it) {
                    const uint8_t* st = smem + stage * Cfg::STAGE_BYTES;
                    const int next = stage + 1 == Cfg::STAGES ? 0 : stage + 1;
                    const uint8_t* st_next = smem + next * Cfg::STAGE_BYTES;
#pragma unroll
                    for (int i = 0; i + 2 < SM; ++i) {
                        const float s_row = (UE8M0 || !LIVE) ? 0.f : sa[i] * sb;
#pragma unroll
                        for (int j = 0; j < SN; ++j) {
                            step(i, j, s_row);
                            if (LIVE && j == 0) af[(i + 2) & 3] = afrag_at(st, i + 2);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if constexpr (Cfg::EARLY_B) if (i == 0) {
                            // Row 0 has consumed every B fragment and the B scale of
                            // this block (read during the previous block), so every
                            // wave past this barrier is done with the stage's B half.
                            // No LDS drain: the A fragments requested since are
                            // still in flight and unaffected.
                            asm volatile("s_barrier" ::: "memory");
                            if (!a_wave && it + 2 < nkb) issue_stage(it + 2, stage);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    // Block it+1 landed for every wave and every read of block it
                    // done: refill (the A half, with early B refill).
                    if constexpr (Cfg::EARLY_B) {
                        // a B wave may have block it+2's B copies in flight behind
                        if (!a_wave && it + 2 < nkb) wait_vmcnt<Cfg::VM_PER_STAGE>();
                        else wait_vmcnt<0>();
                        lgkm_drain_barrier();
                        if (a_wave && it + 2 < nkb) issue_stage(it + 2, stage);
                    } else {
                        wait_stage_copies<Cfg::STAGES - 2, Cfg::VM_PER_STAGE>(
                            max(0, min(Cfg::STAGES - 2, nkb - 2 - it)));
                        lgkm_drain_barrier();
                        if (it + Cfg::STAGES < nkb) issue_stage(it + Cfg::STAGES, stage);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // (after the last block these reads see a stale stage; unused)
                    if constexpr (LIVE) {
                        if constexpr (UE8M0) load_exps(st_next, kb_lo + it + 1, ea_n, eb_n);
                        else load_scales(st_next, sa_n, sb_n);
                    }
#pragma unroll
                    for (int i = SM - 2; i < SM; ++i) {
                        const float s_row = (UE8M0 || !LIVE) ? 0.f : sa[i] * sb;
#pragma unroll
                        for (int j = 0; j < SN; ++j) {
                            step(i, j, s_row);
                            if (LIVE && j == 0) af[(i + 2) & 3] = afrag_at(st_next, i + 2 - SM);
                            if (LIVE && i == SM - 1) bfr[j] = bfrag_at(st_next, j);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    if constexpr (!LIVE) {
                    } else if constexpr (UE8M0) {
#pragma unroll
                        for (int i = 0; i < SM; ++i) ea[i] = ea_n[i];
#pragma unroll
                        for (int j = 0; j < SN; ++j) eb[j] = eb_n[j];
                    } else {
#pragma unroll
                        for (int i = 0; i < SM; ++i) sa[i] = sa_n[i];
                        sb = sb_n;
                    }
                    stage = next;
                }
                if constexpr (LIVE && !UE8M0) {
                    promote1((T - 2) / SN, (T - 2) % SN, ring[0], ring_s[0]);
                    promote1((T - 1) / SN, (T - 1) % SN, ring[1], ring_s[1]);
                }
            };
            if (wave_live) row_pipeline(std::true_type{});
            else row_pipeline(std::false_type{});
        }
        // every wave is past its last LDS read before the next tile's copies
        lds_barrier();

        // ---- split K: partial sums meet in the workgroup that finishes last ----
        // Each work unit stores its fp32 partial tile (lane-private layout, as
        // device-scope stores, which are written through to the point where
        // all XCDs see them), waits for the stores, then bumps the tile's
        // counter.  The unit that brings the counter to splits-1 adds the
        // partials in split order 0, 1, ... (so the result does not depend on
        // which unit finishes last), resets the counter for the next launch,
        // and runs the epilogue; the others are done with the tile.
        if constexpr (FORM == kDense && Cfg::SPLIT_OK) if (p.splits > 1) {
            constexpr int PER_UNIT = Cfg::THREADS * SM * SN * 4;
            float* mine = p.part + ((int64_t)tile_id * p.splits + split) * PER_UNIT;
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    // component c of MFMA tile (i, j) of thread tid at
                    // ((i SN + j) 4 + c) THREADS + tid: each store instruction
                    // writes 256 contiguous bytes
                    float* q = mine + (i * SN + j) * 4 * Cfg::THREADS + tid;
                    __hip_atomic_store(q + 0 * Cfg::THREADS, acc[i][j].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(q + 1 * Cfg::THREADS, acc[i][j].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(q + 2 * Cfg::THREADS, acc[i][j].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(q + 3 * Cfg::THREADS, acc[i][j].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            // every wave's partial stores have completed before the count
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            __shared__ int last_flag;
            if (tid == 0) {
                const int prior = __hip_atomic_fetch_add(p.counters + tile_id, 1, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                last_flag = prior == p.splits - 1;
            }
            __syncthreads();
            const bool last = last_flag;
            __syncthreads();   // last_flag is rewritten by the next tile
            if (!last) continue;
            // All partials (this unit's too, read back) are added in split
            // order.  Loads go in batches of at most 128 floats per lane, all
            // in flight together: GCH MFMA tiles of BATCH partials at a time.
            const float* all = p.part + (int64_t)tile_id * p.splits * PER_UNIT + tid;
            constexpr int NT = SM * SN;                      // MFMA tiles per lane
            constexpr int GCH = NT < 8 ? NT : 8;
            constexpr int BATCH = 32 / GCH;
            static_assert(NT % GCH == 0, "MFMA tiles split into equal groups");
#pragma unroll
            for (int g0 = 0; g0 < NT; g0 += GCH) {
                f32x4 sum[GCH];
#pragma unroll
                for (int g = 0; g < GCH; ++g) sum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int u0 = 0; u0 < p.splits; u0 += BATCH) {
                    f32x4 buf[BATCH][GCH];
#pragma unroll
                    for (int bi = 0; bi < BATCH; ++bi) {
                        const float* q = all + (int64_t)min(u0 + bi, p.splits - 1) * PER_UNIT;
#pragma unroll
                        for (int g = 0; g < GCH; ++g) {
                            const float* e = q + (g0 + g) * 4 * Cfg::THREADS;
                            buf[bi][g].x = __hip_atomic_load(e + 0 * Cfg::THREADS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            buf[bi][g].y = __hip_atomic_load(e + 1 * Cfg::THREADS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            buf[bi][g].z = __hip_atomic_load(e + 2 * Cfg::THREADS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            buf[bi][g].w = __hip_atomic_load(e + 3 * Cfg::THREADS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
#pragma unroll
                    for (int bi = 0; bi < BATCH; ++bi)
                        if (u0 + bi < p.splits) {
#pragma unroll
                            for (int g = 0; g < GCH; ++g) sum[g] += buf[bi][g];
                        }
                }
#pragma unroll
                for (int g = 0; g < GCH; ++g) acc[(g0 + g) / SN][(g0 + g) % SN] = sum[g];
            }
            if (tid == 0)
                __hip_atomic_store(p.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- epilogue of the grouped 256 x 256 tiles: rounded once, staged in bf16 ----
        // The grouped forms write bf16 with no C, so every accumulator is
        // rounded to bf16 before staging: the whole 128 KB tile fits the idle
        // stages in one phase (the fp32 staging below needs two), and all
        // eight waves stage at once.  Row r of the staged tile holds 32 16-byte
        // chunks (8 columns each), chunk c at position c ^ ((r / SM) & 15); a
        // lane's 8-byte write (4 columns of one row) goes to half
        // ((lane >> 4) & 1) ^ ((r >> 6) & 1) of its chunk, so rows with bit 6
        // set hold their chunks' halves swapped (the reads swap them back).
        // gfx950 serves an 8-byte LDS write in four groups of 16 consecutive
        // lanes, each conflict-free when its lanes hit 16 distinct 8-byte slots
        // modulo 128 bytes (measured with the bank-conflict counter): the 16
        // rows of a group differ in (r / SM) & 7 and in bit 6, which together
        // give the 16 slots.  The row reads take 32 distinct chunks of one row
        // per half-wave, conflict-free under the 16-byte read rule.  Each store
        // instruction then writes two whole rows of D (512 bytes each).  Same
        // bits as the fp32 route, which rounds the same fp32 values once.
        if constexpr (FORM != kDense && BM == 256 && BN == 256) {
            static_assert(!OUT_F32 && Cfg::WAVES == 8 && SM == 8, "grouped forms write bf16 from 8 waves of 128 rows");
            const int lane_e = opaque(tid) & 63;
            const int r16_e = lane_e & 15;
            uint8_t* const stg8 = smem;
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int rl = wm * Cfg::WTM + SM * r16_e + (i ^ (r16_e & 1));
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const int c = (wn * Cfg::WTN + 16 * j) / 8 + (lane_e >> 5);
                    const int pos = c ^ ((rl / SM) & 15);
                    const int hx = ((lane_e >> 4) & 1) ^ ((rl >> 6) & 1);
                    *reinterpret_cast<i32x2*>(stg8 + rl * 512 + 16 * pos + 8 * hx) =
                        pack_bf16x4(acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w);
                }
            }
            lds_barrier();
            // wave w stores tile rows w + 8 j, two per instruction (j = 2 k, 2 k + 1)
#pragma unroll 4
            for (int k = 0; k < BM / 16; ++k) {
                const int half = lane_e >> 5;
                const int rl = wave + 16 * k + 8 * half;
                const int c = lane_e & 31;
                i32x4 v = *reinterpret_cast<const i32x4*>(stg8 + rl * 512 + 16 * (c ^ ((rl / SM) & 15)));
                if ((rl >> 6) & 1) v = i32x4{v.z, v.w, v.x, v.y};   // halves stored swapped
                const int m = r0 + rl;   // row within the group
                const int n = n0 + 8 * c;
                bool ok = m < store_rows && n < p.N;
                if constexpr (FORM == kContiguous) {
                    const int e0 = __builtin_amdgcn_readlane(row_expert, 2 * k);
                    const int e1 = __builtin_amdgcn_readlane(row_expert, 2 * k + 1);
                    if (ok) ok = (half ? e1 : e0) == e;
                }
                if (!ok) continue;
                const int64_t off = (grp_row0 + m) * (int64_t)p.N + n;
                __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(reinterpret_cast<uint16_t*>(p.d) + off));
            }
            // every wave is done reading the staged rows before the next tile's copies
            lds_barrier();
        } else {
            // ---- epilogue: staged through LDS, (+C), convert once, masked store ----------
            // The fp32 tile goes to LDS (the stages are idle now), then every wave
            // writes whole rows: lane q of a row owns its 16-byte fp32 chunk q, so
            // each store instruction covers full contiguous rows of D.  Staging
            // runs in phases of WMP wave rows when the whole tile does not fit.
            // Chunk c of staged row r sits at position c ^ ((r / SM) & 15), which
            // keeps both the writes (a lane's SM rows are SM apart) and the row
            // reads free of LDS bank conflicts.  D is written once and never read
            // here, so the stores are nontemporal (they do not displace operand
            // panels from L2).
            {
                static_assert(FORM != kContiguous, "contiguous tiles take the bf16 staging above");
                // the epilogue's lane offsets derive from a fresh copy of the thread index
                const int lane_e = opaque(tid) & 63;
                const int r16_e = lane_e & 15;
                constexpr int WMP = Cfg::EPI_WAVE_ROWS;          // wave rows per phase
                constexpr int PH_ROWS = WMP * Cfg::WTM;           // tile rows per phase
                constexpr int ROW_CHUNKS = BN / 4;                // 16-byte fp32 chunks per row
                constexpr int RPI = 64 / ROW_CHUNKS;              // rows per wave instruction
                float* const stg = reinterpret_cast<float*>(smem);
#pragma unroll
                for (int ph = 0; ph < Cfg::WAVES_M / WMP; ++ph) {
                    if (wm / WMP == ph) {
#pragma unroll
                        for (int i = 0; i < SM; ++i) {
                            const int rl = (wm % WMP) * Cfg::WTM + SM * r16_e + (i ^ (r16_e & 1));
#pragma unroll
                            for (int j = 0; j < SN; ++j) {
                                const int ch = (wn * Cfg::WTN + 16 * j) / 4 + (lane_e >> 4);
                                *reinterpret_cast<f32x4*>(stg + rl * BN + 4 * (ch ^ ((rl / SM) & 15))) =
                                    acc[i][j];
                            }
                        }
                    }
                    lds_barrier();
                    constexpr int NR = PH_ROWS / (Cfg::WAVES * RPI);   // row steps per wave
#pragma unroll 4
                    for (int k = 0; k < NR; ++k) {
                        const int rl = wave * RPI + k * Cfg::WAVES * RPI + lane_e / ROW_CHUNKS;
                        const int ch = lane_e % ROW_CHUNKS;
                        f32x4 v = *reinterpret_cast<const f32x4*>(stg + rl * BN + 4 * (ch ^ ((rl / SM) & 15)));
                        const int m = r0 + ph * PH_ROWS + rl;   // row within the group
                        const int n = n0 + 4 * ch;
                        const bool ok = m < store_rows && n < p.N;
                        if (!ok) continue;
                        const int64_t off = (grp_row0 + m) * (int64_t)p.N + n;
                        if (OUT_F32) {
                            if (p.c) v += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.c) + off);
                            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.d) + off));
                        } else {
                            if (p.c) {
                                const i32x2 cv = *reinterpret_cast<const i32x2*>(
                                    reinterpret_cast<const uint16_t*>(p.c) + off);
                                v.x += bf16_bits_to_f32((uint32_t)cv.x & 0xFFFFu);
                                v.y += bf16_bits_to_f32((uint32_t)cv.x >> 16);
                                v.z += bf16_bits_to_f32((uint32_t)cv.y & 0xFFFFu);
                                v.w += bf16_bits_to_f32((uint32_t)cv.y >> 16);
                            }
                            __builtin_nontemporal_store(pack_bf16x4(v.x, v.y, v.z, v.w),
                                reinterpret_cast<i32x2*>(reinterpret_cast<uint16_t*>(p.d) + off));
                        }
                    }
                    // every wave is done reading the staged rows before they (or the
                    // next tile's copies) are overwritten
                    lds_barrier();
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------
// Host side: configuration choice and launch
// ------------------------------------------------------------------------------

namespace {

constexpr int kBandMDense = 4;        // M tiles per rasterisation band, dense
constexpr int kBandMContiguous = 8;   // contiguous groups (expert panels are larger)

constexpr int64_t kRefCus = 256;   // MI355X CU count: tile and split choices are functions of the shape
constexpr int kMinSplitBlocks = 8;   // K blocks per split work unit, at least
constexpr int kMaxSplits = 8;

// K split for a dense problem with too few output tiles to give every
// resident workgroup slot of the device work: as many splits as fill the
// slots, each split keeping at least kMinSplitBlocks K blocks.  It is a
// function of the shape alone (slots are counted on the 256-CU part, with
// the configuration's designed workgroups per CU), so results and the
// workspace size do not depend on the device, the CU cap or the caller.
int split_count(int64_t tiles, int KB, int wg_per_cu) {
    const int64_t slots = kRefCus * wg_per_cu;
    if (tiles <= 0 || tiles * 2 > slots || KB < 2 * kMinSplitBlocks) return 1;
    int64_t sp = slots / tiles;
    if (sp > KB / kMinSplitBlocks) sp = KB / kMinSplitBlocks;
    if (sp > kMaxSplits) sp = kMaxSplits;
    return sp < 1 ? 1 : (int)sp;
}

// Split-K workspace of a dense problem: a fixed region of arrival counters
// (one int32 per output tile), then the fp32 partial tiles
// [tiles][splits][BM * BN].  The counter region has the same place and size
// for every shape -- a split problem has at most kMaxSplitTiles tiles -- so
// one workspace serves any sequence of shapes: no shape's partials ever land
// on another shape's counters, and every call leaves all counters zero.
// Zero bytes when K is not split.
constexpr int64_t kMaxSplitTiles = kRefCus;        // tiles * 2 <= kRefCus * WG_PER_CU, WG_PER_CU <= 2
constexpr int64_t kCounterBytes = 4 * kMaxSplitTiles;

struct SplitPlan {
    int64_t tiles = 0;
    int splits = 1;
    int64_t bytes = 0;
};

template <class Cfg>
SplitPlan split_plan(int64_t rows, int64_t N, int64_t K) {
    static_assert(!Cfg::SPLIT_OK || Cfg::WG_PER_CU <= 2, "split tiles fit the counter region");
    SplitPlan sp;
    if (!Cfg::SPLIT_OK) return sp;
    sp.tiles = ((rows + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
    sp.splits = split_count(sp.tiles, (int)(K / kKBlk), Cfg::WG_PER_CU);
    if (sp.splits > 1) {
        if (sp.tiles > kMaxSplitTiles) {   // excluded by split_count; kept as a guard
            sp.splits = 1;
            return sp;
        }
        sp.bytes = kCounterBytes + sp.tiles * sp.splits * Cfg::BM * Cfg::BN * 4;
    }
    return sp;
}

template <class Cfg, int FORM, bool OUT_F32, bool UE8M0>
hipError_t launch_cfg(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    NtArgs a;
    a.a = pr.a; a.sfa = pr.sfa; a.b = pr.b; a.sfb = pr.sfb; a.c = pr.c; a.d = pr.d;
    a.m_indices = pr.m_indices; a.masked_m = pr.masked_m;
    a.rows = (int)pr.rows; a.N = (int)pr.N; a.K = (int)pr.K; a.G = (int)pr.G;
    a.tiles_m = (int)((pr.rows + Cfg::BM - 1) / Cfg::BM);
    a.tiles_n = (int)((pr.N + Cfg::BN - 1) / Cfg::BN);
    // Bands of a few M tiles: the tiles in flight share few A row panels and
    // few B column panels (for contiguous groups: few expert weight panels).
    const int band = FORM == kDense ? kBandMDense : kBandMContiguous;
    a.band_m = (FORM != kMasked && a.tiles_m > band) ? band : a.tiles_m;
    a.xcd_remap = FORM == kDense ? 1 : 0;
    static_assert(FORM != kContiguous || Cfg::BM == 2 * kKBlk, "contiguous tiles span two blocks");
    const int64_t groups = (FORM == kMasked) ? pr.G : (FORM == kContiguous ? 2 : 1);
    const int64_t tiles = groups * a.tiles_m * a.tiles_n;
    if (tiles <= 0) return hipSuccess;

    a.splits = 1;
    a.part = nullptr;
    a.counters = nullptr;
    if (FORM == kDense) {
        const SplitPlan sp = split_plan<Cfg>(pr.rows, pr.N, pr.K);
        if (sp.splits > 1) {
            // the C-ABI layer has checked the caller's workspace against the plan
            if (pr.workspace == nullptr || pr.workspace_bytes < sp.bytes) return hipErrorInvalidValue;
            a.splits = sp.splits;
            a.counters = static_cast<int32_t*>(pr.workspace);
            a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(pr.workspace) + kCounterBytes);
        }
    }
    a.num_tiles = (int)(tiles * a.splits);
    // Decode-size launches (one M tile per group) read each B row once: stream
    // B past the caches.  Measured with the caches flushed before each launch:
    // the ten decode-size dense shapes 288 -> 243 us in total (64 x 7168 x 16384:
    // 60 -> 38 us), masked 32 x 256 x 4096 x 2048: 121 -> 86-91 us.
    a.b_nt = (FORM != kContiguous && a.tiles_m == 1) ? 1 : 0;

    const int64_t resident = (int64_t)cu_cap * Cfg::WG_PER_CU;
    const int grid = (int)(a.num_tiles < resident ? a.num_tiles : resident);
    a.xcd_blk_m = 0;
    a.xcd_units = 0;
    a.xcd_m0 = 0;
    if (FORM == kContiguous && grid % 8 == 0 && a.tiles_n % 2 == 0 &&
        (grid / 8) % (a.tiles_n / 2) == 0) {
        const int blk = (grid / 8) / (a.tiles_n / 2);
        const int rounds = a.tiles_m / (4 * blk);
        a.xcd_blk_m = blk;
        a.xcd_units = rounds * grid;
        a.xcd_m0 = rounds * 4 * blk;
    }
    hipLaunchKernelGGL((nt_fp8_kernel<Cfg, FORM, OUT_F32, UE8M0>), dim3(grid), dim3(Cfg::THREADS), 0,
                       stream, a);
    return hipGetLastError();
}

using Cfg256x256 = NtCfg<256, 256, 2, 4, 2>;
using Cfg128x128 = NtCfg<128, 128, 2, 2, 2>;
using Cfg128x64 = NtCfg<128, 64, 2, 2, 3>;
using Cfg64x64 = NtCfg<64, 64, 1, 4, 3>;
using Cfg64x256 = NtCfg<64, 256, 1, 8, 3>;
using Cfg128x256 = NtCfg<128, 256, 2, 4, 3>;


// Tile choice: 256 x 256 (8 waves of 128 x 64) for large dense problems and
// for contiguous groups (a 256-row tile runs once per distinct expert of its
// two 128-row blocks), 128 x 128 for mid-size rows, and for decode-size rows (HBM-bound:
// every B byte is used once) narrow 64-column tiles with deeper pipelines, so
// more workgroups stream B with more bytes in flight each.
enum NtTile { kT64x64, kT128x64, kT128x128, kT256x256, kT64x256, kT128x256 };

NtTile choose_tile(const NtProblem& pr) {
    if (pr.form == kContiguous) return kT256x256;
    // Decode-size rows with a large B (N * K >= 64 Mi): 256-column tiles, one
    // workgroup of 8 waves per CU, stream B with a quarter of the A re-reads
    // per B byte of 64-column tiles; smaller B keeps the 64-column tiles,
    // whose fixed costs are lower.  The same holds for up to 128 rows.
    if (pr.form == kDense && pr.rows <= 64 && pr.N * pr.K >= (int64_t(64) << 20)) return kT64x256;
    if (pr.form == kDense && pr.rows <= 64) return kT64x64;
    if (pr.form == kDense && pr.rows <= 128 && pr.N * pr.K >= (int64_t(64) << 20)) return kT128x256;
    if (pr.form == kDense && pr.rows <= 128) return kT128x64;
    if (pr.rows <= 64) return kT64x64;
    // Masked groups of more than 128 rows: 256 x 256 tiles, so each A row
    // loaded serves 256 columns (the A rows are re-read once per N tile) and
    // rows past masked_m cost placeholder copies only.
    if (pr.form == kMasked && pr.rows > 128) return kT256x256;
    // 256 x 256 tiles when they give at least half a tile per CU; smaller
    // problems take 128 x 128 tiles (4x as many, split along K if still few).
    if (pr.form == kDense && pr.rows >= 1024 && pr.N >= 1024 &&
        ((pr.rows + 255) / 256) * ((pr.N + 255) / 256) * 2 >= (int64_t)kRefCus)
        return kT256x256;
    return kT128x128;
}

SplitPlan dense_split_plan(int64_t M, int64_t N, int64_t K) {
    NtProblem pr{};
    pr.form = kDense;
    pr.rows = M; pr.N = N; pr.K = K; pr.G = 1;
    switch (choose_tile(pr)) {
    case kT64x64: return split_plan<Cfg64x64>(M, N, K);
    case kT128x64: return split_plan<Cfg128x64>(M, N, K);
    case kT256x256: return split_plan<Cfg256x256>(M, N, K);
    case kT64x256: return split_plan<Cfg64x256>(M, N, K);
    case kT128x256: return split_plan<Cfg128x256>(M, N, K);
    default: return split_plan<Cfg128x128>(M, N, K);
    }
}

template <int FORM, bool OUT_F32, bool UE8M0>
hipError_t dispatch_tiles(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    if constexpr (FORM == kContiguous) {
        return launch_cfg<Cfg256x256, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
    } else {
    switch (choose_tile(pr)) {
    case kT64x64: return launch_cfg<Cfg64x64, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
    case kT128x64:
        if constexpr (FORM == kDense)
            return launch_cfg<Cfg128x64, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
        else
            return hipErrorInvalidValue;   // chosen for dense problems only
    case kT256x256: return launch_cfg<Cfg256x256, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
    case kT128x256:
        if constexpr (FORM == kDense)
            return launch_cfg<Cfg128x256, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
        else
            return hipErrorInvalidValue;
    case kT64x256:
        if constexpr (FORM == kDense)
            return launch_cfg<Cfg64x256, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
        else
            return hipErrorInvalidValue;   // chosen for dense problems only
    default: return launch_cfg<Cfg128x128, FORM, OUT_F32, UE8M0>(pr, cu_cap, stream);
    }
    }
}

template <bool UE8M0>
hipError_t dispatch_forms(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    switch (pr.form) {
    case kDense:
        return pr.out_f32 ? dispatch_tiles<kDense, true, UE8M0>(pr, cu_cap, stream)
                          : dispatch_tiles<kDense, false, UE8M0>(pr, cu_cap, stream);
    case kContiguous:
        return dispatch_tiles<kContiguous, false, UE8M0>(pr, cu_cap, stream);
    case kMasked:
        return dispatch_tiles<kMasked, false, UE8M0>(pr, cu_cap, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int64_t nt_dense_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    return dense_split_plan(M, N, K).bytes;
}

// ------------------------------------------------------------------------------
// Split-K workspace for callers that cannot allocate: one static device array
// per GPU (each device that loads this code object holds its own copy until
// the process ends).  Capacity: the counter region plus the largest partial
// set a split shape can need -- at most kRefCus * 2 work units (the slots of
// the 256-CU part at two workgroups per CU) of at most 128 x 128 fp32.  The
// array starts zero (a zero-initialised device variable), and every call
// leaves its counters zero again.
// ------------------------------------------------------------------------------

namespace {
constexpr int64_t kNoAllocScratchBytes = kCounterBytes + kRefCus * 2 * 128 * 128 * 4;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int64_t nt_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t nt_noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        // the device address of this device's copy of `scratch`; in host code
        // the array's name is only a host-side stand-in, never passed on
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_nt(const NtProblem& pr, int cu_cap, hipStream_t stream) {
    return pr.ue8m0 ? dispatch_forms<true>(pr, cu_cap, stream)
                    : dispatch_forms<false>(pr, cu_cap, stream);
}

const char* nt_config_name(const NtProblem& pr) {
    static const char* tiles[] = {"64x64", "128x64", "128x128", "256x256", "64x256", "128x256"};
    static const char* forms[] = {"dense", "contiguous", "masked"};
    static thread_local char buf[64];
    snprintf(buf, sizeof buf, "nt_%s_%s%s_%s", forms[(int)pr.form],
             pr.out_f32 ? "f32" : "bf16", pr.ue8m0 ? "_ue8m0" : "", tiles[choose_tile(pr)]);
    return buf;
}

const char* describe_nt_config(const NtProblem& pr) {
    static thread_local char buf[192];
    snprintf(buf, sizeof buf, "%s rows=%lld N=%lld K=%lld G=%lld", nt_config_name(pr),
             (long long)pr.rows, (long long)pr.N, (long long)pr.K, (long long)pr.G);
    return buf;
}

}  // namespace dg
