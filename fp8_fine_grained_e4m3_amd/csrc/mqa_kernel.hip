// FP8 MQA logits for gfx950 (the indexer kernel, non-paged).
//
//   out[i, j] = sum_h relu(q[i, h, :] . kv[j, :] * sf[j]) * w[i, h]   for j in [ks[i], ke[i])
//   out[i, j] = -inf elsewhere (when cleaning; otherwise those entries are not written)
//
// ("DeepGEMM" README, yuguo-Jack fork, section "Interfaces", "V3.2 MQA
// kernels for the indexer": e4m3 q [S, H, D], e4m3 kv [S_kv, D] with one fp32
// scale per kv token, fp32 weights [S, H], per-query kv ranges.)
//
// The head dimension D = 128 is exactly one K step of
// v_mfma_f32_16x16x128_f8f6f4: one MFMA gives the dot products of 16 heads
// with 16 kv tokens.  The kv scale is positive, so relu(x * sf) = sf * relu(x)
// and it is applied once per logit after the head sum.
//
// Work decomposition
//   * A workgroup of 4 waves covers 256 kv tokens [j0, j0 + 256) and a block
//     of QB = 16 queries; wave w owns tokens j0 + 64 w .. + 63 as four
//     16-token MFMA column fragments, loaded once into registers (lane l:
//     token 16 t + (l & 15), bytes 32 (l >> 4) .. + 31 of its D row).  (With
//     the query operands in LDS, 64 tokens per wave measured 5% faster than
//     128 and than 8 or 32 queries per workgroup.)
//   * The workgroup copies q[i] (H x 128 bytes) and w[i] into LDS with
//     global -> LDS DMA, three queries ahead (four buffers); each wave reads
//     its H / 16 head fragments (the MFMA row operand, same lane layout) and
//     the weights its lanes need from there.
//   * MFMA result lane l holds heads 16 f + 4 (l >> 4) + c (c = 0..3) of token
//     16 t + (l & 15); the lane folds relu(x) * w over its heads, and two
//     cross-lane xor-adds (lanes 16 and 32 apart) complete the head sum.
//     Lane l then writes tokens 64 k + l of the wave: coalesced 256-byte
//     stores.
//   * Waves whose tokens miss a query's range skip its MFMAs; a workgroup
//     whose tokens miss every range of its query block only writes -inf.
#include "dg_internal.h"
#include "tile_common.h"

namespace dg {

namespace {

constexpr int kMqaD = 128;
constexpr int kMqaQB = 16;          // queries per workgroup
constexpr int kMqaTF = 4;           // 16-token kv fragments per wave
constexpr int kMqaTW = 16 * kMqaTF;  // kv tokens per wave
constexpr int kMqaTokens = 4 * kMqaTW;   // kv tokens per workgroup
constexpr int kMqaNBuf = 4;         // LDS buffers of query operands (3 queries ahead)

// max(x, 0) as one integer max on the bit pattern: a negative float (sign
// bit set) is a negative int32 and becomes +0, a non-negative one is kept.
// (fmaxf would add a NaN-quieting step; MFMA results are never signalling.)
__device__ __forceinline__ float relu(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// K-contiguous row staging (as the MN-major GEMM kernel's): position of
// chunk c of row `row`; sigma swaps bits 0 and 1 and is its own inverse.
__device__ __forceinline__ int k_sigma(int c) { return ((c >> 1) & 1) | ((c & 1) << 1) | (c & 4); }
__device__ __forceinline__ int k_pos(int row, int c) { return k_sigma(c) ^ ((row >> 1) & 7); }

struct MqaArgs {
    const uint8_t* q;
    const uint8_t* kv;
    const float* sf;
    const float* w;
    const int32_t* ks;
    const int32_t* ke;
    float* out;
    int S, S_kv, clean;
};

template <int H>
__global__ __launch_bounds__(256) void mqa_logits_kernel(MqaArgs p) {
    static_assert(H % 16 == 0 && H <= 64, "heads in fragments of 16");
    constexpr int F = H / 16;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j0 = blockIdx.x * kMqaTokens;
    const int jw = j0 + kMqaTW * wave;             // first token of this wave
    const int i0 = blockIdx.y * kMqaQB;
    const int i_end = min(i0 + kMqaQB, p.S);
    const int r16 = lane & 15, g = lane >> 4;

    // The block's ranges, clamped, are loaded once: lane q < kMqaQB holds
    // those of query i0 + q, read back with readlane (no memory access, and
    // so no wait, inside the query loop).
    const int q_lane = min(i0 + (lane & (kMqaQB - 1)), p.S - 1);
    const int lo_v = min(max(p.ks[q_lane], 0), p.S_kv);
    const int hi_v = min(max(p.ke[q_lane], 0), p.S_kv);
    auto range = [&](int i, int& lo, int& hi) {
        lo = __builtin_amdgcn_readlane(lo_v, i - i0);
        hi = __builtin_amdgcn_readlane(hi_v, i - i0);
    };
    // lane l writes tokens jw + 64 k + l (k < kMqaTF / 4)
    constexpr int KO = kMqaTF / 4;

    // Does any query of the block reach this workgroup's tokens?
    bool any = false;
    for (int i = i0; i < i_end; ++i) {
        int lo, hi;
        range(i, lo, hi);
        any |= lo < hi && hi > j0 && lo < j0 + kMqaTokens;
    }
    if (!any) {
        if (p.clean)
            for (int i = i0; i < i_end; ++i)
#pragma unroll
                for (int k = 0; k < KO; ++k)
                    if (jw + 64 * k + lane < p.S_kv)
                        __builtin_nontemporal_store(-__builtin_inff(),
                                                    p.out + (int64_t)i * p.S_kv + jw + 64 * k + lane);
        return;
    }

    // kv fragments of the wave's tokens (tokens past S_kv re-read the last)
    i32x8 kvf[kMqaTF];
#pragma unroll
    for (int t = 0; t < kMqaTF; ++t) {
        const int j = min(jw + 16 * t + r16, p.S_kv - 1);
        const i32x4* src = reinterpret_cast<const i32x4*>(p.kv + (int64_t)j * kMqaD + 32 * g);
        const i32x4 lo = src[0], hi = src[1];
        kvf[t] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    float sf_out[KO];
#pragma unroll
    for (int k = 0; k < KO; ++k) sf_out[k] = p.sf[min(jw + 64 * k + lane, p.S_kv - 1)];

    // q[i] and w[i] go through LDS: NBUF buffers, each holding the H head rows
    // of q[i] (128 bytes each, 16-byte chunk c of row h at position
    // sigma(c) ^ ((h >> 1) & 7), conflict-free for the fragment reads) and the
    // H weights.  Every wave issues the same number of copies per query: QC
    // 1 KiB row copies (duplicated when H < 32) and one copy of the weights
    // (all waves write the same bytes to the same slot).
    constexpr int QC = H >= 32 ? H / 32 : 1;
    constexpr int VMQ = QC + 1;                     // copies per wave per query
    constexpr int QBYTES = H * kMqaD;
    constexpr int BUF = QBYTES + 256;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kMqaNBuf * BUF];
    const uint32_t lds0 = lds_addr(smem);
    uint32_t qoff[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) {
        const int u = (wave * QC + c) % (H / 8);    // 1 KiB copy: rows 8 u .. 8 u + 7
        const int row = 8 * u + (lane >> 3);
        const int chunk = k_sigma((lane & 7) ^ ((row >> 1) & 7));
        qoff[c] = (uint32_t)(row * kMqaD + chunk * 16);
    }
    const uint32_t woff = 4u * (uint32_t)min(lane, H - 1);
    auto issue = [&](int i, int buf) {
        const uint8_t* qi = p.q + (int64_t)i * H * kMqaD;
        const uint32_t dst = lds0 + buf * BUF;
#pragma unroll
        for (int c = 0; c < QC; ++c)
            dma16(qi, qoff[c], dst + (uint32_t)(((wave * QC + c) % (H / 8)) * 1024));
        dma4(p.w + (int64_t)i * H, woff, dst + QBYTES);
    };
    // lane offsets of the two 16-byte chunks of head fragment 0 (row r16)
    const int c0 = 2 * g;
    const int q_lo = r16 * kMqaD + (k_pos(r16, c0) << 4);
    const int q_hi = r16 * kMqaD + (k_pos(r16, c0 + 1) << 4);

    // one query: operands from LDS, MFMAs, relu-weighted head sum, stores
    auto process = [&](int i, const uint8_t* st) {
        int lo, hi;
        range(i, lo, hi);
        const bool live = lo < hi && hi > jw && lo < jw + kMqaTW;   // wave-uniform
        float v[KO];
#pragma unroll
        for (int k = 0; k < KO; ++k) v[k] = 0.f;
        if (live) {
            i32x8 qf[F];
            f32x4 wf[F];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const i32x4 a = *reinterpret_cast<const i32x4*>(st + f * 16 * kMqaD + q_lo);
                const i32x4 b = *reinterpret_cast<const i32x4*>(st + f * 16 * kMqaD + q_hi);
                qf[f] = i32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                wf[f] = *reinterpret_cast<const f32x4*>(st + QBYTES + 4 * (16 * f + 4 * g));
            }
            float acc[kMqaTF];
#pragma unroll
            for (int t = 0; t < kMqaTF; ++t) acc[t] = 0.f;
#pragma unroll
            for (int t = 0; t < kMqaTF; ++t) {
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    const f32x4 x = mfma_e4m3_block(qf[f], kvf[t]);
                    acc[t] = __builtin_fmaf(relu(x.x), wf[f].x, acc[t]);
                    acc[t] = __builtin_fmaf(relu(x.y), wf[f].y, acc[t]);
                    acc[t] = __builtin_fmaf(relu(x.z), wf[f].z, acc[t]);
                    acc[t] = __builtin_fmaf(relu(x.w), wf[f].w, acc[t]);
                }
            }
            // head sum across the four 16-lane groups
#pragma unroll
            for (int t = 0; t < kMqaTF; ++t) {
                acc[t] += __shfl_xor(acc[t], 16);
                acc[t] += __shfl_xor(acc[t], 32);
            }
            // lane l writes token 64 k + 16 (l >> 4) + (l & 15) = 64 k + l of the
            // wave, held by fragment t = 4 k + (l >> 4)
#pragma unroll
            for (int k = 0; k < KO; ++k) {
                const float s = g == 0 ? acc[4 * k] : g == 1 ? acc[4 * k + 1]
                              : g == 2 ? acc[4 * k + 2] : acc[4 * k + 3];
                v[k] = s * sf_out[k];
            }
        }
#pragma unroll
        for (int k = 0; k < KO; ++k) {
            const int j = jw + 64 * k + lane;
            const bool in = j >= lo && j < hi;       // (in implies j < S_kv and live)
            if (in)
                __builtin_nontemporal_store(v[k], p.out + (int64_t)i * p.S_kv + j);
            else if (p.clean && j < p.S_kv)
                __builtin_nontemporal_store(-__builtin_inff(), p.out + (int64_t)i * p.S_kv + j);
        }
    };

    // The kv fragments and scales are complete before any copy is issued
    // (the waits below count copies only).  Queries n + 1 .. n + NBUF - 1 are
    // in flight while query n computes; a wave waits until at most the copies
    // of the queries after n are outstanding (loads and stores retire in
    // order, and any stores issued in between only make the wait stricter),
    // then a barrier makes every wave's copies of query n visible.  The
    // barrier after the query frees its buffer for the copies of query
    // n + NBUF.
    __builtin_amdgcn_s_waitcnt(0);
    const int count = i_end - i0;
#pragma unroll
    for (int n = 0; n < kMqaNBuf - 1; ++n)
        if (n < count) issue(i0 + n, n);
    for (int n = 0; n < count; ++n) {
        if (n + kMqaNBuf - 1 < count) issue(i0 + n + kMqaNBuf - 1, (n + kMqaNBuf - 1) % kMqaNBuf);
        const int ahead = min(kMqaNBuf - 1, count - 1 - n);
        wait_stage_copies<kMqaNBuf - 1, VMQ>(ahead);
        asm volatile("s_barrier" ::: "memory");
        process(i0 + n, smem + (n % kMqaNBuf) * BUF);
        lds_barrier();
    }
}

}  // namespace

hipError_t launch_mqa(const MqaProblem& pr, hipStream_t stream) {
    MqaArgs a;
    a.q = pr.q; a.kv = pr.kv; a.sf = pr.kv_sf; a.w = pr.weights; a.ks = pr.ks; a.ke = pr.ke;
    a.out = pr.logits;
    a.S = (int)pr.S; a.S_kv = (int)pr.S_kv; a.clean = pr.clean ? 1 : 0;
    const dim3 grid((unsigned)((pr.S_kv + kMqaTokens - 1) / kMqaTokens),
                    (unsigned)((pr.S + kMqaQB - 1) / kMqaQB));
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    switch (pr.H) {
    case 16: hipLaunchKernelGGL(mqa_logits_kernel<16>, grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL(mqa_logits_kernel<32>, grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(mqa_logits_kernel<64>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dg
