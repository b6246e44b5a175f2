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
//     of QB queries; wave w owns tokens j0 + 64 w .. + 63 as four 16-token
//     MFMA column fragments, loaded once into registers (lane l: token
//     16 t + (l & 15), bytes 32 (l >> 4) .. + 31 of its D row).
//   * Per query the wave loads the H / 16 head fragments of q[i] (the MFMA
//     row operand, same lane layout) and the weights its lanes need, one
//     query ahead, straight from global memory (the 4 waves of a workgroup
//     read the same q rows, served by the CU's cache).
//   * MFMA result lane l holds heads 16 f + 4 (l >> 4) + c (c = 0..3) of token
//     16 t + (l & 15); the lane folds relu(x) * w over its heads, and two
//     cross-lane xor-adds (lanes 16 and 32 apart) complete the head sum.
//     Lane l then writes token 64 w + l: one coalesced 256-byte store per wave
//     per query.
//   * Waves whose tokens miss a query's range skip its MFMAs; a workgroup
//     whose tokens miss every range of its query block only writes -inf.
#include "dg_internal.h"
#include "tile_common.h"

namespace dg {

namespace {

constexpr int kMqaD = 128;
constexpr int kMqaQB = 16;          // queries per workgroup
constexpr int kMqaTokens = 256;     // kv tokens per workgroup (64 per wave)

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
struct QOps {
    i32x8 q[H / 16];    // head fragments
    f32x4 w[H / 16];    // weights of the lane's 4 heads per fragment
};

template <int H>
__global__ __launch_bounds__(256) void mqa_logits_kernel(MqaArgs p) {
    static_assert(H % 16 == 0 && H <= 64, "heads in fragments of 16");
    constexpr int F = H / 16;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j0 = blockIdx.x * kMqaTokens;
    const int jw = j0 + 64 * wave;                 // first token of this wave
    const int i0 = blockIdx.y * kMqaQB;
    const int i_end = min(i0 + kMqaQB, p.S);
    const int r16 = lane & 15, g = lane >> 4;

    // clamped range of query i
    auto range = [&](int i, int& lo, int& hi) {
        lo = min(max(p.ks[i], 0), p.S_kv);
        hi = min(max(p.ke[i], 0), p.S_kv);
    };
    const int j_out = jw + lane;                   // token this lane writes
    const bool j_ok = j_out < p.S_kv;

    // Does any query of the block reach this workgroup's tokens?
    bool any = false;
    for (int i = i0; i < i_end; ++i) {
        int lo, hi;
        range(i, lo, hi);
        any |= lo < hi && hi > j0 && lo < j0 + kMqaTokens;
    }
    if (!any) {
        if (p.clean && j_ok)
            for (int i = i0; i < i_end; ++i)
                __builtin_nontemporal_store(-__builtin_inff(), p.out + (int64_t)i * p.S_kv + j_out);
        return;
    }

    // kv fragments of the wave's 64 tokens (tokens past S_kv re-read the last)
    i32x8 kvf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int j = min(jw + 16 * t + r16, p.S_kv - 1);
        const i32x4* src = reinterpret_cast<const i32x4*>(p.kv + (int64_t)j * kMqaD + 32 * g);
        const i32x4 lo = src[0], hi = src[1];
        kvf[t] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    const float sf_out = p.sf[min(j_out, p.S_kv - 1)];

    auto load_q = [&](int i, QOps<H>& o) {
        const uint8_t* qi = p.q + (int64_t)i * H * kMqaD;
        const float* wi = p.w + (int64_t)i * H;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const i32x4* src = reinterpret_cast<const i32x4*>(qi + (16 * f + r16) * kMqaD + 32 * g);
            const i32x4 lo = src[0], hi = src[1];
            o.q[f] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            o.w[f] = *reinterpret_cast<const f32x4*>(wi + 16 * f + 4 * g);
        }
    };

    QOps<H> cur, nxt;
    load_q(i0, cur);
    for (int i = i0; i < i_end; ++i) {
        if (i + 1 < i_end) load_q(i + 1, nxt);
        int lo, hi;
        range(i, lo, hi);
        const bool live = lo < hi && hi > jw && lo < jw + 64;   // wave-uniform
        float v = 0.f;
        if (live) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int f = 0; f < F; ++f) {
                    const f32x4 x = mfma_e4m3_block(cur.q[f], kvf[t]);
                    acc[t] = __builtin_fmaf(fmaxf(x.x, 0.f), cur.w[f].x, acc[t]);
                    acc[t] = __builtin_fmaf(fmaxf(x.y, 0.f), cur.w[f].y, acc[t]);
                    acc[t] = __builtin_fmaf(fmaxf(x.z, 0.f), cur.w[f].z, acc[t]);
                    acc[t] = __builtin_fmaf(fmaxf(x.w, 0.f), cur.w[f].w, acc[t]);
                }
            }
            // head sum across the four 16-lane groups
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc[t] += __shfl_xor(acc[t], 16);
                acc[t] += __shfl_xor(acc[t], 32);
            }
            // lane l writes token 16 (l >> 4) + (l & 15) = l of the wave
            const float s = g == 0 ? acc[0] : g == 1 ? acc[1] : g == 2 ? acc[2] : acc[3];
            v = s * sf_out;
        }
        const bool in = j_out >= lo && j_out < hi;   // (in implies j_ok and live)
        if (in)
            __builtin_nontemporal_store(v, p.out + (int64_t)i * p.S_kv + j_out);
        else if (p.clean && j_ok)
            __builtin_nontemporal_store(-__builtin_inff(), p.out + (int64_t)i * p.S_kv + j_out);
        cur = nxt;
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
