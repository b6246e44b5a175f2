// FP8 casting on gfx950: bf16 / fp32 -> e4m3 codes + fp32 block scales.
//
// The step before the GEMM.  The "DeepGEMM" README ("Interfaces", "Notices")
// leaves casting to the caller and suggests fusing it into the producing
// kernel; these kernels produce exactly the operand layouts the GEMM entry
// points consume:
//   per token (1 x 128): x [G, R, K] -> codes [G, R, K], sf [G, K/128, R]
//                        (MN-major, the A-side scale layout);
//   per block (128 x 128): w [G, N, K] -> codes [G, N, K],
//                        sf [G, ceil(N/128), K/128] (the B-side layout).
// Per block of 128 K columns (and 1 or 128 rows):
//   s = amax / 448 (fp32, correctly rounded; 1 when amax == 0; optionally
//       rounded up to a power of two, the UE8M0 scale format),
//   code = e4m3 nearest to clamp(x / s, -448, 448), ties to even mantissa,
// with x / s the correctly rounded fp32 quotient.
//
// Work split: a workgroup (4 waves) covers one 128-column block of 64 rows
// (per token) or 128 rows (per block).  Each lane loads 16 bytes per row it
// touches (8 bf16 or 4 fp32), so a row's 128 columns are 16 or 32 lanes and
// one load instruction covers 4 or 2 whole rows: every global access is a
// full 128-byte line or more.  The amax of a row is a reduction over its
// lanes (per token); the block amax goes through LDS across the 4 waves.
//
// The division: one correctly rounded reciprocal y = 1/s per row, then per
// element q = x*y followed by two exact-remainder corrections
// q += fma(-q, s, x) * y.  With y correctly rounded the first correction
// leaves q within one ulp of x/s, and a correction of a quotient within one
// ulp, with a correctly rounded reciprocal, is the correctly rounded quotient
// (Markstein's theorem on division by reciprocal refinement; the remainder
// x - q*s is exact in fp32 for such q).  The result is bit-identical to x / s
// at 5 VALU operations instead of a full division sequence per element.  A
// subnormal s (whose reciprocal overflows) takes the plain division.  The
// final copysign keeps the sign of zero quotients (the corrections turn -0
// into +0).
//
// The e4m3 conversion is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to
// nearest even) on values already clamped to +-448.
#include "dg_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {
namespace {

constexpr int kBlk = 128;
constexpr float kE4m3Max = 448.0f;
constexpr float kMinNormal = 1.17549435e-38f;

template <typename In>
struct Lanes;
template <>
struct Lanes<uint16_t> {   // bf16 bit patterns
    static constexpr int EPL = 8;   // elements per 16-byte load
    __device__ static float at(const uint4& v, int i) {
        const uint32_t word = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
        return __uint_as_float((i & 1) ? (word & 0xFFFF0000u) : (word << 16));
    }
};
template <>
struct Lanes<float> {
    static constexpr int EPL = 4;
    __device__ static float at(const uint4& v, int i) {
        return __uint_as_float(i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w);
    }
};

__device__ __forceinline__ float block_scale(float amax, bool pow2) {
    if (amax == 0.0f) return 1.0f;
    float s = amax / kE4m3Max;
    if (pow2) {
        int e;
        const float f = frexpf(s, &e);   // s = f * 2^e, 0.5 <= f < 1
        if (f != 0.5f) s = ldexpf(1.0f, e);
    }
    return s;
}

// x / s, correctly rounded, given y = 1/s correctly rounded and s normal.
__device__ __forceinline__ float quotient(float x, float s, float y) {
#pragma clang fp contract(off)
    float q = x * y;
    float r = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(r, y, q);
    r = __builtin_fmaf(-q, s, x);
    q = __builtin_fmaf(r, y, q);
    return __builtin_copysignf(q, x);
}

__device__ __forceinline__ float clamp448(float q) {
    return __builtin_fminf(__builtin_fmaxf(q, -kE4m3Max), kE4m3Max);
}

// Four clamped quotients -> four e4m3 bytes (byte i = value i).
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

template <typename In, int WAVE_ROWS, bool BLOCK_SCALE>
__global__ __launch_bounds__(256) void cast_kernel(const In* __restrict__ x,
                                                   uint8_t* __restrict__ codes,
                                                   float* __restrict__ sf, int R, int K,
                                                   int row_tiles, int pow2) {
    using L = Lanes<In>;
    constexpr int EPL = L::EPL;
    constexpr int LPR = kBlk / EPL;          // lanes per row: 16 (bf16) or 32 (fp32)
    constexpr int RPI = 64 / LPR;            // rows per load instruction
    constexpr int NI = WAVE_ROWS / RPI;      // loads per lane
    constexpr int WG_ROWS = 4 * WAVE_ROWS;
    static_assert(WAVE_ROWS % RPI == 0, "whole load instructions per wave");
    static_assert(!BLOCK_SCALE || WG_ROWS == kBlk, "a weight block is 128 rows");

    const int KB = K / kBlk;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int t = blockIdx.x;                      // (g, row tile, kb), kb fastest
    const int kb = t % KB;
    t /= KB;
    const int rt = t % row_tiles;
    const int g = t / row_tiles;
    const int64_t gbase = (int64_t)g * R * K;
    const int col = kb * kBlk + (lane % LPR) * EPL;
    const int row0 = rt * WG_ROWS + wave * WAVE_ROWS + lane / LPR;

    // The input is read once: nontemporal loads (10-13% faster on operands of
    // 350 MB and more than plain loads).  Codes and scales use plain stores,
    // so the GEMM that reads them next can find them in cache.
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    uint4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = row0 + i * RPI;
        v[i] = make_uint4(0, 0, 0, 0);
        if (row < R) {
            const u32x4 t = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(x + gbase + (int64_t)row * K + col));
            v[i] = make_uint4(t.x, t.y, t.z, t.w);
        }
    }

    float m[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(L::at(v[i], e)));
        m[i] = a;
    }
    if constexpr (!BLOCK_SCALE) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int o = LPR / 2; o >= 1; o >>= 1) m[i] = __builtin_fmaxf(m[i], __shfl_xor(m[i], o));
    } else {
        __shared__ float part[4];
        float w = m[0];
#pragma unroll
        for (int i = 1; i < NI; ++i) w = __builtin_fmaxf(w, m[i]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) w = __builtin_fmaxf(w, __shfl_xor(w, o));
        if (lane == 0) part[wave] = w;
        __syncthreads();
        w = __builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3]));
#pragma unroll
        for (int i = 0; i < NI; ++i) m[i] = w;
    }

#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = row0 + i * RPI;
        const float s = block_scale(m[i], pow2 != 0);
        const bool fast = s >= kMinNormal;
        const float y = 1.0f / s;
        float q[EPL];
        if (fast) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) q[e] = clamp448(quotient(L::at(v[i], e), s, y));
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) q[e] = clamp448(L::at(v[i], e) / s);
        }
        if (row < R) {
            uint8_t* dst = codes + gbase + (int64_t)row * K + col;
            if constexpr (EPL == 8)
                *reinterpret_cast<uint2*>(dst) =
                    make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
            else
                *reinterpret_cast<uint32_t*>(dst) = pack4(q[0], q[1], q[2], q[3]);
            if constexpr (!BLOCK_SCALE) {
                if (lane % LPR == 0) sf[((int64_t)g * KB + kb) * R + row] = s;
            }
        }
    }
    if constexpr (BLOCK_SCALE) {
        if (threadIdx.x == 0) sf[((int64_t)g * row_tiles + rt) * KB + kb] = block_scale(m[0], pow2 != 0);
    }
}

template <typename In, int WAVE_ROWS, bool BLOCK_SCALE>
hipError_t launch_cast(const CastProblem& p, hipStream_t stream) {
    constexpr int WG_ROWS = 4 * WAVE_ROWS;
    const int row_tiles = (int)((p.R + WG_ROWS - 1) / WG_ROWS);
    const int64_t grid = p.G * row_tiles * (p.K / kBlk);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((cast_kernel<In, WAVE_ROWS, BLOCK_SCALE>), dim3((unsigned)grid), dim3(256),
                       0, stream, static_cast<const In*>(p.x), p.codes, p.sf, (int)p.R, (int)p.K,
                       row_tiles, p.pow2 ? 1 : 0);
    return hipGetLastError();
}

// Packed UE8M0 scale words: thread t writes word t of packed [G, K4, MN]
// (row mn fastest, so reads of MN-major scales and the writes are coalesced).
// Byte i of word k4 is the 8-bit exponent field of the fp32 scale of K block
// 4 k4 + i, which for a power of two 2^x (x >= -126) is x + 127, the UE8M0
// code of that scale; bytes past the last K block are 0.
__global__ __launch_bounds__(256) void pack_ue8m0_kernel(const float* __restrict__ sf,
                                                         int per_block, int64_t total, int MN,
                                                         int KB, int K4,
                                                         int32_t* __restrict__ packed) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int mn = (int)(t % MN);
    const int64_t rest = t / MN;
    const int k4 = (int)(rest % K4);
    const int64_t g = rest / K4;
    const int row_blocks = (MN + kBlk - 1) / kBlk;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kb = 4 * k4 + i;
        if (kb >= KB) break;
        const float s = per_block ? sf[(g * row_blocks + mn / kBlk) * KB + kb]
                                  : sf[(g * KB + kb) * MN + mn];
        w |= ((__float_as_uint(s) >> 23) & 0xFFu) << (8 * i);
    }
    packed[t] = (int32_t)w;
}

// K-grouped packing: block (x, w) covers columns 256 x .. of word row w; the
// row's group is found by a (uniform) scan of the groups' first word rows.
struct KGroupedPackArgs {
    const float* sf;
    int32_t* packed;
    int MN, G;
    int32_t w_start[kMaxTnGroups + 1];   // first word row of group g (and the total)
    int32_t kb_start[kMaxTnGroups];      // first K block of group g
    int32_t kb_count[kMaxTnGroups];
};

__global__ __launch_bounds__(256) void pack_ue8m0_k_grouped_kernel(KGroupedPackArgs a) {
    const int w = blockIdx.y;
    const int mn = blockIdx.x * 256 + threadIdx.x;
    if (mn >= a.MN) return;
    int g = 0;
    while (g + 1 < a.G && a.w_start[g + 1] <= w) ++g;
    const int k4 = w - a.w_start[g];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * k4 + i;
        if (j >= a.kb_count[g]) break;
        const float s = a.sf[(int64_t)(a.kb_start[g] + j) * a.MN + mn];
        word |= ((__float_as_uint(s) >> 23) & 0xFFu) << (8 * i);
    }
    a.packed[(int64_t)w * a.MN + mn] = (int32_t)word;
}

}  // namespace

hipError_t launch_pack_ue8m0_k_grouped(const float* sf, const int32_t* k_sizes_host, int64_t G,
                                       int64_t MN, int32_t* packed, hipStream_t stream) {
    KGroupedPackArgs a;
    a.sf = sf; a.packed = packed; a.MN = (int)MN; a.G = (int)G;
    int32_t w = 0, kb = 0;
    for (int g = 0; g < G; ++g) {
        a.w_start[g] = w;
        a.kb_start[g] = kb;
        a.kb_count[g] = k_sizes_host[g] / kBlk;
        kb += a.kb_count[g];
        w += (a.kb_count[g] + 3) / 4;
    }
    a.w_start[G] = w;
    if (w == 0 || MN == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_ue8m0_k_grouped_kernel, dim3((unsigned)((MN + 255) / 256), (unsigned)w),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_pack_ue8m0(const PackProblem& p, hipStream_t stream) {
    const int K4 = (int)((p.KB + 3) / 4);
    const int64_t total = p.G * K4 * p.MN;
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(pack_ue8m0_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p.sf,
                       p.per_block ? 1 : 0, total, (int)p.MN, (int)p.KB, K4, p.packed);
    return hipGetLastError();
}

int64_t cast_grid(const CastProblem& p) {
    const int64_t wg_rows = p.block_scale ? 128 : 64;
    return p.G * ((p.R + wg_rows - 1) / wg_rows) * (p.K / kBlk);
}

hipError_t launch_cast(const CastProblem& p, hipStream_t stream) {
    if (p.block_scale)
        return p.in_f32 ? launch_cast<float, 32, true>(p, stream)
                        : launch_cast<uint16_t, 32, true>(p, stream);
    return p.in_f32 ? launch_cast<float, 16, false>(p, stream)
                    : launch_cast<uint16_t, 16, false>(p, stream);
}

}  // namespace dg
