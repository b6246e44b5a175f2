/*
 * CPU oracle for the fine-grained FP8 (e4m3) GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU library shares no code, header, table or
 * constant with it, and it never calls into the GPU library.
 *
 * What it computes is the plain definition, in fp64:
 *
 *   D = C + A @ B^T   (the NT GEMM of the "DeepGEMM" README, yuguo-Jack fork,
 *                      section "Interfaces", subsection "Notices": A row-major,
 *                      B stored [N, K])
 *
 * on block-scaled e4m3 operands.  The news article "Deepseek AI Libera
 * Deepgemm: a GEMM FP8 Library ..." (section "Details and technical benefits")
 * describes fine-grained scaling plus a two-level accumulation: tensor-core
 * FP8 partial sums are promoted into a higher-precision accumulator.  The scale of a product
 * term depends on its K block, so it cannot be pulled out of the K sum; the
 * definition is therefore
 *
 *   D[m,n] = C[m,n] + sum_kb ( sa[kb,m] * sb[n/128,kb] ) * P_kb[m,n]
 *   P_kb[m,n] = sum_{k = 128 kb .. 128 kb + 127} dec(a[m,k]) * dec(b[n,k])
 *
 * Every e4m3 value is an integer multiple of 2^-9 of magnitude <= 448, so each
 * product is an integer multiple of 2^-18 whose magnitude is below 2^36 such
 * units, and a 128-term sum stays below 2^43 units: inside fp64's 53-bit
 * significand, so P_kb is computed exactly.  The
 * scale product sa*sb of two fp32 values is exact in fp64.  The only roundings
 * are the fp64 products s * P_kb and the running sum over kb (kb ascending).
 *
 * dec() is the OCP FP8 E4M3FN decoding: sign bit 7, exponent bits 6..3 with
 * bias 7, mantissa bits 2..0; exponent 0 is subnormal (m * 2^-9); exponent 15
 * with mantissa 7 is NaN; there is no infinity; the largest finite value is
 * 448 (the workloads quantise with scale = amax / 448).
 *
 * Grouped forms are the dense definition applied per group:
 *   M-grouped contiguous: row r uses expert m_indices[r]; rows whose index is
 *     -1 (or outside [0, G)) have no reference (NaN is written).
 *     ("DeepGEMM" README, "Interfaces", "Grouped GEMMs (contiguous layout)")
 *   M-grouped masked: group g, row r < masked_m[g] gets a reference; rows at or
 *     past masked_m[g] have none (NaN).  masked_m is clamped to [0, M_max].
 *     ("DeepGEMM" README, "Interfaces", "Grouped GEMMs (masked layout)")
 *   K-grouped TN: D[g] = C[g] + sum over group g's K blocks of
 *     (sa[kb,m] * sb[kb,n]) * sum_k dec(a[k,m]) * dec(b[k,n]), with A stored
 *     [K_total, M] and B [K_total, N]; a group with K_g = 0 gives D[g] = C[g].
 *     ("DeepGEMM" README, "Interfaces", "Grouped GEMMs (contiguous layout)",
 *      the K-axis-grouped API for the MoE weight backward pass)
 *
 * C, where present, is passed as fp32 (bf16 and fp32 values are exact in it).
 * Outputs are fp64.  Row selections let a test ask for sampled rows of a
 * large problem; rows are independent, so OpenMP splits them across threads
 * without changing any arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define KBLK 128

/* OCP E4M3FN closed form. */
static double e4m3_value(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

static double g_dec[256];
static int g_dec_ready = 0;

static void build_table(void)
{
    if (g_dec_ready)
        return;
    for (int i = 0; i < 256; ++i)
        g_dec[i] = e4m3_value((uint8_t)i);
    g_dec_ready = 1;
}

void oracle_e4m3_decode(const uint8_t* codes, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_value(codes[i]);
}

/*
 * One output row of the NT definition.
 *   a_row [K] codes; sa_row[kb * sa_stride] is this row's scale for block kb;
 *   b [N, K] codes; sfb [ceil(N/128), K/128]; c_row [N] or NULL.
 */
static void nt_row(const uint8_t* a_row, const float* sa_row, int64_t sa_stride,
                   const uint8_t* b, const float* sfb, const float* c_row,
                   int64_t N, int64_t K, double* out)
{
    const int64_t KB = K / KBLK;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t* b_row = b + n * K;
        double acc = 0.0;
        for (int64_t kb = 0; kb < KB; ++kb) {
            double p = 0.0;                               /* exact block sum */
            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                p += g_dec[a_row[k]] * g_dec[b_row[k]];
            double s = (double)sa_row[kb * sa_stride] * (double)sfb[(n / KBLK) * KB + kb];
            acc += s * p;                                 /* promotion, kb ascending */
        }
        out[n] = acc + (c_row ? (double)c_row[n] : 0.0);
    }
}

/* Dense NT: out[i, :] = D[rows[i], :].  sfa is [K/128, M]. */
int oracle_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   const float* c, int64_t M, int64_t N, int64_t K,
                   const int64_t* rows, int64_t n_rows, double* out)
{
    if (K % KBLK != 0)
        return 1;
    build_table();
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows[i];
        if (m < 0 || m >= M) { bad |= 1; continue; }
        nt_row(a + m * K, sfa + m, M, b, sfb, c ? c + m * N : NULL, N, K, out + i * N);
    }
    return bad;
}

/* M-grouped contiguous: A [M_tot, K], sfa [K/128, M_tot], B [G, N, K],
 * sfb [G, ceil(N/128), K/128], m_indices [M_tot]. */
int oracle_m_grouped_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                const float* sfb, const int32_t* m_indices,
                                int64_t M_tot, int64_t N, int64_t K, int64_t G,
                                const int64_t* rows, int64_t n_rows, double* out)
{
    if (K % KBLK != 0)
        return 1;
    build_table();
    const int64_t NB = (N + KBLK - 1) / KBLK, KB = K / KBLK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = rows[i];
        if (r < 0 || r >= M_tot) { bad |= 1; continue; }
        int64_t e = m_indices[r];
        if (e < 0 || e >= G) {
            for (int64_t n = 0; n < N; ++n)
                out[i * N + n] = NAN;
            continue;
        }
        nt_row(a + r * K, sfa + r, M_tot, b + e * N * K, sfb + e * NB * KB, NULL, N, K,
               out + i * N);
    }
    return bad;
}

/* M-grouped masked: A [G, M_max, K], sfa [G, K/128, M_max], B [G, N, K],
 * sfb [G, ceil(N/128), K/128], masked_m [G].  Selection is (groups[i], rows[i]). */
int oracle_m_grouped_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                            const float* sfb, const int32_t* masked_m,
                            int64_t G, int64_t M_max, int64_t N, int64_t K,
                            const int64_t* groups, const int64_t* rows, int64_t n_sel,
                            double* out)
{
    if (K % KBLK != 0)
        return 1;
    build_table();
    const int64_t NB = (N + KBLK - 1) / KBLK, KB = K / KBLK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t g = groups[i], r = rows[i];
        if (g < 0 || g >= G || r < 0 || r >= M_max) { bad |= 1; continue; }
        int64_t mm = masked_m[g];
        if (mm < 0) mm = 0;
        if (mm > M_max) mm = M_max;
        if (r >= mm) {
            for (int64_t n = 0; n < N; ++n)
                out[i * N + n] = NAN;
            continue;
        }
        nt_row(a + (g * M_max + r) * K, sfa + g * KB * M_max + r, M_max,
               b + g * N * K, sfb + g * NB * KB, NULL, N, K, out + i * N);
    }
    return bad;
}

/* K-grouped TN: A [K_tot, M], sfa [K_tot/128, M], B [K_tot, N], sfb [K_tot/128, N],
 * k_sizes [G] (multiples of 128, summing to K_tot), c [G, M, N] fp32 or NULL.
 * Selection is (groups[i], rows[i] = m); out[i, :] = D[g, m, :]. */
int oracle_k_grouped_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                        const int32_t* k_sizes, const float* c,
                        int64_t G, int64_t M, int64_t N, int64_t K_tot,
                        const int64_t* groups, const int64_t* rows, int64_t n_sel,
                        double* out)
{
    build_table();
    int64_t total = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (k_sizes[g] < 0 || k_sizes[g] % KBLK != 0)
            return 1;
        total += k_sizes[g];
    }
    if (total != K_tot)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t g = groups[i], m = rows[i];
        if (g < 0 || g >= G || m < 0 || m >= M) { bad |= 1; continue; }
        int64_t k0 = 0;
        for (int64_t h = 0; h < g; ++h)
            k0 += k_sizes[h];
        int64_t k1 = k0 + k_sizes[g];
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t kb = k0 / KBLK; kb < k1 / KBLK; ++kb) {
                double p = 0.0;                           /* exact block sum */
                for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                    p += g_dec[a[k * M + m]] * g_dec[b[k * N + n]];
                double s = (double)sfa[kb * M + m] * (double)sfb[kb * N + n];
                acc += s * p;
            }
            out[i * N + n] = acc + (c ? (double)c[(g * M + m) * N + n] : 0.0);
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * FP8 casting: the step before the GEMM.  The "DeepGEMM" README ("Interfaces",
 * "Notices") leaves casting to the caller and suggests fusing it into the
 * producing kernel; the granularities are the ones the GEMM consumes.  The
 * pages give no formula; the reading is the one the workloads are built with:
 *
 *   amax = max |x| over the block (1 x 128 for activations, 128 x 128 for
 *          weights; a weight block at the N tail covers the rows that exist)
 *   s    = amax / 448 in fp32 (correctly rounded); s = 1 when amax == 0;
 *          with pow2, s is then rounded up to a power of two (the UE8M0 scale
 *          format the README's "Notices" names for its newer path)
 *   q    = the e4m3 code nearest to clamp(x / s, -448, 448), the quotient
 *          taken in fp32 (correctly rounded), ties to the code whose mantissa
 *          is even; a negative value that rounds to zero keeps its sign (0x80)
 *
 * x is fp32 (bf16 inputs are exact in it).
 * ------------------------------------------------------------------------- */

/* Nearest e4m3 code to y, ties to even mantissa; |y| >= 448 gives +-448. */
static uint8_t e4m3_encode(double y)
{
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs(y);
    if (a >= 448.0)
        return sign | 0x7E;
    /* codes 0x00 .. 0x7E hold increasing values; find lo with
     * value(lo) <= a < value(lo + 1) */
    int lo = 0, hi = 0x7E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    const double below = a - e4m3_value((uint8_t)lo);
    const double above = e4m3_value((uint8_t)hi) - a;
    int code;
    if (below < above)
        code = lo;
    else if (above < below)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;   /* tie: the even mantissa */
    return sign | (uint8_t)code;
}

void oracle_e4m3_encode(const double* y, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_encode(y[i]);
}

static float cast_scale(float amax, int pow2)
{
    if (amax == 0.0f)
        return 1.0f;
    float s = amax / 448.0f;
    if (pow2) {
        int e;
        const double f = frexp((double)s, &e);   /* s = f * 2^e, 0.5 <= f < 1 */
        if (f != 0.5)
            s = (float)ldexp(1.0, e);
    }
    return s;
}

static uint8_t cast_one(float x, float s)
{
    float q = x / s;
    if (q > 448.0f)
        q = 448.0f;
    if (q < -448.0f)
        q = -448.0f;
    return e4m3_encode((double)q);
}

/* Activations, 1 x 128: x [G, R, K] -> codes [G, R, K], sf [G, K/128, R]. */
int oracle_cast_rows(const float* x, int64_t G, int64_t R, int64_t K, int pow2,
                     uint8_t* codes, float* sf)
{
    if (K % KBLK != 0 || G < 0 || R < 0)
        return 1;
    build_table();
    const int64_t KB = K / KBLK;
#pragma omp parallel for schedule(static)
    for (int64_t gr = 0; gr < G * R; ++gr) {
        const int64_t g = gr / R, r = gr % R;
        const float* xr = x + gr * K;
        for (int64_t kb = 0; kb < KB; ++kb) {
            float amax = 0.0f;
            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                if (fabsf(xr[k]) > amax)
                    amax = fabsf(xr[k]);
            const float s = cast_scale(amax, pow2);
            sf[(g * KB + kb) * R + r] = s;
            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                codes[gr * K + k] = cast_one(xr[k], s);
        }
    }
    return 0;
}

/* Weights, 128 x 128: w [G, N, K] -> codes [G, N, K], sf [G, ceil(N/128), K/128]. */
int oracle_cast_blocks(const float* w, int64_t G, int64_t N, int64_t K, int pow2,
                       uint8_t* codes, float* sf)
{
    if (K % KBLK != 0 || G < 0 || N < 0)
        return 1;
    build_table();
    const int64_t KB = K / KBLK, NB = (N + KBLK - 1) / KBLK;
#pragma omp parallel for schedule(static)
    for (int64_t gb = 0; gb < G * NB * KB; ++gb) {
        const int64_t g = gb / (NB * KB), nb = (gb / KB) % NB, kb = gb % KB;
        const int64_t n1 = (nb + 1) * KBLK < N ? (nb + 1) * KBLK : N;
        const float* wg = w + g * N * K;
        float amax = 0.0f;
        for (int64_t n = nb * KBLK; n < n1; ++n)
            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                if (fabsf(wg[n * K + k]) > amax)
                    amax = fabsf(wg[n * K + k]);
        const float s = cast_scale(amax, pow2);
        sf[gb] = s;
        for (int64_t n = nb * KBLK; n < n1; ++n)
            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                codes[g * N * K + n * K + k] = cast_one(wg[n * K + k], s);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Power-of-two (UE8M0) scales.  The "DeepGEMM" README ("Interfaces",
 * "Notices") gives its newer path scale factors as UE8M0 exponents packed
 * four to a 32-bit integer.  Reading: byte i of word [k4][mn] is the exponent
 * e of the scale 2^(e - 127) of K block 4 k4 + i for row mn (MN-major, K
 * blocks packed little-end first); bytes past the last K block are 0.  Both
 * operands carry per-row scales in this form (a 128 x 128 weight scale is
 * given to each of its 128 rows).  The GEMM is the same definition as above
 * with those scales:
 *   D[m,n] = C[m,n] + sum_kb 2^(ea(m,kb) - 127) * 2^(eb(n,kb) - 127) * P_kb[m,n]
 * ------------------------------------------------------------------------- */

static double ue8m0_scale(const int32_t* packed, int64_t MN, int64_t mn, int64_t kb)
{
    const uint32_t w = (uint32_t)packed[(kb / 4) * MN + mn];
    const int e = (int)((w >> (8 * (kb % 4))) & 0xFF);
    return e == 0xFF ? NAN : ldexp(1.0, e - 127);
}

int oracle_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                         const int32_t* sfb, const float* c, int64_t M, int64_t N, int64_t K,
                         const int64_t* rows, int64_t n_rows, double* out)
{
    if (K % KBLK != 0)
        return 1;
    build_table();
    const int64_t KB = K / KBLK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t m = rows[i];
        if (m < 0 || m >= M) { bad |= 1; continue; }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t kb = 0; kb < KB; ++kb) {
                double p = 0.0;                           /* exact block sum */
                for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                    p += g_dec[a[m * K + k]] * g_dec[b[n * K + k]];
                acc += ue8m0_scale(sfa, M, m, kb) * ue8m0_scale(sfb, N, n, kb) * p;
            }
            out[i * N + n] = acc + (c ? (double)c[m * N + n] : 0.0);
        }
    }
    return bad;
}

/* fp32 power-of-two scales -> packed UE8M0 words [ceil(K/512), MN].
 * layout 0: sf [K/128, MN], one scale per (row, K block) (the A side);
 * layout 1: sf [ceil(MN/128), K/128], one per 128 x 128 block, given to each
 *           of the block's rows (the B side).
 * A scale that is not a power of two in [2^-127, 2^127] is rejected (1). */
int oracle_pack_ue8m0(const float* sf, int layout, int64_t MN, int64_t K, int32_t* packed)
{
    if (K % KBLK != 0 || (layout != 0 && layout != 1))
        return 1;
    const int64_t KB = K / KBLK, K4 = (KB + 3) / 4;
    for (int64_t k4 = 0; k4 < K4; ++k4)
        for (int64_t mn = 0; mn < MN; ++mn) {
            uint32_t w = 0;
            for (int64_t i = 0; i < 4 && 4 * k4 + i < KB; ++i) {
                const int64_t kb = 4 * k4 + i;
                const double s = layout == 0 ? sf[kb * MN + mn] : sf[(mn / KBLK) * KB + kb];
                int x;
                const double f = frexp(s, &x);            /* s = f * 2^x */
                const int e = x - 1 + 127;                /* s = 2^(x-1) when f == 0.5 */
                if (f != 0.5 || e < 0 || e > 254)
                    return 1;
                w |= (uint32_t)e << (8 * i);
            }
            packed[k4 * MN + mn] = (int32_t)w;
        }
    return 0;
}

/* ---------------------------------------------------------------------------
 * The other memory layouts.  The "DeepGEMM" README ("Interfaces", "Notices")
 * names a GEMM D = C + A @ B by two letters for the layouts of A and B, NT
 * being A as stored ([M, K]) times B transposed (B stored [N, K]); its newer
 * path supports all four of NT, TN, NN and TT.  Reading: the first letter is
 * A's, "N" = A stored [M, K] (K contiguous), "T" = A stored [K, M] (the
 * operand is its transpose); the second letter is B's, "T" = B stored [N, K]
 * (the operand is its transpose), "N" = B stored [K, N].  So
 *   NN: D = C + A @ B        A [M, K],  B [K, N]
 *   TN: D = C + A^T @ B      A [K, M],  B [K, N]   (the K-grouped form's layout)
 *   TT: D = C + A^T @ B^T    A [K, M],  B [N, K]
 * For these layouts each operand carries one fp32 scale per row of the output
 * side it belongs to (m for A, n for B) per 128-wide K block, stored
 * MN-major: sfa [K/128, M], sfb [K/128, N] (the per-row scale granularity the
 * newer path uses for both operands, and the K-grouped form's layout).
 * The definition is the one at the top of this file with those scales:
 *   D[m,n] = C[m,n] + sum_kb (sa[kb,m] * sb[kb,n]) * sum_{k in kb} A(m,k) * B(k,n)
 * where A(m,k) is a[m*K + k] (A stored [M, K]) or a[k*M + m] (stored [K, M]),
 * and B(k,n) is b[n*K + k] (stored [N, K]) or b[k*N + n] (stored [K, N]).
 * ------------------------------------------------------------------------- */
int oracle_gemm_layout(const uint8_t* a, int a_stored_mk, const float* sfa, const uint8_t* b,
                       int b_stored_nk, const float* sfb, const float* c, int64_t M, int64_t N,
                       int64_t K, const int64_t* rows, int64_t n_rows, double* out)
{
    if (K % KBLK != 0)
        return 1;
    build_table();
    const int64_t KB = K / KBLK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t m = rows[i];
        if (m < 0 || m >= M) { bad |= 1; continue; }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t kb = 0; kb < KB; ++kb) {
                double p = 0.0;                           /* exact block sum */
                for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k) {
                    const uint8_t av = a_stored_mk ? a[m * K + k] : a[k * M + m];
                    const uint8_t bv = b_stored_nk ? b[n * K + k] : b[k * N + n];
                    p += g_dec[av] * g_dec[bv];
                }
                acc += ((double)sfa[kb * M + m] * (double)sfb[kb * N + n]) * p;
            }
            out[i * N + n] = acc + (c ? (double)c[m * N + n] : 0.0);
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * MQA logits (non-paged), the indexer kernel of the "DeepGEMM" README
 * ("Interfaces", "V3.2 MQA kernels for the indexer").  Inputs: q e4m3
 * [S, H, D]; kv e4m3 [S_kv, D] with one fp32 scale per kv token; weights fp32
 * [S, H]; per query i a kv range [ks[i], ke[i]).  For j in the range:
 *   kv_j      = kv[j, :] * sf[j]                         (decoded, scaled)
 *   out[i, j] = sum_h max(0, q[i, h, :] . kv_j) * weights[i, h]
 * and, with clean set, out[i, j] = -inf outside the range (without it those
 * entries are not defined here: NaN).  The range is clamped to [0, S_kv]; an
 * empty range (ks >= ke) selects nothing.  The dot product over D of decoded
 * e4m3 values is exact in fp64 (as the block sums above); it is multiplied by
 * sf[j], passed through the ReLU, weighted and summed over h in ascending
 * order in fp64.
 * ------------------------------------------------------------------------- */
int oracle_mqa_logits(const uint8_t* q, const uint8_t* kv, const float* sf, const float* w,
                      const int32_t* ks, const int32_t* ke, int64_t S, int64_t S_kv, int64_t H,
                      int64_t D, int clean, const int64_t* rows, int64_t n_rows, double* out)
{
    if (S < 0 || S_kv < 0 || H < 0 || D < 0)
        return 1;
    build_table();
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows[r];
        if (i < 0 || i >= S) { bad |= 1; continue; }
        int64_t lo = ks[i], hi = ke[i];
        lo = lo < 0 ? 0 : (lo > S_kv ? S_kv : lo);
        hi = hi < 0 ? 0 : (hi > S_kv ? S_kv : hi);
        for (int64_t j = 0; j < S_kv; ++j) {
            if (j < lo || j >= hi) {
                out[r * S_kv + j] = clean ? -INFINITY : NAN;
                continue;
            }
            double logit = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double dot = 0.0;                        /* exact */
                for (int64_t d = 0; d < D; ++d)
                    dot += g_dec[q[(i * H + h) * D + d]] * g_dec[kv[j * D + d]];
                const double s = dot * (double)sf[j];
                logit += (s > 0.0 ? s : 0.0) * (double)w[i * H + h];
            }
            out[r * S_kv + j] = logit;
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * K-grouped TN with packed UE8M0 scales.  The documentation's section 10
 * lists a packing utility for the K-grouped GEMM's UE8M0 scales.  Reading:
 * each group's K blocks are packed on their own, so that a group starts on a
 * word boundary: group g's KB_g = k_sizes[g] / 128 blocks take ceil(KB_g / 4)
 * words per column, at word rows w_g = sum_{h < g} ceil(KB_h / 4) ..; byte i
 * of word [w_g + k4][mn] is the exponent e (scale 2^(e - 127)) of the
 * group's K block 4 k4 + i for column mn; unused bytes are 0.
 *   D[g][m,n] = C[g][m,n] + sum over group g's blocks of
 *               2^(ea - 127) * 2^(eb - 127) * sum_k dec(a[k,m]) * dec(b[k,n])
 * ------------------------------------------------------------------------- */
static int k_grouped_word_rows(const int32_t* k_sizes, int64_t G, int64_t g)
{
    int64_t w = 0;
    for (int64_t h = 0; h < g; ++h)
        w += (k_sizes[h] / KBLK + 3) / 4;
    return (int)w;
}

int oracle_k_grouped_tn_ue8m0(const uint8_t* a, const int32_t* sfa, const uint8_t* b,
                              const int32_t* sfb, const int32_t* k_sizes, const float* c,
                              int64_t G, int64_t M, int64_t N, int64_t K_tot,
                              const int64_t* groups, const int64_t* rows, int64_t n_sel,
                              double* out)
{
    build_table();
    int64_t total = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (k_sizes[g] < 0 || k_sizes[g] % KBLK != 0)
            return 1;
        total += k_sizes[g];
    }
    if (total != K_tot)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t g = groups[i], m = rows[i];
        if (g < 0 || g >= G || m < 0 || m >= M) { bad |= 1; continue; }
        int64_t k0 = 0;
        for (int64_t h = 0; h < g; ++h)
            k0 += k_sizes[h];
        const int64_t w0 = k_grouped_word_rows(k_sizes, G, g);
        const int64_t kb0 = k0 / KBLK, nkb = k_sizes[g] / KBLK;
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < nkb; ++j) {             /* the group's block j */
                const int64_t kb = kb0 + j;
                double p = 0.0;                              /* exact block sum */
                for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)
                    p += g_dec[a[k * M + m]] * g_dec[b[k * N + n]];
                acc += ue8m0_scale(sfa + (w0 + j / 4) * M, M, m, j % 4)
                       * ue8m0_scale(sfb + (w0 + j / 4) * N, N, n, j % 4) * p;
            }
            out[i * N + n] = acc + (c ? (double)c[(g * M + m) * N + n] : 0.0);
        }
    }
    return bad;
}

/* fp32 power-of-two scales sf [K_tot/128, MN] -> the per-group packed words
 * above, [sum_g ceil(KB_g / 4), MN].  Non-powers of two are rejected (1). */
int oracle_pack_ue8m0_k_grouped(const float* sf, const int32_t* k_sizes, int64_t G, int64_t MN,
                                int32_t* packed)
{
    int64_t kb0 = 0, w = 0;
    for (int64_t g = 0; g < G; ++g) {
        if (k_sizes[g] < 0 || k_sizes[g] % KBLK != 0)
            return 1;
        const int64_t nkb = k_sizes[g] / KBLK;
        for (int64_t k4 = 0; k4 < (nkb + 3) / 4; ++k4, ++w)
            for (int64_t mn = 0; mn < MN; ++mn) {
                uint32_t word = 0;
                for (int64_t i = 0; i < 4 && 4 * k4 + i < nkb; ++i) {
                    const double s = sf[(kb0 + 4 * k4 + i) * MN + mn];
                    int x;
                    const double f = frexp(s, &x);
                    const int e = x - 1 + 127;
                    if (f != 0.5 || e < 0 || e > 254)
                        return 1;
                    word |= (uint32_t)e << (8 * i);
                }
                packed[w * MN + mn] = (int32_t)word;
            }
        kb0 += nkb;
    }
    return 0;
}
