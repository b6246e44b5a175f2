/*
 * dg.h -- C ABI of the MI355X (gfx950) fine-grained FP8 e4m3 GEMM library.
 *
 * The operation of every GEMM entry point is D = C + A @ B^T (NT; the other
 * layouts below transpose the stored operands) on FP8 operands in the OCP
 * E4M3FN encoding, each carrying scale factors at a fine granularity, with
 * the FP8 partial sums of every 128-wide K block scaled and promoted into an
 * fp32 accumulator:
 *
 *   D[m,n] = C[m,n] + sum_kb (sa[kb,m] * sb(n,kb)) * sum_{k in block kb} a[m,k] * b[n,k]
 *
 * Sources (the pages this library is built from):
 *   - "DeepGEMM" README (GitHub, yuguo-Jack fork), section "Interfaces":
 *     subsection "Notices" (the D = C + A @ B naming, NT = row-major A and
 *     B stored [N, K], LHS scale factors in a transposed (MN-major) layout,
 *     fp32 scale factors on the SM90 path, casting and transposition left to
 *     the caller); "Grouped GEMMs (contiguous layout)" (M-axis grouping with
 *     fixed N and K, expert segments aligned to the M block, and the K-axis
 *     grouped TN form for the MoE weight backward pass); "Grouped GEMMs
 *     (masked layout)" (decode under graph capture, the host does not know the
 *     per-expert token counts, only the valid rows are computed).
 *   - News article "Deepseek AI Libera Deepgemm: a GEMM FP8 Library ...",
 *     section "Details and technical benefits" (fine-grained scaling and the
 *     two-level accumulation, i.e. promotion).
 *   - DeepGEMM Documentation (docsearch page), section 10 "Use DeepGEMM
 *     Utility Functions" (SM-count cap and the contiguous-layout alignment
 *     getter, here CU count and 128).
 *   The block sizes (1 x 128 for A, 128 x 128 for B) and the promotion interval
 *   of one 128-wide K block are the workload definitions this library serves;
 *   the pages themselves only say "fine-grained".
 *
 * Conventions for every GEMM entry point:
 *   - All pointers are DEVICE pointers unless the name ends in _host.  The
 *     caller owns every buffer; the library keeps no pointer to them after
 *     it returns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Each call
 *     enqueues one kernel on it and returns; there is no host synchronisation
 *     in the steady state, so calls may be captured into a HIP graph.
 *   - Workspace (the dense NT entry points only): a dense problem with too
 *     few output tiles to occupy the device splits K over several
 *     workgroups, whose fp32 partial tiles meet in a CALLER-OWNED device
 *     buffer passed as `workspace` / `workspace_bytes`.  The size a shape
 *     needs is dg_fp8_gemm_nt_workspace_bytes(M, N, K): a pure function of
 *     the shape (no HIP call, the same on every device), 0 when K is not
 *     split (then workspace may be NULL).  A split shape called with a NULL
 *     or smaller workspace is rejected (DG_ERR_INVALID_ARG), never run a
 *     different way, so a shape always has one summation order.  The first
 *     1 KiB of the buffer holds per-tile arrival counters, at the same place
 *     for every shape: they must be zero when a call starts (zero-fill a new
 *     buffer once) and every call leaves them zero when it completes, so one
 *     buffer serves any sequence of shapes.  The library allocates nothing, frees
 *     nothing, keeps no state between calls and never synchronises;
 *     stream-ordered calls may reuse one buffer, calls that may run
 *     concurrently (other streams, concurrent graph replays) need their
 *     own.  The workspace must not overlap any operand or the output.
 *   - FP8 operands are raw e4m3 bytes (uint8_t).  Scale factors are fp32.
 *   - Outputs: bf16 is stored as uint16_t bit patterns (round to nearest
 *     even, once, from the fp32 accumulator); fp32 as float.
 *   - Host-side validation runs before any HIP call.  On a non-OK status
 *     nothing is launched and no output is touched; dg_last_error() explains
 *     the failure.  A zero-sized problem returns DG_OK without launching.
 *   - Every device pointer (operands, scale factors, metadata, outputs,
 *     workspace) must be 16-byte aligned.
 *   - Device-side metadata cannot be checked without a synchronisation, so it
 *     gets fixed readings instead: masked_m values are clamped to [0, M_max];
 *     m_indices values outside [0, G) mark padding rows.
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs on a given device, whatever the CU cap (fixed summation order;
 *     the only atomics are split-K arrival counters, never sums).
 *   - Split-K ordering: each workgroup writes its fp32 partial tile with
 *     agent-scope atomic stores (on gfx950 these are write-through stores
 *     with the device-coherence bit set, which reach the point every XCD
 *     reads from), waits until they have completed (s_waitcnt vmcnt(0)),
 *     and only then increments the tile's counter with an agent-scope
 *     atomic; the workgroup that takes the last ticket reads the partials
 *     with agent-scope atomic loads (which read at that same point), issued
 *     after its increment has returned.  The order therefore rests on the
 *     ISA's completion order of these device-coherent accesses; no release
 *     fence is used because on this part it would write back the whole L2.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = 1,   /* a shape, pointer, alignment or dtype rule is broken */
    DG_ERR_UNSUPPORTED = 2,   /* current device is not gfx950, or a size limit is hit  */
    DG_ERR_HIP = 3            /* a HIP runtime call or the kernel launch failed        */
} dg_status;

typedef enum {
    DG_BF16 = 1,
    DG_F32 = 2
} dg_dtype;

/*
 * Dense NT GEMM:  D[M,N] = C + A @ B^T.
 *   a    [M, K]            e4m3, row-major (K contiguous)
 *   sfa  [K/128, M]        fp32, one scale per (row, 128-K block), MN-major
 *   b    [N, K]            e4m3, row-major (K contiguous), i.e. B^T column-major
 *   sfb  [ceil(N/128), K/128] fp32, one scale per 128 x 128 block of B
 *   c    NULL (treated as 0), or [M, N] of d_dtype; c == d (in-place
 *        accumulate) is allowed, any other overlap with d is rejected
 *   d    [M, N] of d_dtype (DG_BF16 or DG_F32)
 *   workspace, workspace_bytes
 *        caller-owned split-K buffer of at least
 *        dg_fp8_gemm_nt_workspace_bytes(M, N, K) bytes (counters zero at
 *        the start of the call; see "Workspace" above); NULL / 0 when that
 *        size is 0
 * Rules: K % 128 == 0, N % 16 == 0, M >= 0.
 * Source: "DeepGEMM" README, "Interfaces", "Notices" and "Normal dense GEMMs
 * (non-grouped)" (the caller allocates every buffer and passes it in).
 */
dg_status dg_fp8_gemm_nt(const uint8_t* a, const float* sfa,
                         const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype,
                         int64_t M, int64_t N, int64_t K,
                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * dg_fp8_gemm_nt for callers that cannot allocate device memory or manage a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, rules, results (bit for bit) and
 * errors as dg_fp8_gemm_nt without the workspace pair: a split-K shape uses
 * the library's static device scratch instead, a file-scope array of
 * 32 MiB + 1 KiB per GPU (every dense shape fits it; a larger need would be
 * DG_ERR_UNSUPPORTED), which each GPU the library runs on holds until the
 * process ends.  Nothing is allocated, freed or synchronised; the scratch's
 * device address is looked up once per device (hipGetSymbolAddress) on the
 * first call that needs it.  Every call on a GPU shares that GPU's scratch:
 * calls that may overlap on one GPU (concurrent streams, concurrent graph
 * replays) race and must not be issued.  The scratch's arrival counters
 * start at zero and every call leaves them zero.
 */
dg_status dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa,
                                 const uint8_t* b, const float* sfb,
                                 const void* c, void* d, dg_dtype d_dtype,
                                 int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Workspace bytes a dense NT call (dg_fp8_gemm_nt or dg_fp8_gemm_nt_ue8m0)
 * of this shape needs: 0 when K is not split (and for sizes the entry
 * points would reject).  A function of the shape alone: no HIP call, the
 * same value on every device.  At most 32 MiB + 1 KiB for any shape (at
 * most 512 split work units of at most 128 x 128 fp32, plus the counters).
 */
int64_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * M-grouped contiguous NT GEMM (MoE forward / prefill):
 *   D[r,:] = A[r,:] @ B[e_r]^T  with e_r = m_indices[r].
 *   a         [M_tot, K]   e4m3; segments of rows per expert, concatenated
 *   sfa       [K/128, M_tot] fp32
 *   b         [G, N, K]    e4m3, one [N, K] matrix per expert
 *   sfb       [G, ceil(N/128), K/128] fp32
 *   m_indices [M_tot]      int32: expert of each row, or -1 for padding
 *   d         [M_tot, N]   bf16
 * Rules: M_tot % 128 == 0 (every expert segment is padded to a multiple of
 * dg_get_mk_alignment_for_contiguous_layout() == 128 rows, padding at the
 * segment's tail), K % 128 == 0, N % 16 == 0, G >= 1.
 * The expert of a 128-row block is the index of its first row; a block whose
 * first index is outside [0, G) is skipped.  Rows whose index differs from
 * their block's expert (the padding rows) are not written.
 * Source: "DeepGEMM" README, "Interfaces", "Grouped GEMMs (contiguous layout)".
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* m_indices, void* d,
                                              int64_t M_tot, int64_t N, int64_t K, int64_t G,
                                              void* stream);

/*
 * M-grouped masked NT GEMM (MoE decode, graph-capturable):
 *   D[g,r,:] = A[g,r,:] @ B[g]^T  for r < masked_m[g].
 *   a        [G, M_max, K]   e4m3 (rows >= masked_m[g] may hold anything)
 *   sfa      [G, K/128, M_max] fp32
 *   b        [G, N, K]       e4m3
 *   sfb      [G, ceil(N/128), K/128] fp32
 *   masked_m [G]             int32, device memory, read by the kernel only;
 *                            each value is clamped to [0, M_max]
 *   d        [G, M_max, N]   bf16; rows >= masked_m[g] are never written
 * Rules: K % 128 == 0, N % 16 == 0, G >= 0, M_max >= 0.
 * Source: "DeepGEMM" README, "Interfaces", "Grouped GEMMs (masked layout)".
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa,
                                          const uint8_t* b, const float* sfb,
                                          const int32_t* masked_m, void* d,
                                          int64_t G, int64_t M_max, int64_t N, int64_t K,
                                          void* stream);

/*
 * K-grouped contiguous TN GEMM (MoE weight gradient), fp32 out:
 *   D[g] = C[g] + A_g^T @ B_g, A_g / B_g = the k_sizes_host[g] rows of group g.
 *   a            [K_tot, M]  e4m3, M contiguous (group segments along K)
 *   sfa          [K_tot/128, M] fp32, one scale per (column m, 128-K block)
 *   b            [K_tot, N]  e4m3, N contiguous
 *   sfb          [K_tot/128, N] fp32, one scale per (column n, 128-K block)
 *   k_sizes_host [G]         HOST int32 array, read during the call: each
 *                            >= 0 and a multiple of 128, summing to K_tot
 *   c            NULL (treated as 0) or [G, M, N] fp32; c == d allowed
 *   d            [G, M, N]   fp32; a group with k_sizes_host[g] == 0 gets C[g]
 * Rules: M % 16 == 0, N % 16 == 0, 1 <= G <= 256.
 * Source: "DeepGEMM" README, "Interfaces", "Grouped GEMMs (contiguous
 * layout)" (the K-axis-grouped API for the MoE weight backward pass).
 */
dg_status dg_k_grouped_fp8_gemm_tn_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* k_sizes_host,
                                              const float* c, float* d,
                                              int64_t G, int64_t M, int64_t N, int64_t K_tot,
                                              void* stream);

/*
 * The other memory layouts.  Source: "DeepGEMM" README, "Interfaces",
 * "Notices" (D = C + A @ B named by two layout letters; the newer path takes
 * all four of NT, TN, NN and TT) and "Grouped GEMMs (contiguous layout)" (the
 * nt and nn contiguous variants).  Reading: the first letter is A's, "N" = A
 * stored [M, K] (K contiguous), "T" = A stored [K, M] (the operand is its
 * transpose); the second letter is B's, "T" = B stored [N, K], "N" = B stored
 * [K, N].  In these layouts both operands carry one fp32 scale per output row
 * (m, for A) or column (n, for B) per 128-K block, MN-major:
 *   sfa [K/128, M], sfb [K/128, N]
 * (the per-row granularity of the newer path, and the K-grouped form's
 * layout; a 128 x 128 weight scale is given to each of its rows).
 *   D[m,n] = C[m,n] + sum_kb (sa[kb,m] * sb[kb,n]) * sum_{k in kb} A(m,k) * B(k,n)
 *
 * dg_fp8_gemm_nn:  D = C + A @ B      a [M, K],  b [K, N]
 * dg_fp8_gemm_tn:  D = C + A^T @ B    a [K, M],  b [K, N]
 * dg_fp8_gemm_tt:  D = C + A^T @ B^T  a [K, M],  b [N, K]
 *   c    NULL (0) or [M, N] of d_dtype; c == d allowed, other overlap rejected
 *   d    [M, N], DG_BF16 or DG_F32
 * Rules: K % 128 == 0, N % 16 == 0, and M % 16 == 0 when A is stored [K, M];
 * every pointer 16-byte aligned.  One kernel launch, no workspace; results
 * are deterministic.
 */
dg_status dg_fp8_gemm_nn(const uint8_t* a, const float* sfa,
                         const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);
dg_status dg_fp8_gemm_tn(const uint8_t* a, const float* sfa,
                         const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);
dg_status dg_fp8_gemm_tt(const uint8_t* a, const float* sfa,
                         const uint8_t* b, const float* sfb,
                         const void* c, void* d, dg_dtype d_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * M-grouped contiguous NN GEMM: D[r,:] = A[r,:] @ B[e_r], e_r = m_indices[r].
 *   a         [M_tot, K]     e4m3 (K contiguous); expert segments as in the
 *                            NT contiguous form (128-row aligned, padding at
 *                            each segment's tail)
 *   sfa       [K/128, M_tot] fp32
 *   b         [G, K, N]      e4m3, one [K, N] matrix per expert (N contiguous)
 *   sfb       [G, K/128, N]  fp32, one scale per (column n, 128-K block)
 *   m_indices [M_tot]        int32 expert of each row, -1 for padding
 *   d         [M_tot, N]     bf16; rows whose index differs from their 128-row
 *                            block's expert (padding) are not written
 * Rules: M_tot % 128 == 0, K % 128 == 0, N % 16 == 0, G >= 1; pointers
 * 16-byte aligned.  A block whose first index is outside
 * [0, G) is skipped.
 */
dg_status dg_m_grouped_fp8_gemm_nn_contiguous(const uint8_t* a, const float* sfa,
                                              const uint8_t* b, const float* sfb,
                                              const int32_t* m_indices, void* d,
                                              int64_t M_tot, int64_t N, int64_t K, int64_t G,
                                              void* stream);

/*
 * FP8 casting, the step before the GEMM (the "DeepGEMM" README, "Interfaces",
 * "Notices", leaves casting to the caller and suggests fusing it into the
 * producer; these kernels write exactly the operand layouts the GEMM entry
 * points above take).  For every block of 128 consecutive K columns and
 *   - 1 row  (dg_per_token_cast_to_fp8: activations, the A operand), or
 *   - 128 rows (dg_per_block_cast_to_fp8: weights, the B operand; the last
 *     block of a group covers the rows that exist):
 *   amax  = max |x| over the block
 *   s     = amax / 448 in fp32, correctly rounded; 1 when amax == 0; with
 *           DG_CAST_POW2_SCALE, s is then rounded up to a power of two
 *   code  = the e4m3 (OCP E4M3FN) value nearest to clamp(x / s, -448, 448),
 *           x / s the correctly rounded fp32 quotient, ties to the even
 *           mantissa; negative values that round to zero give 0x80
 * These are the casting rules the GEMM workloads are defined with; the pages
 * give the granularities' names only ("fine-grained").
 *
 * dg_per_token_cast_to_fp8:
 *   x      [G, R, K]  DG_BF16 (uint16_t bit patterns) or DG_F32, row-major;
 *                     values must be finite
 *   codes  [G, R, K]  e4m3 bytes
 *   sf     [G, K/128, R] fp32, MN-major: with G == 1 this is the sfa of
 *                     dg_fp8_gemm_nt / the contiguous form, with G groups of
 *                     R = M_max rows the sfa of the masked form
 * dg_per_block_cast_to_fp8:
 *   w      [G, N, K]  DG_BF16 or DG_F32 (finite)
 *   codes  [G, N, K]  e4m3 bytes
 *   sf     [G, ceil(N/128), K/128] fp32 (the sfb of the GEMM entry points)
 * Rules: K % 128 == 0; G, R / N >= 0; x / w, codes and sf 16-byte aligned;
 * flags is 0 or DG_CAST_POW2_SCALE; outputs must not overlap
 * the input.  One kernel launch on `stream`, no synchronisation, no
 * workspace.  Results are deterministic and bit-exact (no rounding freedom).
 */
#define DG_CAST_POW2_SCALE 1
dg_status dg_per_token_cast_to_fp8(const void* x, dg_dtype x_dtype, uint8_t* codes, float* sf,
                                   int64_t G, int64_t R, int64_t K, int flags, void* stream);
dg_status dg_per_block_cast_to_fp8(const void* w, dg_dtype w_dtype, uint8_t* codes, float* sf,
                                   int64_t G, int64_t N, int64_t K, int flags, void* stream);

/*
 * Power-of-two (UE8M0) scale factors, packed four to a 32-bit integer.
 * Source: "DeepGEMM" README, "Interfaces", "Notices" (the newer path takes
 * its scale factors as UE8M0 values packed four per int instead of fp32),
 * and DeepGEMM Documentation, section 10 (a utility packs fp32 scales into
 * that MN-major layout).  Reading of the layout:
 *   word [k4][mn] (int32, MN-major, row mn fastest) holds in byte i (bits
 *   8i .. 8i+7) the exponent e of the scale 2^(e - 127) of K block 4 k4 + i
 *   of row mn; K4 = ceil(K/512) words per row; bytes past the last K block
 *   are ignored (the packer writes 0).  Both operands carry one scale per
 *   row per 128-K block in this form (a 128 x 128 weight scale is given to
 *   each of its 128 rows).  e = 255 (NaN) is not supported.
 * The GEMM is the definition at the top of this file with those scales:
 *   D[m,n] = C[m,n] + sum_kb 2^(ea(m,kb) - 127) * 2^(eb(n,kb) - 127) * P_kb[m,n]
 * Scaling by a power of two is exact, so the MFMA applies the scales to the
 * FP8 products itself and accumulates every K block into the fp32
 * accumulator; there is no separate promotion step.
 *
 * The three entry points take exactly the arguments, rules, error behaviour
 * and output conventions of their fp32-scale counterparts above, except:
 *   dg_fp8_gemm_nt_ue8m0:                   sfa [K4, M],  sfb [K4, N]
 *   dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0: sfa [K4, M_tot], sfb [G, K4, N]
 *   dg_m_grouped_fp8_gemm_nt_masked_ue8m0:  sfa [G, K4, M_max], sfb [G, K4, N]
 * (int32 words, 16-byte aligned).  The dense form splits K over workgroups
 * like dg_fp8_gemm_nt and takes the same caller-owned workspace (same size
 * query, same rules).
 */
dg_status dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const int32_t* sfa,
                               const uint8_t* b, const int32_t* sfb,
                               const void* c, void* d, dg_dtype d_dtype,
                               int64_t M, int64_t N, int64_t K,
                               void* workspace, int64_t workspace_bytes, void* stream);
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                    const uint8_t* b, const int32_t* sfb,
                                                    const int32_t* m_indices, void* d,
                                                    int64_t M_tot, int64_t N, int64_t K,
                                                    int64_t G, void* stream);
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                const uint8_t* b, const int32_t* sfb,
                                                const int32_t* masked_m, void* d,
                                                int64_t G, int64_t M_max, int64_t N, int64_t K,
                                                void* stream);

/*
 * K-grouped TN form with packed UE8M0 scales.  Reading of the K-grouped
 * packed layout (DeepGEMM Documentation, section 10, lists a packing utility
 * for the K-grouped GEMM): each group's K blocks are packed on their own, so
 * every group starts on a word boundary.  Group g's KB_g = k_sizes_host[g] / 128
 * blocks take ceil(KB_g / 4) word rows, after the previous groups' rows; byte
 * i of word row w_g + k4 holds the exponent of the group's block 4 k4 + i.
 *   sfa [W, M] int32, sfb [W, N] int32, W = sum_g ceil(KB_g / 4)
 * Everything else (layouts, C, rules, errors) is dg_k_grouped_fp8_gemm_tn_contiguous's.
 * The exponents go into the block-scaled MFMA; there is no promotion step.
 */
dg_status dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0(const uint8_t* a, const int32_t* sfa,
                                                    const uint8_t* b, const int32_t* sfb,
                                                    const int32_t* k_sizes_host,
                                                    const float* c, float* d,
                                                    int64_t G, int64_t M, int64_t N, int64_t K_tot,
                                                    void* stream);
/* fp32 power-of-two scales sf [K_tot/128, MN] (MN-major, per column per K
 * block) -> the per-group packed words above, [W, MN] int32.  Byte i of a word
 * is the fp32 exponent field (the UE8M0 code of a positive power of two in
 * [2^-126, 2^127]); unused bytes are 0.  Rules as the K-grouped GEMM's for
 * k_sizes_host; sf and packed 16-byte aligned, not overlapping. */
dg_status dg_pack_ue8m0_scales_k_grouped(const float* sf, const int32_t* k_sizes_host,
                                         int32_t* packed, int64_t G, int64_t MN, int64_t K_tot,
                                         void* stream);

/*
 * fp32 power-of-two scales -> packed UE8M0 words (layout above), G batches:
 *   per_block == 0: sf [G, K/128, MN] fp32, one scale per (row, K block),
 *                   MN-major (the sfa layout, e.g. from dg_per_token_cast_to_fp8
 *                   with DG_CAST_POW2_SCALE)
 *   per_block == 1: sf [G, ceil(MN/128), K/128] fp32, one per 128 x 128 block
 *                   (the sfb layout, e.g. from dg_per_block_cast_to_fp8 with
 *                   DG_CAST_POW2_SCALE), given to each of the block's rows
 *   packed          [G, ceil(K/512), MN] int32
 * Byte i of a word is the 8-bit exponent field of the fp32 scale of K block
 * 4 k4 + i, which is its UE8M0 code when the scale is a positive power of two
 * in [2^-126, 2^127] (the precondition; other values give the exponent field
 * regardless, i.e. the mantissa and sign are dropped).  Bytes past the last
 * K block are 0.
 * Rules: K % 128 == 0; sf and packed 16-byte aligned and not overlapping.
 * One kernel launch on `stream`; errors as for the GEMMs.
 * Source: DeepGEMM Documentation, section 10 (the packed-UE8M0 MN-major
 * layout utility).
 */
dg_status dg_pack_ue8m0_scales(const float* sf, int per_block, int32_t* packed, int64_t G,
                               int64_t MN, int64_t K, void* stream);

/*
 * FP8 MQA logits, non-paged (the indexer kernel).  Source: "DeepGEMM" README,
 * "Interfaces", "V3.2 MQA kernels for the indexer".  For every query i and
 * every kv token j in [ks[i], ke[i]):
 *   kv_j        = kv[j, :] * kv_sf[j]
 *   logits[i,j] = sum_h relu(q[i, h, :] . kv_j) * weights[i, h]
 * and, when clean_logits is 1, logits[i, j] = -inf for every other j (when
 * it is 0 those entries are not written).
 *   q       [S, H, D]  e4m3 (no scale), D = head_dim = 128
 *   kv      [S_kv, D]  e4m3
 *   kv_sf   [S_kv]     fp32, one scale per kv token, > 0
 *   weights [S, H]     fp32
 *   ks, ke  [S]        int32 device arrays; each range is clamped to
 *                      [0, S_kv], and ks >= ke selects nothing
 *   logits  [S, S_kv]  fp32, row-major
 * Rules: D == 128, H in {16, 32, 64}, S <= 1048560, S_kv <= 2^31 - 4097;
 * every pointer 16-byte aligned.  One kernel launch on
 * `stream`, no workspace, deterministic.  The dot product over D runs on the
 * MFMA unit in fp32; the kv scale, being positive, is applied once after the
 * head sum (relu(x * s) = s * relu(x)).
 */
dg_status dg_fp8_mqa_logits(const uint8_t* q, const uint8_t* kv, const float* kv_sf,
                            const float* weights, const int32_t* ks, const int32_t* ke,
                            float* logits, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                            int clean_logits, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* dg_last_error(void);

/*
 * Cap on the compute units the persistent kernels size their grid for
 * (DeepGEMM Documentation, section 10: set/get the maximum SM count).
 * dg_get_num_cus() returns the current cap (the device's CU count by
 * default, 0 if no device is visible); dg_set_num_cus(n) accepts
 * 1 <= n <= device CU count, or 0 to restore the default.
 */
int dg_get_num_cus(void);
dg_status dg_set_num_cus(int n);

/*
 * Name of the kernel instance (tile configuration) a call with these sizes
 * launches, e.g. "nt_dense_bf16_256x256", for profiling and tuning (the
 * configuration report of DeepGEMM Documentation, section 6, variable
 * DG_PRINT_CONFIGS; setting DG_PRINT_CONFIGS=1 also prints it per call).
 *   form: 0 dense, 1 M-grouped contiguous, 2 M-grouped masked (rows = M,
 *   M_tot or M_max), 3 K-grouped TN (rows = M), 4 dense NN, 5 dense TN,
 *   6 dense TT, 7 M-grouped contiguous NN.  out_f32: dense output dtype.
 * Returns a static string; "" for an unknown form.  No HIP call is made.
 */
const char* dg_kernel_config_name(int form, int64_t rows, int64_t N, int64_t K, int out_f32);

/* Row alignment of every expert segment in the contiguous layout: 128
 * (DeepGEMM Documentation, section 9, and section 10's alignment getter). */
int dg_get_mk_alignment_for_contiguous_layout(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
