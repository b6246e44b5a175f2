// Device helpers shared by the NT and TN kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKBlk = 128;   // K extent of one scale block = one MFMA K step

// LDS tiles hold 128-byte rows (one 128-wide K block of one row of A or B).
// A row is eight 16-byte chunks; chunk c of row r lives at position
// c ^ swz(r).  Eight consecutive rows spread one chunk index over all eight
// positions, and so do rows eight apart (conflict-free fragment reads for
// both the plain and the strided row maps, and conflict-light transposed
// writes in the TN kernel).
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int lds_chunk_off(int row, int chunk) {
    return row * kKBlk + ((chunk ^ swz(row)) << 4);
}

// One e4m3 x e4m3 block product over exactly one 128-wide K block into a
// fresh fp32 accumulator: v_mfma_f32_16x16x128_f8f6f4 with both operands in
// the FP8 E4M3 format (format code 0) and no block scaling (the scale operands
// of 0 select the unscaled instruction).
//
// Operand layout (16 rows x 128 K each): lane l holds row (l & 15) and the 32
// K bytes [32 * (l >> 4), 32 * (l >> 4) + 32).  Both operands use the same
// lane -> K map, so the product pairs matching K indices whatever order the
// unit sums them in.  Result: lane l holds out[4 * (l >> 4) + i][l & 15],
// i = 0..3, where the first operand indexes rows and the second columns.
__device__ __forceinline__ f32x4 mfma_e4m3_block(const i32x8& rows, const i32x8& cols) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rows, cols, zero, 0, 0, 0, 0, 0, 0);
}

// The same block product with power-of-two scales applied inside the MFMA
// and accumulated into `acc`: v_mfma_scale_f32_16x16x128_f8f6f4, where lane l
// passes, in bits 7..0 of e_rows / e_cols, the UE8M0 exponent e (scale
// 2^(e - 127)) of the 32 K values it holds for its row of each operand.  The
// scales are powers of two, so scaling the products is exact and the sum over
// K blocks needs no separate promotion step.
__device__ __forceinline__ f32x4 mfma_e4m3_block_ue8m0(const i32x8& rows, const i32x8& cols,
                                                       const f32x4& acc, int e_rows, int e_cols) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rows, cols, acc, 0, 0, 0, e_rows, 0,
                                                            e_cols);
}

// Fragment whose lane l takes LDS row `row` (callers pass the row of their
// lane) and the 32 K bytes [32 * (l >> 4), +32) of it.
__device__ __forceinline__ i32x8 lds_fragment_row(const uint8_t* tile, int row, int lane) {
    const int c0 = (lane >> 4) * 2;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + lds_chunk_off(row, c0));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + lds_chunk_off(row, c0 + 1));
    i32x8 r;
    r.s0 = lo.x; r.s1 = lo.y; r.s2 = lo.z; r.s3 = lo.w;
    r.s4 = hi.x; r.s5 = hi.y; r.s6 = hi.z; r.s7 = hi.w;
    return r;
}

// Fragment of 16 consecutive LDS rows starting at row0.
__device__ __forceinline__ i32x8 lds_fragment(const uint8_t* tile, int row0, int lane) {
    return lds_fragment_row(tile, row0 + (lane & 15), lane);
}

// Round-to-nearest-even fp32 -> bf16 of four values, packed as two dwords
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ i32x2 pack_bf16x4(float x0, float x1, float x2, float x3) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 lo, hi;
    lo.x = (__bf16)x0; lo.y = (__bf16)x1;
    hi.x = (__bf16)x2; hi.y = (__bf16)x3;
    i32x2 r;
    r.x = __builtin_bit_cast(int, lo);
    r.y = __builtin_bit_cast(int, hi);
    return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// LDS address (byte offset in the workgroup's LDS) of a pointer into a
// __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}

// Direct global -> LDS copies (global_load_lds_dwordx4 / _dword).  Lane l's
// 16 (or 4) bytes at base + voff land at LDS byte lds + 16 * l (or 4 * l), so
// one wave instruction fills 1024 (or 256) consecutive LDS bytes.  `base` and
// `lds` must be wave-uniform; `lds` travels in M0, which the compiler loads
// (the "{m0}" operand).  The hazard recognizer does not look inside inline
// asm, so the asm pads itself: s_nop 4 gives the five wait states the gfx9
// family needs between a VALU write of an SGPR (v_readlane of a spilled
// SGPR, v_readfirstlane) and a VMEM instruction reading it as its address
// base, which also covers the one wait state between a write of M0 and an
// LDS DMA reading it.
// Written as inline asm so the compiler does not treat the in-flight copies
// as aliasing every LDS read (which would drain the vector-memory counter
// before each fragment read); the kernels wait for the copies explicitly
// (vm_drain_barrier).  Extra outstanding loads the compiler does not know
// about only make its own vmcnt waits stricter.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "{m0}"(lds)
                 : "memory");
}

// The same copy with the nontemporal cache policy, for operand rows read
// exactly once by the whole launch (streamed from HBM without displacing
// reused data).
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(base), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(base), "{m0}"(lds)
                 : "memory");
}

// A copy of v that the compiler cannot see through.  Values derived from it
// are computed where the copy is taken: the per-tile prologue and epilogue
// derive their lane-dependent offsets from a fresh copy of the thread index,
// so the compiler does not hoist them out of the tile loop and keep them live
// (spilled) across the K loop, where the accumulators hold the registers.
__device__ __forceinline__ int opaque(int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Wait for this wave's outstanding vector-memory loads (including the LDS
// DMA above), then a workgroup barrier.  The asm memory clobber keeps the
// compiler from moving LDS or global accesses across it.
__device__ __forceinline__ void vm_drain_barrier() {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void vm_lgkm_drain_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most ahead * PER copies of this wave are outstanding
// (ahead in [0, MAXA]); copies retire in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int MAXA, int PER>
__device__ __forceinline__ void wait_stage_copies(int ahead) {
    if constexpr (MAXA >= 6) { if (ahead >= 6) { wait_vmcnt<6 * PER>(); return; } }
    if constexpr (MAXA >= 5) { if (ahead == 5) { wait_vmcnt<5 * PER>(); return; } }
    if constexpr (MAXA >= 4) { if (ahead == 4) { wait_vmcnt<4 * PER>(); return; } }
    if constexpr (MAXA >= 3) { if (ahead == 3) { wait_vmcnt<3 * PER>(); return; } }
    if constexpr (MAXA >= 2) { if (ahead == 2) { wait_vmcnt<2 * PER>(); return; } }
    if constexpr (MAXA >= 1) { if (ahead == 1) { wait_vmcnt<1 * PER>(); return; } }
    wait_vmcnt<0>();
}

__device__ __forceinline__ void lgkm_drain_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace dg
