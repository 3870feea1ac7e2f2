// kev_mfma_core.h -- gfx950 building blocks shared by the prefill and decode kernels.
//
// One wavefront computes, for up to 32 query rows (the B-operand columns),
//     S^T[key][q]  = K[key][:] . Q[q][:]          (v_mfma_f32_32x32x16_bf16)
//     O^T[d][q]   += V^T[d][key] . P^T[key][q]
// with K and V tiles staged in LDS in their natural row-major [key][d] layout.
// These are the decode's and the head_dim-64 prefill's building blocks; the
// head_dim-128 prefill runs three 16-row blocks on v_mfma_f32_16x16x32_bf16
// with its own fragment reads and swizzle (Geom<128, 1>, kev_prefill_bf16.hip).
//
// Staging: global_load_lds_dwordx4 writes 64 lanes x 16 B straight into LDS
// (no VGPR round trip).  A row of D bf16 is D/8 16-byte chunks; chunk c of row
// r is stored at position c ^ swz(r) so that both read patterns below hit
// distinct LDS banks.  Since a direct load writes lane i to base + 16*i, each
// lane fetches the global chunk that belongs at its LDS position.
//
// Reads:
//   K (A operand of S^T): lane l reads 16 B of row l%32 -> one ds_read_b128.
//   V^T (A operand of O^T): ds_read_b64_tr_b16 -- within a 16-lane group,
//   destination lane 4a+b receives element b of the 8-byte rows addressed by
//   lanes a, a+4, a+8, a+12 -- turns four key rows x 16 d into 16 lanes of
//   (one d, four keys); two such reads give the 8 keys of an MFMA k-slice.
//   The key order of those 8 slots matches the rows of the S^T accumulator a
//   lane holds (rows 8*(i/4) + 4*(lane/32) + i%4), so P^T goes from the first
//   MFMA's accumulators to the second MFMA's B operand without leaving the lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kev {
namespace core {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(1))) const void gbl_void;
typedef __attribute__((address_space(3))) void lds_void;

// LDS row layout of a staged tile: row r's 16-byte chunk c sits at chunk c ^ swz(r).  The
// LDS has 64 banks of 4 bytes.  Measured with a probe of the bank-conflict counter on
// gfx950: a 16-byte read serves its lanes in four groups of 16 (lanes with the same bit 5
// and the same parity of bits 2..4), a transposed 8-byte read (ds_read_b64_tr_b16) in two
// groups of 32 (lanes 0..31 and 32..63).  The swizzle keeps every group of the kernel's
// read patterns on distinct banks:
//   SW = 0: 32 consecutive rows at one chunk (K reads of the 32x32 MFMA) and 4 consecutive
//           rows x 4 aligned chunks (its transposed V^T reads);
//   SW = 1 (head_dim 128): rows 0..15 at chunks 4s + g (K reads of the 16x16 MFMA, lane
//           16g + m reading row m) and 8 consecutive rows x 2 aligned chunks (its
//           transposed V^T reads).
template <int D, int SW = 0>
struct Geom {
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;    // rows per 1 KB direct-load instruction
    static constexpr int ROWB = D * 2;      // bytes per row
    static_assert(SW == 0 || D == 128, "the second swizzle is laid out for head_dim 128");
    __device__ static int swz(int r) {
        if (SW == 1) return (((r & 7) << 1) | ((r >> 3) & 1)) ^ (r & 8);
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
    }
    __device__ static int off(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }
};

// s_waitcnt vmcnt(N) only (gfx9 encoding; expcnt / lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that the compiler may not move memory operations across.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 64 lanes x 16 B from global straight into LDS at lds_addr + 16*lane
// (global_load_lds_dwordx4; the LDS address goes through m0), each lane from its own
// 64-bit address.  Issued as inline asm so the compiler does not add its own
// conservative vmcnt waits before LDS reads: the callers wait for these loads
// explicitly (wait_vmcnt + barrier) before reading the stage they fill, and never read
// a stage that has loads in flight.
__device__ __forceinline__ void dma16(const void *g, unsigned lds_addr) {
    const unsigned m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(m0v)
                 : "memory", "m0");
}

// Same load with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset
// (the global address is base + voff), so the per-tile address step is one scalar add.
__device__ __forceinline__ void dma16s(const void *base, unsigned voff, unsigned lds_addr) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    const unsigned m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sb), "s"(m0v)
                 : "memory", "m0");
}

// Per-lane part of a direct load of tile rows [r0, r0 + RPI): the row this lane fills and
// the global chunk that belongs at its LDS position (chunk c ^ swz(r) of the row).
template <int D, int SW = 0>
struct DmaLane {
    int row;     // tile row (key offset inside the tile)
    int coff;    // element offset of the chunk inside the row
    __device__ void init(int r0) {
        using G = Geom<D, SW>;
        const int lane = threadIdx.x & 63;
        row = r0 + lane / G::CPR;
        coff = ((lane % G::CPR) ^ G::swz(row)) * 8;
    }
};

// S^T for the 32 keys [kb*32, kb*32+32) of a staged K tile.
template <int D>
__device__ __forceinline__ f32x16 scores1(const lds_t *ktile, int kb, const bf16x8 *qf) {
    using G = Geom<D>;
    const int lane = threadIdx.x & 63;
    const int row = kb * 32 + (lane & 31), half = lane >> 5;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
        const u32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
            ktile + G::off(row, 2 * dc + half));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[dc], acc, 0, 0, 0);
    }
    return acc;
}

// K fragment (A operand of S^T) for k step dc of a staged 32-key K tile: lane l holds
// row l%32, d = dc*16 + (l/32)*8 .. +8.
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const lds_t *ktile, int dc) {
    using G = Geom<D>;
    const int lane = threadIdx.x & 63;
    const int row = lane & 31, half = lane >> 5;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                                          ktile + G::off(row, 2 * dc + half)));
}

// V^T fragment (A operand) for d-block db and 16-key chunk c of a staged V tile.
template <int D>
__device__ __forceinline__ bf16x8 vt_frag(const lds_t *vtile, int c, int db) {
    using G = Geom<D>;
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, s = lane & 15;
    const int d = db * 32 + (grp & 1) * 16 + 4 * (s & 3);
    const int row = c * 16 + (grp >> 1) * 4 + (s >> 2);
    const int inb = (d & 7) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(vtile + G::off(row, d >> 3) + inb));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(vtile + G::off(row + 8, d >> 3) + inb));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Max / sum over lanes l and l^32 (every lane gets the value for its pair).  ds_bpermute
// through the LDS unit: its wait also waits for every LDS read issued before it.
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32); }

// Max over lanes l and l^32 on the VALU (v_permlane32_swap: with both operands holding x,
// one result holds the low half twice and the other the high half twice), so no LDS
// instruction and no wait on earlier LDS reads is involved.
__device__ __forceinline__ float max_halves_valu(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Online-softmax state of one lane (one query column; the lane pair l, l^32 shares it).
// The running max is only moved (and O^T, l rescaled) when a new score exceeds it by more
// than kLazy (log2 units); otherwise weights are taken against the stale max, so they stay
// below 2^kLazy.  Either way out = O / l is the same softmax average.
constexpr float kLazy = 8.0f;

}  // namespace core
}  // namespace kev
