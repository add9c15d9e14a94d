// Device helpers shared by the fused decode-attention kernels (32-row and
// 16-row waves): vector types, tile geometry and LDS swizzles, the direct
// global->LDS loads, waits, bf16 conversions and lane exchanges.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_attn_internal.h"

namespace gr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int KT = FUSED_KT;    // keys per context tile
constexpr int PSTEPS = 4;       // beam steps gathered into LDS at a time, at most
constexpr int PTAB_BYTES = FUSED_PTAB_BYTES;  // LDS for the BeamPath entries of a workgroup's beams
constexpr float SAFE_SUM = 1.8446744e19f;  // 2^64: largest row sum accepted in pass 0
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr uint32_t BF16_ONES = 0x3f803f80u;  // two bf16 ones

template <int D>
struct Geo {
    static constexpr int ROW = D * 2;                    // bytes per K or V row in LDS
    static constexpr int CH = D / 8;                     // 16-byte chunks per row
    static constexpr int KBYTES = KT * ROW;
    static constexpr int TILE = 2 * KBYTES;              // K tile then V tile
    static constexpr int LOADS = TILE / 1024;            // 1 KB direct loads per tile
    static constexpr int DC = D / 16;                    // 16-wide d chunks (QK contraction)
    static constexpr int DB = D / 32;                    // 32-row d blocks of O^T
    static constexpr int OPITCH = (D + 4) * 4;           // bytes per query row in the merge area
    static constexpr int OSLOT = 32 * OPITCH + 32 * 16;  // one wave's O partial + (max, sums)
};

// XOR swizzles of the 16-byte chunks of a row (row-major K and V tiles, no
// padding): the slot of chunk c of row r is c ^ f(r).  For K the 16 rows a
// ds_read_b128 touches land in 16 different slots; for V the 4 rows x 4
// chunks each half-wave touches in a transposing read are 16 different slots.
template <int D>
__device__ __forceinline__ int kswz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return (4 * (r & 3)) & (D / 8 - 1); }

// LDS of the fused kernel: the tile ring (reused by the beam gathers and
// the merge of the key streams), then the staged BeamPath entries.
template <int D, int NQT, int NKS, int NBUF>
constexpr int lds_main()
{
    constexpr int stage = NKS * NBUF * Geo<D>::TILE;
    constexpr int merge = (NKS - 1) * NQT * Geo<D>::OSLOT;
    static_assert((stage > merge ? stage : merge) == fused_lds_main(D, NQT, NKS, NBUF),
                  "host and device LDS layouts differ");
    return stage > merge ? stage : merge;
}
template <int D, int NQT, int NKS, int NBUF>
constexpr int lds_bytes()
{
    return lds_main<D, NQT, NKS, NBUF>() + PTAB_BYTES;
}

// One 1 KB direct global->LDS load: lane i of the wave writes bytes
// [lds + 16 i, lds + 16 i + 16) from `g`.  Issued through inline assembly so
// that the compiler does not serialise later LDS reads behind it; the kernel
// waits for completion itself (vmcnt, then a workgroup barrier).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}

// Same, with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (no 64-bit address arithmetic per lane).
__device__ __forceinline__ void dma16_s(const void *base, uint32_t off, uint32_t lds)
{
    // base and lds are wave-uniform; make that explicit so they live in SGPRs
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x2 ldg8(const uint16_t *p)
{
    return *reinterpret_cast<const u32x2 *>(p);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l^32.  v_permlane32_swap exchanges lanes 32..63 of its
// first operand with lanes 0..31 of its second; with both operands equal to
// x, lanes 0..31 find their partner's value in the second result and lanes
// 32..63 in the first.  `h` is lane / 32.
__device__ __forceinline__ float swap32(float x, int h)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const uint32_t lo = r[0], hi = r[1];
    return __uint_as_float(h ? lo : hi);
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc)
{
    // vector elements are copied to scalars before the bit casts: a bit cast
    // applied directly to a subscripted vector element reads element 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                              __builtin_bit_cast(bf16x2, y), acc, false);
    }
    return acc;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 8-byte words addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ i16x4 lds_tr16(const char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

}  // namespace gr
