// Device helpers shared by the prefill GEMM kernels (gemm.hip, gemm256.hip):
// LDS-DMA through buffer resources, explicit wait counts, the LDS swizzle of
// activation tiles, the bf16 32x32x16 MFMA, and compile-time loop helpers.
#pragma once

#include <type_traits>

#include "tf_common.h"

namespace tf {

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

// Row tiles per band of the tile order: with two, the 32 workgroups an XCD runs
// at once cover 2 activation panels x 16 weight column tiles (measured best of
// 1, 2, 4 and all).
constexpr int kBand = 2;
constexpr int kStage = 64; // k rows per pipeline stage

// 16-byte unit (row, c) of a [rows][64] bf16 tile, c = 0..7.  Rows are 128
// bytes, so two share a 256-byte bank line; the XOR with (row / 2) % 8 puts
// the 16 rows that 16 consecutive lanes read at one c into 16 distinct bank
// groups.
__device__ __forceinline__ int swz(int row, int c) { return (row << 3) + (c ^ ((row >> 1) & 7)); }

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; counters not named stay at their maximum (no wait).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier for LDS filled by LDS-DMA: each wave has already waited
// for its own loads; the empty asm statements keep the compiler from moving
// memory operations across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS-DMA: lane i's 16 (or 4) bytes land at lds + 16 i (or 4 i).
// LDS-DMA loads go through buffer instructions (buffer_load_dword[x4] ...
// lds) on a raw buffer resource whose base is wave-uniform: lane L's bytes
// land at lds + size * L.  The buffer form matters: the compiler treats the
// global-segment form as a flat access that may touch LDS and then drains
// every outstanding LDS read before it and after it, which would serialise
// the fragment reads with the MFMAs.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *base)
{
    // stride 0, no range limit below 4 GiB (offsets are built in bounds),
    // dword data format (required for the resource to be valid on gfx9)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void dma16(Rsrc r, uint32_t voff, uint32_t soff, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, (int)voff,
                                             (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(Rsrc r, uint32_t voff, uint32_t soff, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, (int)voff,
                                             (int)soff, 0, 0);
}

// bf16 operands, or fp16 (F16)
template <bool F16 = false> __device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 &a, const u32x4 &b, const f32x16 &c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// How groups map onto the 16-row slices of the k loop.  kGSplit32/64 and
// kGOneTile are the slices per group (G = 32, 64, 128); kGWhole covers groups
// of whole k-tiles (G a multiple of 256, or G == K).
enum GemmGroups { kGWhole = 0, kGSplit32 = 2, kGSplit64 = 4, kGOneTile = 8 };

template <int V> using ic = std::integral_constant<int, V>;

// f(ic<I>{}), ..., f(ic<N - 1>{}): loop indices usable as constants
template <int I, int N, typename F> __device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(ic<I>{});
        static_for<I + 1, N>(f);
    }
}

} // namespace tf
