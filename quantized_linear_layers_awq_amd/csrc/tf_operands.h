// MFMA operand builders of the fused kernels: how each kernel turns packed
// codes into bf16 (or, with F16, fp16) B operands (TileFuse summary,
// Methodology section 1: unpack and dequantize inside the kernel, never
// writing full-precision weights).
// They live here, not in the kernels' sources, so that the dequantization
// test hooks (repack.hip) decode a packed buffer with the very functions the
// kernels run.
#pragma once

#include "tf_common.h"

namespace tf {

// ---- GEMM: the exact bf16 values (q - z) that a weight tile holds in LDS ----

// q * s + c for eight W8 codes held in two words (row i in byte i); with
// c = -z * s this is (q - z) * s exactly.
__device__ __forceinline__ void dequant_w8_pair(uint32_t w0, uint32_t w1, float s, float c, float out[8])
{
    out[0] = fmaf((float)(w0 & 0xFFu), s, c);
    out[1] = fmaf((float)((w0 >> 8) & 0xFFu), s, c);
    out[2] = fmaf((float)((w0 >> 16) & 0xFFu), s, c);
    out[3] = fmaf((float)(w0 >> 24), s, c);
    out[4] = fmaf((float)(w1 & 0xFFu), s, c);
    out[5] = fmaf((float)((w1 >> 8) & 0xFFu), s, c);
    out[6] = fmaf((float)((w1 >> 16) & 0xFFu), s, c);
    out[7] = fmaf((float)(w1 >> 24), s, c);
}

// Exact bf16 (or fp16) (q - z) * live of eight W4 codes (rows 0..7 of a
// column's k-octet in one word).  `lo` / `hi` hold the even / odd nibbles as
// bytes; the empty asm keeps the compiler from merging the masks into
// per-value bit-field extracts, so each value is one v_cvt_f32_ubyteN and one
// fma.
template <bool F16 = false> __device__ __forceinline__ u32x4 unpack_w4(uint32_t w, float live, float nz)
{
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    asm volatile("" : "+v"(lo), "+v"(hi));
    // nibble 2j holds row j/2... see w4_row_shift: rows 0,4,1,5 in lo, 2,6,3,7 in hi
    const float r0 = fmaf((float)(lo & 0xFFu), live, nz), r4 = fmaf((float)((lo >> 8) & 0xFFu), live, nz);
    const float r1 = fmaf((float)((lo >> 16) & 0xFFu), live, nz), r5 = fmaf((float)(lo >> 24), live, nz);
    const float r2 = fmaf((float)(hi & 0xFFu), live, nz), r6 = fmaf((float)((hi >> 8) & 0xFFu), live, nz);
    const float r3 = fmaf((float)((hi >> 16) & 0xFFu), live, nz), r7 = fmaf((float)(hi >> 24), live, nz);
    return u32x4{pack_int_x2<F16>(r0, r1), pack_int_x2<F16>(r2, r3), pack_int_x2<F16>(r4, r5),
                 pack_int_x2<F16>(r6, r7)};
}

// Same for eight W8 codes held in two words (row i in byte i).
template <bool F16 = false> __device__ __forceinline__ u32x4 unpack_w8(uint32_t w0, uint32_t w1, float live, float nz)
{
    float f[8];
    dequant_w8_pair(w0, w1, live, nz, f);
    return u32x4{pack_int_x2<F16>(f[0], f[1]), pack_int_x2<F16>(f[2], f[3]), pack_int_x2<F16>(f[4], f[5]),
                 pack_int_x2<F16>(f[6], f[7])};
}

// ---- GEMV: bf16 128 + q (W4) or q (W8), with the zero point as a second
//      operand of the same form; the scale is applied to the difference of
//      the two MFMA sums ----

// Eight W4 codes (one column, rows 0..7 of an octet) -> B operand of the
// values 128 + q, exactly: OR-ing a nibble into the mantissa of 128.0.  In
// bf16 (0x4300) the unit step of that binade is mantissa bit 0; in fp16
// (0x5800) it is bit 3, so each nibble pair is shifted 3 bits further left.
// `magic` is 128.0 in both halves held in a vector register, so each pair
// costs one v_and_or_b32 (the mask comes from a scalar register) after its
// shift.
template <bool F16 = false> __device__ __forceinline__ u32x4 w4_operand(uint32_t w, uint32_t magic)
{
    u32x4 b;
    if constexpr (F16) {
        b[0] = ((w << 3) & 0x00780078u) | magic;
        b[1] = ((w >> 1) & 0x00780078u) | magic;
        b[2] = ((w >> 5) & 0x00780078u) | magic;
        b[3] = ((w >> 9) & 0x00780078u) | magic;
    } else {
        b[0] = (w & 0x000F000Fu) | magic;
        b[1] = ((w >> 4) & 0x000F000Fu) | magic;
        b[2] = ((w >> 8) & 0x000F000Fu) | magic;
        b[3] = ((w >> 12) & 0x000F000Fu) | magic;
    }
    return b;
}

template <bool F16 = false> __device__ __forceinline__ uint32_t magic_in_vgpr()
{
    uint32_t m;
    if constexpr (F16)
        asm volatile("v_mov_b32 %0, 0x58005800" : "=v"(m));
    else
        asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(m));
    return m;
}

// Eight W8 codes (bytes of w0, w1) -> B operand of the values q (exact).
template <bool F16 = false> __device__ __forceinline__ u32x4 w8_operand(uint32_t w0, uint32_t w1)
{
    u32x4 b;
    b[0] = pack_int_x2<F16>((float)(w0 & 0xFFu), (float)((w0 >> 8) & 0xFFu));
    b[1] = pack_int_x2<F16>((float)((w0 >> 16) & 0xFFu), (float)(w0 >> 24));
    b[2] = pack_int_x2<F16>((float)(w1 & 0xFFu), (float)((w1 >> 8) & 0xFFu));
    b[3] = pack_int_x2<F16>((float)((w1 >> 16) & 0xFFu), (float)(w1 >> 24));
    return b;
}

// B operand whose eight rows all hold the zero point, in the same form as the
// code operand: 128 + z for W4, z for W8.
template <int BITS, bool F16 = false> __device__ __forceinline__ u32x4 zero_operand(uint32_t z)
{
    uint32_t v;
    if constexpr (BITS == 4) {
        const uint32_t h = F16 ? (0x5800u | (z << 3)) : (0x4300u | z);
        v = h | (h << 16);
    } else {
        v = pack_int_x2<F16>((float)z, (float)z);
    }
    return u32x4{v, v, v, v};
}

} // namespace tf
