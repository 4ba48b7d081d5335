// Shared device/host definitions of the fused W4A16 / W8A16 linear layer:
// vector types, the packed (pre-tiled) layout geometry, helpers for the two
// 16-bit formats of activations, scales and outputs (bf16, and the IEEE fp16
// of many AWQ checkpoints; F16 selects it).
//
// The packed layout implements the interleaved pre-tiling of the TileFuse
// summary (Methodology section 2): scales and zero points packed next to the
// codes they dequantize, and everything one consumer streams kept contiguous.
// On MI355X the consumer of a 16-column block is one workgroup; one 16-byte
// load per lane of a wavefront fetches, for four consecutive 32-row k-steps,
// eight rows of one column -- four 16x16x32 bf16 MFMA B operands after
// unpacking.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tf {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFormatVersion = 2;

// Epilogue and 16-bit format of a linear launch (a template argument of the
// kernels): a plain store with x, scales and y in bf16; silu(gate) * up over
// a [gate | up] layer (bf16); or a plain store with x, scales and y in IEEE
// fp16.
constexpr int kActNone = 0, kActSiluMul = 1, kActF16 = 2;
constexpr int kBlockCols = 16;  // output columns per packed block (one MFMA column tile)
constexpr int kTileRows = 128;  // rows per k-tile of codes
constexpr int kStepRows = 32;   // rows per MFMA (k depth of 16x16x32)

__host__ __device__ constexpr int tile_bytes(int bits) { return bits == 4 ? 1024 : 2048; }
__host__ __device__ constexpr int record_bytes(int bits) { return bits == 4 ? 40 : 48; }

// Geometry of one packed buffer (all offsets in bytes).  A block is its
// metadata (one record per group: 16 bf16 scales at 2c, then the 16 zero
// points -- W4 nibble c%2 of byte 32 + c/2, W8 byte 32 + c -- region padded
// to 16 bytes) followed by its k-tiles of codes.  In a k-tile, lane
// L = 16o + r of a wavefront owns 16 bytes at 16L (W4; W8 also 16 bytes at
// 1024 + 16L) holding rows 32u + 8o + i of column r for the four k-steps u.
struct Layout {
    int64_t K, N, G;
    int64_t ngroups;         // K / G
    int64_t ktiles;          // ceil(K / 128)
    int64_t steps;           // K / 32
    int64_t nblocks;         // ceil(N / 16)
    int64_t meta_bytes;      // records, padded to 16
    int64_t block_bytes;     // meta_bytes + ktiles * tile_bytes
    int64_t tiles_per_group; // G >= 128 (or G == K): k-tiles per group; else 0
    int64_t groups_per_tile; // G < 128: 128 / G; else 1

    __host__ __device__ static Layout make(int bits, int64_t K, int64_t N, int64_t G)
    {
        Layout l;
        l.K = K;
        l.N = N;
        l.G = G;
        l.ngroups = K / G;
        l.ktiles = (K + kTileRows - 1) / kTileRows;
        l.steps = K / kStepRows;
        l.nblocks = (N + kBlockCols - 1) / kBlockCols;
        l.meta_bytes = (l.ngroups * record_bytes(bits) + 15) / 16 * 16;
        l.block_bytes = l.meta_bytes + l.ktiles * tile_bytes(bits);
        const bool whole = G % kTileRows == 0 || G == K;
        l.tiles_per_group = whole ? (G == K ? l.ktiles : G / kTileRows) : 0;
        l.groups_per_tile = whole ? 1 : kTileRows / G;
        return l;
    }
    // every k-tile lies inside one group
    __host__ __device__ bool whole_tiles() const { return tiles_per_group > 0; }
    __host__ __device__ int64_t total_bytes() const { return nblocks * block_bytes; }
    __host__ __device__ int64_t record(int bits, int64_t blk, int64_t g) const
    {
        return blk * block_bytes + g * record_bytes(bits);
    }
    __host__ __device__ int64_t tile(int bits, int64_t blk, int64_t t) const
    {
        return blk * block_bytes + meta_bytes + t * tile_bytes(bits);
    }
};

// A 16-bit value (bf16, or fp16 when F16) widened to fp32, exactly.
template <bool F16> __device__ __forceinline__ float half_bits_to_f32(uint32_t b)
{
    if constexpr (F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    else
        return __uint_as_float(b << 16);
}

// Metadata of one column inside a record: scale (16-bit bits in the
// format of the call: bf16, or fp16 when F16) and zero point.
template <int BITS, bool F16 = false> __device__ __forceinline__ float record_scale(const uint8_t *rec, int c)
{
    return half_bits_to_f32<F16>(*reinterpret_cast<const uint16_t *>(rec + 2 * c));
}
template <int BITS> __device__ __forceinline__ uint32_t record_zero(const uint8_t *rec, int c)
{
    if constexpr (BITS == 4)
        return (rec[32 + (c >> 1)] >> (4 * (c & 1))) & 0xFu;
    else
        return rec[32 + c];
}

// AWQ checkpoint word: column 8c + j of a row lives in nibble kAwqNibble[j].
__device__ __forceinline__ uint32_t awq_nibble_shift(int j)
{
    // (0, 4, 1, 5, 2, 6, 3, 7) * 4 packed as 4-bit fields of one constant
    return ((0x73625140u >> (4 * j)) & 0xFu) * 4u;
}

// Position of row i (0..7) of a k-octet inside a packed W4 word: rows 2j and
// 2j+1 sit in nibbles j and j+4, so (word >> 4j) & 0x000F000F isolates the
// pair as the low and high halves of one 32-bit register.
__device__ __forceinline__ uint32_t w4_row_shift(int i) { return 4u * (uint32_t)(i / 2 + 4 * (i % 2)); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) { return (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu); }

// Output rounding: fp32 -> bf16 or fp16 (F16), nearest even; an fp16 value
// past 65504 rounds to infinity (v_cvt_f16_f32 in the default mode).
template <bool F16> __device__ __forceinline__ uint16_t f32_to_half_bits(float v)
{
    if constexpr (F16)
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    else
        return f32_to_bf16_bits(v);
}
template <bool F16> __device__ __forceinline__ uint32_t pack_half_x2(float lo, float hi)
{
    if constexpr (F16) {
        f32x2 f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    } else {
        return pack_bf16x2(lo, hi);
    }
}
// Operand building: two small integers (|v| <= 2^8, exact in either
// format) packed as 16-bit values; for fp16 the round-toward-zero pack
// (v_cvt_pkrtz_f16_f32) is exact and costs one instruction.
template <bool F16> __device__ __forceinline__ uint32_t pack_int_x2(float lo, float hi)
{
    if constexpr (F16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    else
        return pack_bf16x2(lo, hi);
}

template <bool F16 = false> __device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Streamed once per call: hint the memory system not to keep the lines.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

} // namespace tf
