// Device-side helpers shared by the libqi4 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qi4.h"

namespace qi4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kGroup = 128;        // weights per quantization group along K
constexpr int kTileRows = 16;      // rows per packed tile (one MFMA 16x16 column block)
constexpr int kTileGroupBytes = 1024;  // codes of one (tile, group) block: 64 lanes x 16 B
constexpr int kScaleBytes = 32;    // 16 binary16 scales per (tile, group)
constexpr int kZeroBytes = 8;      // 16 zero points, two per byte, per (tile, group)

// Number of 16-row tiles of an N-row matrix.  With the gate/up pairing the
// gate half and the up half are each padded to whole tiles.
__host__ __device__ inline int64_t num_tiles(int64_t N, int flags) {
    if (flags & QI4_PACK_GATEUP) return 2 * ((N / 2 + kTileRows - 1) / kTileRows);
    return (N + kTileRows - 1) / kTileRows;
}

// Canonical row held by row r (0..15) of tile t, or -1 for a padding row.
__host__ __device__ inline int64_t tile_row(int64_t t, int r, int64_t N, int flags) {
    if (flags & QI4_PACK_GATEUP) {
        int64_t half = N / 2;
        int64_t idx = (t >> 1) * kTileRows + r;
        if (idx >= half) return -1;
        return (t & 1) * half + idx;
    }
    int64_t row = t * kTileRows + r;
    return row < N ? row : -1;
}

// Byte offsets of the three regions of a packed matrix.
struct PackedLayout {
    int64_t nt, G;
    int64_t scales_off, zeros_off, bytes;
    __host__ __device__ PackedLayout(int64_t N, int64_t K, int flags) {
        nt = num_tiles(N, flags);
        G = K / kGroup;
        scales_off = nt * G * kTileGroupBytes;
        zeros_off = scales_off + nt * G * kScaleBytes;
        int64_t end = zeros_off + nt * G * kZeroBytes;
        bytes = (end + 255) & ~int64_t(255);
    }
};

// Within one lane's dword, the code of k-offset e (0..7) sits at nibble
// position (e >> 1) + 4 * (e & 1).  Unpacking then needs only a mask, a shift
// and an OR per pair: (d >> 4p) & 0x000F000F puts positions p and p+4, i.e.
// k-offsets 2p and 2p+1, into the low and high halves of a dword -- the order
// of two consecutive bf16 MFMA operand elements.
__host__ __device__ constexpr int nibble_pos(int e) { return (e >> 1) + 4 * (e & 1); }

// float32 -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ inline uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ inline float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Four codes pairs of one dword -> four dwords of bf16 pairs holding 128 + q.
// bf16 0x4300 is 128.0 and its last mantissa bit weighs 1, so OR-ing a code
// q <= 15 into the low mantissa bits gives exactly 128 + q.
__device__ inline uint4 unpack_codes_bf16(uint32_t d) {
    const uint32_t m = 0x000F000Fu, magic = 0x43004300u;
    uint4 r;
    r.x = (d & m) | magic;
    r.y = ((d >> 4) & m) | magic;
    r.z = ((d >> 8) & m) | magic;
    r.w = ((d >> 12) & m) | magic;
    return r;
}

}  // namespace qi4
