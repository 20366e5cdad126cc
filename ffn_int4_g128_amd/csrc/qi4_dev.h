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
// Scales and zero points of four consecutive tiles (a "quad") are stored
// together per group, so a wave serving 1, 2 or 4 aligned tiles fetches them
// with one scale load and one zero load per lane.
constexpr int kQuadTiles = 4;
constexpr int kQuadScaleBytes = 128;   // [row 0..15][tile slot 0..3] binary16
constexpr int kQuadZeroBytes = 32;     // [row 0..15][2 bytes]: tile slot s in nibble s

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

// Quantization group sizes: 64, or a multiple of 128 that divides K (128,
// 256, ..., K for one scale and zero per row).  The kernels work on 128-wide
// blocks of K; with 64-wide groups a block holds two groups and its records
// two halves, else the records of every block of a group repeat that group's
// scale and zero (dequantization is per weight, so this is exact).
__host__ __device__ inline int halves_for(int group_size) { return group_size == 64 ? 2 : 1; }

// Byte offsets of the three regions of a packed matrix.  G counts 128-wide
// blocks of K.
struct PackedLayout {
    int64_t nt, nq, G;
    int halves;                 // 2 for 64-wide groups, else 1
    int64_t srec, zrec;         // bytes of one (quad, block) scale / zero record
    int64_t scales_off, zeros_off, bytes;
    __host__ __device__ PackedLayout(int64_t N, int64_t K, int flags, int group_size) {
        nt = num_tiles(N, flags);
        nq = (nt + kQuadTiles - 1) / kQuadTiles;
        G = K / kGroup;
        halves = halves_for(group_size);
        srec = (int64_t)kQuadScaleBytes * halves;
        zrec = (int64_t)kQuadZeroBytes * halves;
        scales_off = nt * G * kTileGroupBytes;
        zeros_off = scales_off + nq * G * srec;
        int64_t end = zeros_off + nq * G * zrec;
        bytes = (end + 255) & ~int64_t(255);
    }
    // Start of the (quad of tile t, block g) scale and zero records; half h
    // (64-wide groups: k in 128 g + 64 h + [0, 64)) starts kQuadScaleBytes * h
    // and kQuadZeroBytes * h further.  Within a half, row r's scale of tile t
    // is at + 8 r + 2 (t & 3) and its zero is nibble 4 (t & 1) of byte
    // + 2 r + ((t & 3) >> 1).
    __host__ __device__ int64_t scale_rec(int64_t t, int64_t g) const {
        return scales_off + ((t / kQuadTiles) * G + g) * srec;
    }
    __host__ __device__ int64_t zero_rec(int64_t t, int64_t g) const {
        return zeros_off + ((t / kQuadTiles) * G + g) * zrec;
    }
};

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return zero, which lets loads run unconditionally.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// Out-of-range offsets.  Valid lane offsets stay below 2^31 (every buffer is
// smaller than 2 GiB), so kOob (lane part) and kOobS (wave part) reach past
// every resource and their sum, at most 2^32 - 1, never wraps around.
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kOobS = 0x7FFFFFFFu;

__device__ inline uint4 buf_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Scale and zero records of NB (1, 2 or 4) aligned tiles of one quad for one
// row, one load each: lane offsets vs = 8 r + 2 slot0 and vz = 2 r + slot0 / 2
// (slot0 = first tile's slot in its quad), record starts os and oz in soffset.
// Afterwards the scale of tile nb is half (nb & 1) of sc[nb >> 1] and its zero
// is nibble nb of zb (NB = 1: nibble slot0 & 1).
template <int NB>
__device__ inline void load_meta(__amdgpu_buffer_rsrc_t r, uint32_t vs, uint32_t vz, uint32_t os,
                                 uint32_t oz, uint32_t *sc, uint32_t &zb) {
    static_assert(NB == 1 || NB == 2 || NB == 4, "tiles per quad load");
    if constexpr (NB == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, vs, os, 0);
        sc[0] = v[0];
        sc[1] = v[1];
        zb = __builtin_amdgcn_raw_buffer_load_b16(r, vz, oz, 0);
    } else {
        sc[0] = NB == 2 ? __builtin_amdgcn_raw_buffer_load_b32(r, vs, os, 0)
                        : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, vs, os, 0);
        zb = __builtin_amdgcn_raw_buffer_load_b8(r, vz, oz, 0);
    }
}

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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// int8 x int8 -> int32, 16x16 outputs, 64-deep: lane 16 j + r supplies 16 bytes
// of row r of A (and of column r of B) for the j-th quarter of the k range; the
// same (lane group, byte) position of A and B holds the same k.
__device__ inline i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
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
