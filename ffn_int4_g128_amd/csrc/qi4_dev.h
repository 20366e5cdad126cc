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
// every resource, and kOob + kOobS = 2^32 - 1 does not wrap around.  (The
// decode GEMM adds up to a few hundred bytes to a lane part of kOob for the
// fragments of a row past the end; with a wave part of kOobS such a sum wraps
// and the load may read the first bytes of the buffer, which only reach a
// result row that is never stored.)
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kOobS = 0x7FFFFFFFu;

__device__ inline uint4 buf_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// The same load with the non-temporal cache policy (the nt bit, 2 in the
// buffer instruction's cache-policy operand): for data read once per call,
// the weight codes of the decode GEMMs.  Measured on MI355X at MoE decode
// T = 32: the grouped gate/up GEMM 5.89 -> 6.29 TB/s, the step 47.5K -> 50.0K
// tokens/s; the streaming-read probe 6.0 -> 6.8-6.9 TB/s.  Not for the
// scale/zero records or the activations, which other waves and workgroups
// read again (measured: no gain or a loss), nor for the prefill's big tiles,
// whose expert's other tiles read the same weights again.
constexpr int kCpolNonTemporal = 2;
__device__ inline uint4 buf_b128_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNonTemporal));
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

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ inline f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// (a & m) | c in one VALU instruction (m in a scalar register, c in a vector
// register: a three-operand VALU op takes no literal here).
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

// fp16 1024 in both halves, produced opaquely so that it stays in one vector
// register instead of being rematerialized at every use.
__device__ inline uint32_t f16_magic_pair() {
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    return magic;
}

// Exact fp16 operands q - zero of the 8 codes of one packed dword, with the
// elements at k-offsets 2, 3, 6 and 7 sixteen times larger.  Masking a code in
// place under fp16 1024 (whose last mantissa bit weighs 1) gives 1024 + q for
// codes at bits 0..3 of a half and 1024 + 16 q for codes at bits 4..7; adding
// -(1024 + zero) or -(1024 + 16 zero) (packed fp16, exact) leaves q - zero or
// 16 (q - zero).  negz / negz16 hold those negated constants in both halves.
// One shift, four and-or and four packed adds per 8 codes.
__device__ inline uint4 codes_minus_zero_f16(uint32_t d, uint32_t negz, uint32_t negz16,
                                             uint32_t magic) {
    const f16x2 nz = __builtin_bit_cast(f16x2, negz), nz16 = __builtin_bit_cast(f16x2, negz16);
    const uint32_t t = d >> 8;
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(d, 0x000F000Fu, magic)) + nz);
    r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(d, 0x00F000F0u, magic)) + nz16);
    r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(t, 0x000F000Fu, magic)) + nz);
    r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(t, 0x00F000F0u, magic)) + nz16);
    return r;
}

// fp16 -(1024 + zero) and -(1024 + 16 zero) in both halves of a dword.
__device__ inline uint32_t f16_negz(uint32_t z) { return (0xE400u | z) * 0x00010001u; }
__device__ inline uint32_t f16_negz16(uint32_t z) { return (0xE400u | (z << 4)) * 0x00010001u; }

// ---- bf16 activations as exact fp16 operands ---------------------------------
//
// A bf16 value 2^(e-127) (1 + m/128) (exponent field e, 7 mantissa bits m) is
// an fp16 value times a power of two as long as it lands in fp16's range.  One
// power of two per (operand row, 128-wide block) is taken from the largest
// exponent field E of the row's 128 values: c = max(E - 29, 0), and the fp16
// operand is x * 2^(112 - c) (x * 2^(108 - c) at k-offsets 2, 3, 6, 7, whose
// weights are 16x).  Its bits are built from the bf16 bits with integer ops:
// (|bits| - (c << 7)) saturated at 0, shifted left by 3, with the sign put
// back.  Exponent fields e > c give exact fp16 normals (field e - c <= 29);
// e == c reads as an fp16 subnormal and e < c saturates to 0, an error below
// 2^-15 in the scaled units, i.e. below 2^-29 of the block's largest value.
// The product of the block's integer sums with 2^(c - 112) undoes the scale.

__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ inline uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a),
                                                                      __builtin_bit_cast(u16x2, b)));
}
__device__ inline uint32_t pk_shl3_u16(uint32_t a) {
    const u16x2 s = {3, 3};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) << s);
}

// Largest |bits| (sign cleared) of the 16 bf16 pairs of one lane, both halves.
__device__ inline uint32_t bf16_absmax_bits(const uint4 (&v)[4]) {
    uint32_t mx = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        mx = pk_max_u16(mx, v[s].x & 0x7FFF7FFFu);
        mx = pk_max_u16(mx, v[s].y & 0x7FFF7FFFu);
        mx = pk_max_u16(mx, v[s].z & 0x7FFF7FFFu);
        mx = pk_max_u16(mx, v[s].w & 0x7FFF7FFFu);
    }
    const uint32_t lo = mx & 0xFFFFu, hi = mx >> 16;
    return lo > hi ? lo : hi;
}

// The block exponent offset c of operand row r16 from this lane's |bits|
// maximum: the row's 128 values sit in lanes r16, r16 + 16, r16 + 32, r16 + 48
// (one per 16-lane row of the wave); the permlane swaps pair rows 0/1 and 2/3,
// then the wave's halves.
__device__ inline uint32_t row_block_offset(uint32_t mx) {
    const auto s16 = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
    mx = s16[0] > s16[1] ? s16[0] : s16[1];
    const auto s32 = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = s32[0] > s32[1] ? s32[0] : s32[1];
    const uint32_t E = mx >> 7;
    return E > 29u ? E - 29u : 0u;
}

// One lane's 8 bf16 values of a k step (4 dwords, k-offsets 0..7) -> fp16
// operands; cc = (c << 7) and cc4 = ((c + 4) << 7) in both halves.
__device__ inline f16x8 bf16_to_f16_scaled(uint4 v, uint32_t cc, uint32_t cc4) {
    uint4 r;
    r.x = (v.x & 0x80008000u) | pk_shl3_u16(pk_sub_sat_u16(v.x & 0x7FFF7FFFu, cc));
    r.y = (v.y & 0x80008000u) | pk_shl3_u16(pk_sub_sat_u16(v.y & 0x7FFF7FFFu, cc4));
    r.z = (v.z & 0x80008000u) | pk_shl3_u16(pk_sub_sat_u16(v.z & 0x7FFF7FFFu, cc));
    r.w = (v.w & 0x80008000u) | pk_shl3_u16(pk_sub_sat_u16(v.w & 0x7FFF7FFFu, cc4));
    return __builtin_bit_cast(f16x8, r);
}

}  // namespace qi4
