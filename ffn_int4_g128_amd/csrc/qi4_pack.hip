// Offline reorder of int4-g128 weights (and 8-bit ones, as two 4-bit planes)
// into the device layout, its exact inverse, and an exact float32
// dequantization.
//
// The FastLLM page (section 3.1) keeps the codes of a group together in memory
// so that the product streams through contiguous bytes.  On CDNA4 the unit
// that must be contiguous is one wave load: 64 lanes x 16 bytes.
// Each (16-row tile, 128-wide group) block is exactly that kilobyte, ordered so
// that lane 16*j + r receives row r's codes for the k values its MFMA operand
// fragment consumes (see qi4.h for the full description).
#include "qi4_dev.h"
#include "qi4_host.h"

namespace qi4 {
namespace {

constexpr int kThreads = 256;

// One thread per packed dword: 8 codes of one row, k in [k0, k0 + 8).
__global__ void __launch_bounds__(kThreads)
pack_codes_kernel(const uint8_t *__restrict__ qweight, int64_t N, int64_t K, int flags,
                  uint32_t *__restrict__ out, int64_t n_dwords) {
    const int64_t G = K / kGroup;
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_dwords;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tg = idx >> 8;           // tile * G + g
        const int64_t t = tg / G, g = tg % G;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        uint32_t o = 0;
        if (row >= 0) {
            const int64_t k0 = g * kGroup + 32 * s + 8 * j;
            // codes k0..k0+7 are bytes k0/2..k0/2+3 of the row: code e at bit 4e
            const uint32_t in = *reinterpret_cast<const uint32_t *>(qweight + row * (K / 2) + k0 / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) o |= ((in >> (4 * e)) & 15u) << (4 * nibble_pos(e));
        }
        out[idx] = o;
    }
}

// One thread per (quad, block, half, row): the scales and zeros of that row in
// the quad's four tiles (missing tiles and rows hold 0).  Half h of block b
// holds group 2 b + h for 64-wide groups, else the group of the block.
__global__ void __launch_bounds__(kThreads)
pack_meta_kernel(const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                 int64_t N, int64_t K, int flags, int gs, int64_t nt,
                 uint64_t *__restrict__ sc_out, uint16_t *__restrict__ zr_out, int64_t n_rec) {
    const int64_t G = K / kGroup, ng = K / gs;
    const int H = halves_for(gs);
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_rec * 16;
         idx += (int64_t)gridDim.x * kThreads) {
        const int r = idx & 15;
        const int64_t rec = idx >> 4;               // (quad * G + block) * H + half
        const int h = (int)(rec % H);
        const int64_t qb = rec / H;
        const int64_t q = qb / G, b = qb % G;
        const int64_t g = H == 2 ? 2 * b + h : b * kGroup / gs;
        uint64_t sv = 0;
        uint32_t zv = 0;
#pragma unroll
        for (int s = 0; s < kQuadTiles; ++s) {
            const int64_t t = q * kQuadTiles + s;
            const int64_t row = t < nt ? tile_row(t, r, N, flags) : -1;
            if (row < 0) continue;
            sv |= (uint64_t)scales[row * ng + g] << (16 * s);
            zv |= (zeros[row * ng + g] & 15u) << (4 * s);
        }
        sc_out[idx] = sv;
        zr_out[idx] = (uint16_t)zv;
    }
}

__global__ void __launch_bounds__(kThreads)
unpack_codes_kernel(const uint32_t *__restrict__ in, int64_t N, int64_t K, int flags,
                    uint8_t *__restrict__ qweight, int64_t n_dwords) {
    const int64_t G = K / kGroup;
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_dwords;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tg = idx >> 8;
        const int64_t t = tg / G, g = tg % G;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        if (row < 0) continue;
        const int64_t k0 = g * kGroup + 32 * s + 8 * j;
        const uint32_t d = in[idx];
        uint32_t o = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) o |= ((d >> (4 * nibble_pos(e))) & 15u) << (4 * e);
        *reinterpret_cast<uint32_t *>(qweight + row * (K / 2) + k0 / 2) = o;
    }
}

// The inverse: every group is read back from the first record that holds it.
__global__ void __launch_bounds__(kThreads)
unpack_meta_kernel(const uint64_t *__restrict__ sc_in, const uint16_t *__restrict__ zr_in,
                   int64_t N, int64_t K, int flags, int gs, int64_t nt,
                   uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros, int64_t n_rec) {
    const int64_t G = K / kGroup, ng = K / gs;
    const int H = halves_for(gs);
    const int64_t bpg = H == 2 ? 1 : gs / kGroup;   // blocks per group
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_rec * 16;
         idx += (int64_t)gridDim.x * kThreads) {
        const int r = idx & 15;
        const int64_t rec = idx >> 4;
        const int h = (int)(rec % H);
        const int64_t qb = rec / H;
        const int64_t q = qb / G, b = qb % G;
        if (b % bpg != 0) continue;                  // a repeat of an earlier block
        const int64_t g = H == 2 ? 2 * b + h : b / bpg;
        const uint64_t sv = sc_in[idx];
        const uint32_t zv = zr_in[idx];
#pragma unroll
        for (int s = 0; s < kQuadTiles; ++s) {
            const int64_t t = q * kQuadTiles + s;
            const int64_t row = t < nt ? tile_row(t, r, N, flags) : -1;
            if (row < 0) continue;
            scales[row * ng + g] = (uint16_t)(sv >> (16 * s));
            zeros[row * ng + g] = (uint8_t)((zv >> (4 * s)) & 15u);
        }
    }
}

// One thread per packed dword: 8 consecutive weights of one row in float32.
__global__ void __launch_bounds__(kThreads)
dequant_kernel(const uint8_t *__restrict__ packed, int64_t N, int64_t K, int flags, int gs,
               float *__restrict__ w, int64_t n_dwords) {
    const int64_t G = K / kGroup;
    const PackedLayout L(N, K, flags, gs);
    const uint32_t *codes = reinterpret_cast<const uint32_t *>(packed);
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_dwords;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tg = idx >> 8;
        const int64_t t = tg / G, g = tg % G;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        if (row < 0) continue;
        const int64_t k0 = g * kGroup + 32 * s + 8 * j;
        const uint32_t d = codes[idx];
        const int h = L.halves == 2 ? (32 * s + 8 * j) / 64 : 0;   // half of the block
        const float scale = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(
            packed + L.scale_rec(t, g) + kQuadScaleBytes * h + 8 * r + 2 * (t & 3)));
        const int z = (packed[L.zero_rec(t, g) + kQuadZeroBytes * h + 2 * r + ((t & 3) >> 1)] >>
                       (4 * (t & 1))) & 15;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = (d >> (4 * nibble_pos(e))) & 15;
            v[e] = scale * (float)(q - z);
        }
        float4 *dst = reinterpret_cast<float4 *>(w + row * K + k0);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ---- 8-bit matrices: two 4-bit planes ----------------------------------------
// Block 2b of the packed width-2K matrix holds the high nibbles of block b of
// the 8-bit matrix (zero z >> 4, scale 16 s), block 2b + 1 the low nibbles
// (zero z & 15, scale s).  Kp = 2K is the packed width.

// binary16 bits of 16 * s (exact whenever the product is a binary16).
__device__ inline uint32_t f16_times16(uint32_t sb) {
    const _Float16 v = (_Float16)(f16_bits_to_f32((uint16_t)sb) * 16.0f);
    return __builtin_bit_cast(uint16_t, v);
}

// One thread per packed dword of either plane.
__global__ void __launch_bounds__(kThreads)
pack_codes8_kernel(const uint8_t *__restrict__ qweight, int64_t N, int64_t K, int flags,
                   uint32_t *__restrict__ out, int64_t n_dwords) {
    const int64_t Gp = 2 * (K / kGroup);
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_dwords;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tg = idx >> 8;           // tile * Gp + packed block
        const int64_t t = tg / Gp, bp = tg % Gp;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        uint32_t o = 0;
        if (row >= 0) {
            const int64_t k0 = (bp >> 1) * kGroup + 32 * s + 8 * j;
            const uint2 in = *reinterpret_cast<const uint2 *>(qweight + row * K + k0);
            const int sh = (bp & 1) ? 0 : 4;   // low plane: bits 0..3, high plane: 4..7
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t byte = ((e < 4 ? in.x : in.y) >> (8 * (e & 3))) & 0xFFu;
                o |= ((byte >> sh) & 15u) << (4 * nibble_pos(e));
            }
        }
        out[idx] = o;
    }
}

// One thread per (quad, packed block, half, row) record.
__global__ void __launch_bounds__(kThreads)
pack_meta8_kernel(const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
                  int64_t N, int64_t K, int flags, int gs, int64_t nt,
                  uint64_t *__restrict__ sc_out, uint16_t *__restrict__ zr_out, int64_t n_rec) {
    const int64_t Gp = 2 * (K / kGroup), ng = K / gs;
    const int H = halves_for(gs);
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_rec * 16;
         idx += (int64_t)gridDim.x * kThreads) {
        const int r = idx & 15;
        const int64_t rec = idx >> 4;               // (quad * Gp + packed block) * H + half
        const int h = (int)(rec % H);
        const int64_t qb = rec / H;
        const int64_t q = qb / Gp, bp = qb % Gp, b = bp >> 1;
        const bool low = bp & 1;
        const int64_t g = H == 2 ? 2 * b + h : b * kGroup / gs;
        uint64_t sv = 0;
        uint32_t zv = 0;
#pragma unroll
        for (int sl = 0; sl < kQuadTiles; ++sl) {
            const int64_t t = q * kQuadTiles + sl;
            const int64_t row = t < nt ? tile_row(t, r, N, flags) : -1;
            if (row < 0) continue;
            const uint32_t sb = scales[row * ng + g], z = zeros[row * ng + g];
            sv |= (uint64_t)(low ? sb : f16_times16(sb)) << (16 * sl);
            zv |= (low ? (z & 15u) : (z >> 4)) << (4 * sl);
        }
        sc_out[idx] = sv;
        zr_out[idx] = (uint16_t)zv;
    }
}

// One thread per dword of the high plane: the 8 codes it and its low-plane
// twin (the next block, 256 dwords on) hold.
__global__ void __launch_bounds__(kThreads)
unpack_codes8_kernel(const uint32_t *__restrict__ in, int64_t N, int64_t K, int flags,
                     uint8_t *__restrict__ qweight, int64_t n_threads) {
    const int64_t G = K / kGroup;
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_threads;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tb = idx >> 8;            // tile * G + block
        const int64_t t = tb / G, b = tb % G;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        if (row < 0) continue;
        const int64_t hi_idx = ((t * 2 * G + 2 * b) << 8) | (idx & 255);
        const uint32_t dh = in[hi_idx], dl = in[hi_idx + 256];
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t q = (((dh >> (4 * nibble_pos(e))) & 15u) << 4) |
                               ((dl >> (4 * nibble_pos(e))) & 15u);
            o[e >> 2] |= q << (8 * (e & 3));
        }
        const int64_t k0 = b * kGroup + 32 * s + 8 * j;
        *reinterpret_cast<uint2 *>(qweight + row * K + k0) = make_uint2(o[0], o[1]);
    }
}

// One thread per (quad, block of K, half, row): scale from the low plane's
// record, zero from both.  Every group is read back from its first block.
__global__ void __launch_bounds__(kThreads)
unpack_meta8_kernel(const uint64_t *__restrict__ sc_in, const uint16_t *__restrict__ zr_in,
                    int64_t N, int64_t K, int flags, int gs, int64_t nt,
                    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros, int64_t n_rec) {
    const int64_t G = K / kGroup, Gp = 2 * G, ng = K / gs;
    const int H = halves_for(gs);
    const int64_t bpg = H == 2 ? 1 : gs / kGroup;
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_rec * 16;
         idx += (int64_t)gridDim.x * kThreads) {
        const int r = idx & 15;
        const int64_t rec = idx >> 4;               // (quad * G + block) * H + half
        const int h = (int)(rec % H);
        const int64_t qb = rec / H;
        const int64_t q = qb / G, b = qb % G;
        if (b % bpg != 0) continue;
        const int64_t g = H == 2 ? 2 * b + h : b / bpg;
        const int64_t hi = (((q * Gp + 2 * b) * H + h) << 4) | r;
        const int64_t lo = (((q * Gp + 2 * b + 1) * H + h) << 4) | r;
        const uint64_t sv = sc_in[lo];
        const uint32_t zh = zr_in[hi], zl = zr_in[lo];
#pragma unroll
        for (int sl = 0; sl < kQuadTiles; ++sl) {
            const int64_t t = q * kQuadTiles + sl;
            const int64_t row = t < nt ? tile_row(t, r, N, flags) : -1;
            if (row < 0) continue;
            scales[row * ng + g] = (uint16_t)(sv >> (16 * sl));
            zeros[row * ng + g] =
                (uint8_t)((((zh >> (4 * sl)) & 15u) << 4) | ((zl >> (4 * sl)) & 15u));
        }
    }
}

// One thread per dword of the high plane: 8 consecutive weights in float32.
__global__ void __launch_bounds__(kThreads)
dequant8_kernel(const uint8_t *__restrict__ packed, int64_t N, int64_t K, int flags, int gs,
                float *__restrict__ w, int64_t n_threads) {
    const int64_t G = K / kGroup;
    const PackedLayout L(N, 2 * K, flags, gs);
    const uint32_t *codes = reinterpret_cast<const uint32_t *>(packed);
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_threads;
         idx += (int64_t)gridDim.x * kThreads) {
        const int s = idx & 3;
        const int lane = (idx >> 2) & 63;
        const int64_t tb = idx >> 8;
        const int64_t t = tb / G, b = tb % G;
        const int r = lane & 15, j = lane >> 4;
        const int64_t row = tile_row(t, r, N, flags);
        if (row < 0) continue;
        const int64_t hi_idx = ((t * 2 * G + 2 * b) << 8) | (idx & 255);
        const uint32_t dh = codes[hi_idx], dl = codes[hi_idx + 256];
        const int h = L.halves == 2 ? (32 * s + 8 * j) / 64 : 0;
        const float scale = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(
            packed + L.scale_rec(t, 2 * b + 1) + kQuadScaleBytes * h + 8 * r + 2 * (t & 3)));
        const int zo = kQuadZeroBytes * h + 2 * r + ((t & 3) >> 1), zs = 4 * (t & 1);
        const int z = (((packed[L.zero_rec(t, 2 * b) + zo] >> zs) & 15) << 4) |
                      ((packed[L.zero_rec(t, 2 * b + 1) + zo] >> zs) & 15);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = (int)((((dh >> (4 * nibble_pos(e))) & 15u) << 4) |
                                ((dl >> (4 * nibble_pos(e))) & 15u));
            v[e] = scale * (float)(q - z);
        }
        const int64_t k0 = b * kGroup + 32 * s + 8 * j;
        float4 *dst = reinterpret_cast<float4 *>(w + row * K + k0);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

inline int grid_for(int64_t n) {
    int64_t b = ceil_div(n, kThreads);
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (int)b;
}

}  // namespace
}  // namespace qi4

using namespace qi4;

extern "C" {

int qi4_pack(const uint8_t *qweight, const uint16_t *scales, const uint8_t *zeros, int64_t N,
             int64_t K, int group_size, int flags, void *packed, void *stream) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (!qweight || !scales || !zeros || !packed) return QI4_ERR_NULL;
    const bool b8 = flags & QI4_INT8;
    if (!aligned(qweight, b8 ? 8 : 4) || !aligned(scales, 2) || !aligned(packed, 16))
        return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, packed_k(K, flags), flags, gs);
    const int64_t ng = K / gs;
    if (overlaps(packed, L.bytes, qweight, code_bytes(N, K, flags)) ||
        overlaps(packed, L.bytes, scales, N * ng * 2) || overlaps(packed, L.bytes, zeros, N * ng))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    hipStream_t st = as_stream(stream);
    uint8_t *p = static_cast<uint8_t *>(packed);
    const int64_t n_dwords = L.nt * L.G * 256;
    const int64_t n_rec = L.nq * L.G * L.halves;
    uint64_t *sc_out = reinterpret_cast<uint64_t *>(p + L.scales_off);
    uint16_t *zr_out = reinterpret_cast<uint16_t *>(p + L.zeros_off);
    if (b8) {
        pack_codes8_kernel<<<grid_for(n_dwords), kThreads, 0, st>>>(
            qweight, N, K, flags, reinterpret_cast<uint32_t *>(p), n_dwords);
        if ((rc = launch_status())) return rc;
        pack_meta8_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
            scales, zeros, N, K, flags, gs, L.nt, sc_out, zr_out, n_rec);
        return launch_status();
    }
    pack_codes_kernel<<<grid_for(n_dwords), kThreads, 0, st>>>(
        qweight, N, K, flags, reinterpret_cast<uint32_t *>(p), n_dwords);
    if ((rc = launch_status())) return rc;
    pack_meta_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
        scales, zeros, N, K, flags, gs, L.nt, sc_out, zr_out, n_rec);
    return launch_status();
}

int qi4_unpack(const void *packed, int64_t N, int64_t K, int group_size, int flags,
               uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (!qweight || !scales || !zeros || !packed) return QI4_ERR_NULL;
    const bool b8 = flags & QI4_INT8;
    if (!aligned(qweight, b8 ? 8 : 4) || !aligned(scales, 2) || !aligned(packed, 16))
        return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, packed_k(K, flags), flags, gs);
    const int64_t ng = K / gs;
    if (overlaps(packed, L.bytes, qweight, code_bytes(N, K, flags)) ||
        overlaps(packed, L.bytes, scales, N * ng * 2) || overlaps(packed, L.bytes, zeros, N * ng))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    hipStream_t st = as_stream(stream);
    const uint8_t *p = static_cast<const uint8_t *>(packed);
    const uint64_t *sc_in = reinterpret_cast<const uint64_t *>(p + L.scales_off);
    const uint16_t *zr_in = reinterpret_cast<const uint16_t *>(p + L.zeros_off);
    if (b8) {
        // one thread per dword of the high plane / record of a block of K
        const int64_t n_threads = L.nt * (L.G / 2) * 256;
        unpack_codes8_kernel<<<grid_for(n_threads), kThreads, 0, st>>>(
            reinterpret_cast<const uint32_t *>(p), N, K, flags, qweight, n_threads);
        if ((rc = launch_status())) return rc;
        const int64_t n_rec = L.nq * (L.G / 2) * L.halves;
        unpack_meta8_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
            sc_in, zr_in, N, K, flags, gs, L.nt, scales, zeros, n_rec);
        return launch_status();
    }
    const int64_t n_dwords = L.nt * L.G * 256;
    unpack_codes_kernel<<<grid_for(n_dwords), kThreads, 0, st>>>(
        reinterpret_cast<const uint32_t *>(p), N, K, flags, qweight, n_dwords);
    if ((rc = launch_status())) return rc;
    const int64_t n_rec = L.nq * L.G * L.halves;
    unpack_meta_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
        sc_in, zr_in, N, K, flags, gs, L.nt, scales, zeros, n_rec);
    return launch_status();
}

int qi4_dequant_f32(const void *packed, int64_t N, int64_t K, int group_size, int flags,
                    float *w, void *stream) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (!packed || !w) return QI4_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(w, 16)) return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, packed_k(K, flags), flags, gs);
    if (overlaps(packed, L.bytes, w, N * K * 4)) return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    if (flags & QI4_INT8) {
        const int64_t n_threads = L.nt * (L.G / 2) * 256;
        dequant8_kernel<<<grid_for(n_threads), kThreads, 0, as_stream(stream)>>>(
            static_cast<const uint8_t *>(packed), N, K, flags, gs, w, n_threads);
        return launch_status();
    }
    const int64_t n_dwords = L.nt * L.G * 256;
    dequant_kernel<<<grid_for(n_dwords), kThreads, 0, as_stream(stream)>>>(
        static_cast<const uint8_t *>(packed), N, K, flags, gs, w, n_dwords);
    return launch_status();
}

}  // extern "C"
