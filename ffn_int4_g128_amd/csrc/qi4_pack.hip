// Offline reorder of int4-g128 weights into the device layout, its exact
// inverse, and an exact float32 dequantization.
//
// The pages store the codes "group by group, so inference reads one contiguous
// span" ("FastLLM: zero-dependency CPU inference framework", section 3.1).  On
// CDNA4 the unit that must be contiguous is one wave load: 64 lanes x 16 bytes.
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
    if (!aligned(qweight, 4) || !aligned(scales, 2) || !aligned(packed, 16)) return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, K, flags, gs);
    const int64_t ng = K / gs;
    if (overlaps(packed, L.bytes, qweight, N * K / 2) ||
        overlaps(packed, L.bytes, scales, N * ng * 2) || overlaps(packed, L.bytes, zeros, N * ng))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    hipStream_t st = as_stream(stream);
    uint8_t *p = static_cast<uint8_t *>(packed);
    const int64_t n_dwords = L.nt * L.G * 256;
    pack_codes_kernel<<<grid_for(n_dwords), kThreads, 0, st>>>(
        qweight, N, K, flags, reinterpret_cast<uint32_t *>(p), n_dwords);
    if ((rc = launch_status())) return rc;
    const int64_t n_rec = L.nq * L.G * L.halves;
    pack_meta_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
        scales, zeros, N, K, flags, gs, L.nt, reinterpret_cast<uint64_t *>(p + L.scales_off),
        reinterpret_cast<uint16_t *>(p + L.zeros_off), n_rec);
    return launch_status();
}

int qi4_unpack(const void *packed, int64_t N, int64_t K, int group_size, int flags,
               uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (!qweight || !scales || !zeros || !packed) return QI4_ERR_NULL;
    if (!aligned(qweight, 4) || !aligned(scales, 2) || !aligned(packed, 16)) return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, K, flags, gs);
    const int64_t ng = K / gs;
    if (overlaps(packed, L.bytes, qweight, N * K / 2) ||
        overlaps(packed, L.bytes, scales, N * ng * 2) || overlaps(packed, L.bytes, zeros, N * ng))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    hipStream_t st = as_stream(stream);
    const uint8_t *p = static_cast<const uint8_t *>(packed);
    const int64_t n_dwords = L.nt * L.G * 256;
    unpack_codes_kernel<<<grid_for(n_dwords), kThreads, 0, st>>>(
        reinterpret_cast<const uint32_t *>(p), N, K, flags, qweight, n_dwords);
    if ((rc = launch_status())) return rc;
    const int64_t n_rec = L.nq * L.G * L.halves;
    unpack_meta_kernel<<<grid_for(n_rec * 16), kThreads, 0, st>>>(
        reinterpret_cast<const uint64_t *>(p + L.scales_off),
        reinterpret_cast<const uint16_t *>(p + L.zeros_off), N, K, flags, gs, L.nt,
        scales, zeros, n_rec);
    return launch_status();
}

int qi4_dequant_f32(const void *packed, int64_t N, int64_t K, int group_size, int flags,
                    float *w, void *stream) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (!packed || !w) return QI4_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(w, 16)) return QI4_ERR_SHAPE;
    const int gs = (int)effective_group(group_size, K);
    PackedLayout L(N, K, flags, gs);
    if (overlaps(packed, L.bytes, w, N * K * 4)) return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    const int64_t n_dwords = L.nt * L.G * 256;
    dequant_kernel<<<grid_for(n_dwords), kThreads, 0, as_stream(stream)>>>(
        static_cast<const uint8_t *>(packed), N, K, flags, gs, w, n_dwords);
    return launch_status();
}

}  // extern "C"
