// int4-g128 weight-only GEMM for few rows of activations (decode, T <= 32 per
// problem per pass), on bf16 MFMA with float32 accumulation.
//
// The pages' pipeline is "read 4-bit weight -> dequantize -> multiply" with no
// separate dequantization pass ("FastLLM: zero-dependency CPU inference
// framework", section 3.1), and decode time is set by how fast the weights are
// read, not by arithmetic (same section: every token re-reads all weights).  On
// CDNA4 that becomes:
//  * one 16-byte load per lane per (16-row tile, 128-wide group): a contiguous
//    kilobyte per wave, prepared by qi4_pack;
//  * the codes become MFMA operands with one AND/OR per pair: bf16 with the
//    bits 0x4300 | q is exactly 128 + q;
//  * MFMA 16x16x32 bf16 multiplies the activations (as they are, bf16) with
//    those operands, giving acc = sum_k x * (128 + q) per group; a second MFMA
//    chain in the same order against a constant operand 128 + zero gives
//    xz = sum_k x * (128 + zero), and the group adds scale * (acc - xz), which
//    equals scale * sum_k x * (q - zero).  Both chains see identical operands
//    where q == zero, so an all-zero group contributes exactly 0;
//  * the K range is split across the waves of a workgroup and reduced in LDS in
//    a fixed order, so results are deterministic.
// Activations in float32 are split exactly into three bf16 terms (hi + mid +
// lo), each an MFMA row; the epilogue adds the rows of one token back together.
#include "qi4_gemm.h"
#include "qi4_host.h"

namespace qi4 {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kRedSlots = 16;   // (wave, m, nb) partial tiles the LDS buffer holds

// Part `part` of the exact split of v into bf16 terms v = hi + mid + lo.
__device__ inline uint32_t split_part(float v, int part) {
    const uint32_t hi = f32_to_bf16_rne(v);
    const float r1 = v - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    const uint32_t lo = f32_to_bf16_rne(r2);
    return part == 0 ? hi : part == 1 ? mid : part == 2 ? lo : 0u;
}

template <bool AF32>
__device__ inline uint4 load_a_frag(const void *row, int64_t elem, int part) {
    if constexpr (!AF32) {
        return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(row) + elem);
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(row) + elem);
        const float4 u = p[0], v = p[1];
        uint4 r;
        r.x = split_part(u.x, part) | (split_part(u.y, part) << 16);
        r.y = split_part(u.z, part) | (split_part(u.w, part) << 16);
        r.z = split_part(v.x, part) | (split_part(v.y, part) << 16);
        r.w = split_part(v.z, part) | (split_part(v.w, part) << 16);
        return r;
    }
}

template <int NB, int MT, bool AF32>
__global__ void __launch_bounds__(kMaxWaves * 64)
qgemm_kernel(const GemmArgs args) {
    __shared__ float red[kRedSlots * 256];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int W = blockDim.x >> 6;
    const int r16 = lane & 15;   // operand row / output column within the tile
    const int j = lane >> 4;     // k quarter of the operand, row block of the result

    // ---- which problem this workgroup serves
    const uint8_t *w;
    int64_t row0, n, src0 = 0;
    const int32_t *gather = nullptr;
    if (!args.moe) {
        w = args.w;
        row0 = 0;
        n = args.T;
    } else {
        const int py = blockIdx.y;
        if (py < args.routed_slots) {
            if (py >= args.active[0]) return;
            const int e = args.active[1 + py];
            row0 = args.offsets[e];
            n = args.offsets[e + 1] - row0;
            w = args.w + (int64_t)e * args.w_stride;
            if (args.gather_tokens) gather = args.sorted_pairs;
            else src0 = row0;
        } else {
            w = args.w_shared;
            row0 = args.T * args.top_k;
            n = args.T;
            src0 = args.gather_tokens ? 0 : row0;
        }
    }
    if (n <= 0) return;

    const PackedLayout L(args.N, args.K, args.flags);
    const int64_t nt = L.nt, G = L.G;
    const int64_t tile0 = (int64_t)blockIdx.x * NB;
    const uint4 *codes = reinterpret_cast<const uint4 *>(w);
    const uint16_t *scl = reinterpret_cast<const uint16_t *>(w + L.scales_off);
    const uint8_t *zrs = w + L.zeros_off;

    const int gb = (int)((G * wave) / W), ge = (int)((G * (wave + 1)) / W);
    const int P = args.P;
    const int spt = 16 / P;                 // slots per M tile
    const int64_t chunk = (int64_t)MT * spt;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    for (int64_t c0 = 0; c0 < n; c0 += chunk) {
        // ---- A rows of this lane (operand row r16 of each M tile)
        const void *arow[MT];
        bool avalid[MT];
        int apart[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int64_t slot = c0 + (int64_t)m * spt + r16 / P;
            const int part = r16 % P;
            const bool ok = (r16 < spt * P) && slot < n;
            avalid[m] = ok;
            apart[m] = part;
            arow[m] = nullptr;
            if (ok) {
                const int64_t src = gather ? (int64_t)(gather[row0 + slot] / args.top_k) : src0 + slot;
                if constexpr (AF32)
                    arow[m] = static_cast<const float *>(args.a) + src * args.lda;
                else
                    arow[m] = static_cast<const uint16_t *>(args.a) + (src * P + part) * args.lda;
            }
        }

        f32x4 res[MT][NB];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) res[m][nb] = zero4;

        for (int g = gb; g < ge; ++g) {
            uint4 cw[NB];
            float sc[NB];
            uint32_t zc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int64_t tile = tile0 + nb;
                if (tile < nt) {
                    const int64_t tg = tile * G + g;
                    cw[nb] = codes[tg * 64 + lane];
                    sc[nb] = f16_bits_to_f32(scl[tg * 16 + r16]);
                    zc[nb] = (zrs[tg * 8 + (r16 >> 1)] >> (4 * (r16 & 1))) & 15u;
                } else {
                    cw[nb] = make_uint4(0, 0, 0, 0);
                    sc[nb] = 0.f;
                    zc[nb] = 0u;
                }
            }
            uint4 af[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    af[m][s] = avalid[m] ? load_a_frag<AF32>(arow[m], (int64_t)g * 128 + 32 * s + 8 * j, apart[m])
                                         : make_uint4(0, 0, 0, 0);

#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const bf16x8 b0 = as_bf16x8(unpack_codes_bf16(cw[nb].x));
                const bf16x8 b1 = as_bf16x8(unpack_codes_bf16(cw[nb].y));
                const bf16x8 b2 = as_bf16x8(unpack_codes_bf16(cw[nb].z));
                const bf16x8 b3 = as_bf16x8(unpack_codes_bf16(cw[nb].w));
                const uint32_t zz = (0x4300u | zc[nb]) * 0x00010001u;   // bf16 pair (128+z, 128+z)
                const bf16x8 bz = as_bf16x8(make_uint4(zz, zz, zz, zz));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    f32x4 acc = mfma16x16x32(as_bf16x8(af[m][0]), b0, zero4);
                    f32x4 xz = mfma16x16x32(as_bf16x8(af[m][0]), bz, zero4);
                    acc = mfma16x16x32(as_bf16x8(af[m][1]), b1, acc);
                    xz = mfma16x16x32(as_bf16x8(af[m][1]), bz, xz);
                    acc = mfma16x16x32(as_bf16x8(af[m][2]), b2, acc);
                    xz = mfma16x16x32(as_bf16x8(af[m][2]), bz, xz);
                    acc = mfma16x16x32(as_bf16x8(af[m][3]), b3, acc);
                    xz = mfma16x16x32(as_bf16x8(af[m][3]), bz, xz);
#pragma unroll
                    for (int v = 0; v < 4; ++v) res[m][nb][v] += sc[nb] * (acc[v] - xz[v]);
                }
            }
        }

        // ---- fixed-order reduction of the waves' partial sums
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[((wave * MT + m) * NB + nb) * 256 + v * 64 + lane] = res[m][nb][v];
        __syncthreads();

        const int pairs = args.epi == QI4_EPI_SILU_MUL ? NB / 2 : NB;
        const int items = MT * pairs * 64;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int l = it & 63;
            const int rest = it >> 6;
            const int pi = rest % pairs;
            const int m = rest / pairs;
            const int nbA = args.epi == QI4_EPI_SILU_MUL ? 2 * pi : pi;
            float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
            for (int ww = 0; ww < W; ++ww) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    a4[v] += red[((ww * MT + m) * NB + nbA) * 256 + v * 64 + l];
                    if (args.epi == QI4_EPI_SILU_MUL)
                        b4[v] += red[((ww * MT + m) * NB + nbA + 1) * 256 + v * 64 + l];
                }
            }
            const int col = l & 15;
            const int64_t tile = tile0 + nbA;
            int64_t oc;
            if (args.epi == QI4_EPI_SILU_MUL)
                oc = (tile >> 1) * 16 + col;
            else
                oc = tile < nt ? tile_row(tile, col, args.N, args.flags) : -1;
            if (oc < 0 || oc >= args.n_out) continue;
            const int rbase = 4 * (l >> 4);
            for (int v0 = 0; v0 < 4; v0 += P) {
                const int r = rbase + v0;
                if (r / P >= spt) continue;
                const int64_t slot = c0 + (int64_t)m * spt + r / P;
                if (slot >= n) continue;
                float val = 0.f, uval = 0.f;
                for (int p = 0; p < P; ++p) {
                    val += a4[v0 + p];
                    uval += b4[v0 + p];
                }
                if (args.epi == QI4_EPI_SILU_MUL) val = val / (1.0f + expf(-val)) * uval;
                const int64_t dst = row0 + slot;
                if (args.out_mode == OUT_F32) {
                    static_cast<float *>(args.out)[dst * args.ldo + oc] = val;
                } else if (args.out_mode == OUT_BF16) {
                    static_cast<uint16_t *>(args.out)[dst * args.ldo + oc] = (uint16_t)f32_to_bf16_rne(val);
                } else {
                    const uint32_t hi = f32_to_bf16_rne(val);
                    const uint32_t lo = f32_to_bf16_rne(val - bf16_to_f32(hi));
                    uint16_t *o = static_cast<uint16_t *>(args.out);
                    o[(dst * 2) * args.ldo + oc] = (uint16_t)hi;
                    o[(dst * 2 + 1) * args.ldo + oc] = (uint16_t)lo;
                }
            }
        }
        __syncthreads();
    }
}

template <int NB, int MT>
int launch_nb_mt(const GemmArgs &a, dim3 grid, int threads, hipStream_t st) {
    if (a.a_f32)
        qgemm_kernel<NB, MT, true><<<grid, threads, 0, st>>>(a);
    else
        qgemm_kernel<NB, MT, false><<<grid, threads, 0, st>>>(a);
    return launch_status();
}

}  // namespace

int launch_qgemm(const GemmArgs &args, int n_problems, int64_t max_slots, hipStream_t st) {
    if (n_problems <= 0 || max_slots <= 0) return QI4_OK;
    const int64_t nt = num_tiles(args.N, args.flags);
    const int64_t G = args.K / kGroup;
    const int spt = 16 / args.P;
    const int MT = max_slots > spt ? 2 : 1;
    const int nb_min = args.epi == QI4_EPI_SILU_MUL ? 2 : 1;
    int NB = 4;
    while (NB > nb_min && ceil_div(nt, NB) * n_problems < 2048) NB /= 2;
    int W = kMaxWaves;
    while (W > 1 && (G / W < 2 || W * MT * NB > kRedSlots)) W /= 2;
    const int64_t gx = ceil_div(nt, NB);
    if (gx > 0x7fffffff || n_problems > 65535) return QI4_ERR_SHAPE;
    dim3 grid((unsigned)gx, (unsigned)n_problems);
    const int threads = W * 64;
    if (MT == 1) {
        if (NB == 4) return launch_nb_mt<4, 1>(args, grid, threads, st);
        if (NB == 2) return launch_nb_mt<2, 1>(args, grid, threads, st);
        return launch_nb_mt<1, 1>(args, grid, threads, st);
    }
    if (NB == 4) return launch_nb_mt<4, 2>(args, grid, threads, st);
    if (NB == 2) return launch_nb_mt<2, 2>(args, grid, threads, st);
    return launch_nb_mt<1, 2>(args, grid, threads, st);
}

}  // namespace qi4

using namespace qi4;

extern "C" int qlinear_int4_g128(const void *x, int x_dtype, int64_t T, int64_t K,
                                 const void *packed_w, int64_t N, int flags, void *y,
                                 int y_dtype, int epilogue, void *stream) {
    int rc = check_matrix(N, K, 128, flags);
    if (rc) return rc;
    if (x_dtype != QI4_F32 && x_dtype != QI4_BF16) return QI4_ERR_DTYPE;
    if (y_dtype != QI4_F32 && y_dtype != QI4_BF16) return QI4_ERR_DTYPE;
    if (epilogue != QI4_EPI_NONE && epilogue != QI4_EPI_SILU_MUL) return QI4_ERR_DTYPE;
    if (epilogue == QI4_EPI_SILU_MUL && flags != QI4_PACK_GATEUP) return QI4_ERR_UNSUPPORTED;
    if (T < 0 || T > (int64_t(1) << 31)) return QI4_ERR_SHAPE;
    if (T == 0) return QI4_OK;
    if (!x || !packed_w || !y) return QI4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed_w, 16) || !aligned(y, 4)) return QI4_ERR_SHAPE;
    const int64_t n_out = epilogue == QI4_EPI_SILU_MUL ? N / 2 : N;
    const int64_t xb = T * K * (x_dtype == QI4_F32 ? 4 : 2);
    const int64_t yb = T * n_out * (y_dtype == QI4_F32 ? 4 : 2);
    const int64_t wb = PackedLayout(N, K, flags).bytes;
    if (overlaps(y, yb, x, xb) || overlaps(y, yb, packed_w, wb)) return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;

    GemmArgs a = {};
    a.w = static_cast<const uint8_t *>(packed_w);
    a.N = N;
    a.K = K;
    a.flags = flags;
    a.a = x;
    a.lda = K;
    a.a_f32 = x_dtype == QI4_F32;
    a.P = a.a_f32 ? 4 : 1;
    a.moe = 0;
    a.T = T;
    a.out = y;
    a.ldo = n_out;
    a.out_mode = y_dtype == QI4_F32 ? OUT_F32 : OUT_BF16;
    a.epi = epilogue;
    a.n_out = n_out;
    return launch_qgemm(a, 1, T, as_stream(stream));
}
