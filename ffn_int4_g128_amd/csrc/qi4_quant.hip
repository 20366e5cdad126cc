// Load-time quantizer: float32 or bf16 weights -> canonical 4-bit (or 8-bit)
// codes, scales and zero points for groups of 64, 128, 256, ... (up to a whole
// row) along K.
//
// The fastllm README (gittoolsai.com), section "model export", notes that
// loading a model with an int4 dtype quantizes it online at every load, which is
// slow.  This kernel does that step on the GPU.  Per group of weights w of one
// row (asymmetric min/max, with 0 always inside the range):
//   lo = min(0, min w), hi = max(0, max w)
//   scale = (hi - lo) / L rounded to binary16 (nearest, ties to even);
//           1.0 when that rounds to 0
//   zero  = clamp(rint(-lo / scale), 0, L)
//   q     = clamp(rint(w / scale) + zero, 0, L)          rint: half to even
// with L = 15 levels for 4-bit codes and 255 for 8-bit ones (the --quant-bit 8
// option of the FastLLM page, section 4.2).
// The decisions are those of the formula evaluated in binary64 (float32 and
// bf16 widen exactly; divisions are correctly rounded); the per-weight quotient
// is formed in float32 and checked against the rounding boundaries (below).
// NaN weights are ignored by the min/max; their codes are unspecified (finite
// weights are the contract).
#include "qi4_dev.h"
#include "qi4_host.h"

namespace qi4 {
namespace {

constexpr int kQuantWaves = 4;    // waves per workgroup
constexpr int kQuantPasses = 4;   // passes per wave, loads issued together

// Nearest binary16 (ties to even) of a non-negative, non-NaN double.  Scaling
// by a power of two is exact, so rint of the scaled value is the rounding.
__device__ inline uint32_t f64_to_f16_bits_rne(double v) {
    if (v == 0.0) return 0u;
    if (!(v < 65520.0)) return 0x7C00u;   // rounds to infinity (also v == inf)
    const int e = ilogb(v);                // v in [2^e, 2^(e+1))
    if (e < -14) {
        // subnormal quantum 2^-24; 1024 quanta is the smallest normal 0x0400
        return (uint32_t)rint(ldexp(v, 24));
    }
    double m = rint(ldexp(v, 10 - e));     // in [1024, 2048]
    int be = e + 15;
    if (m == 2048.0) {
        m = 1024.0;
        ++be;
    }
    if (be >= 31) return 0x7C00u;
    return ((uint32_t)be << 10) | ((uint32_t)m - 1024u);
}

template <int BITS>
__device__ inline double clampL(double v) {
    constexpr double L = (double)((1 << BITS) - 1);
    return v < 0.0 ? 0.0 : (v > L ? L : v);
}

// Eight consecutive weights (float32 or bf16) at element offset off.
template <bool F32>
__device__ inline void load8(const void *w, int64_t off, float (&v)[8]) {
    if constexpr (F32) {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(w) + off);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(w) + off + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(w) + off);
        const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[2 * c] = bf16_to_f32(u[c] & 0xFFFFu);
            v[2 * c + 1] = bf16_to_f32(u[c] >> 16);
        }
    }
}

// Scale (binary16 bits and value) and zero of a group with range [lo, hi].
template <int BITS>
__device__ inline void scale_zero(float lo, float hi, uint32_t &sb, double &s, double &z) {
    sb = f64_to_f16_bits_rne(((double)hi - (double)lo) / (double)((1 << BITS) - 1));
    s = (double)__builtin_bit_cast(_Float16, (uint16_t)sb);
    if (s == 0.0) {
        sb = 0x3C00u;   // binary16 1.0
        s = 1.0;
    }
    z = clampL<BITS>(rint(-(double)lo / s));
}

// Codes of eight weights: 4-bit codes packed even k in the low nibble (low 32
// bits), 8-bit codes one per byte.  rint(w / s) is formed from x = w * (1/s)
// in float32 (w and s are exact in float32; two roundings: |x - w/s| <= |x| 2^-23,
// at most 6.2e-5 for |x| <= 2 (L + 1)).  Away from the half-integers x rounds
// like w/s; within 1e-4 of one (|x - rint(x)| > 0.4999) the decision is taken
// on the binary64 quotient, in a branch that the lanes needing it take alone
// (a wave where none does skips it).  The sum with the zero point is exact in
// float32 for |x| <= 2^24, and beyond 2 (L + 1) any value clamps alike, so
// the clamp to [0, L] is taken on the float sum.
template <int BITS>
__device__ inline uint64_t codes8(const float (&v)[8], double s, double z) {
    constexpr float XMAX = 2.0f * (1 << BITS);
    constexpr float L = (float)((1 << BITS) - 1);
    const float rs = 1.0f / (float)s;
    const float zf = (float)z;
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = v[e] * rs;
        float r = rintf(x);
        if (fabsf(x - r) > 0.4999f && fabsf(x) <= XMAX) r = (float)rint((double)v[e] / s);
        c[e] = (uint32_t)fminf(fmaxf(r + zf, 0.0f), L);
    }
    if constexpr (BITS == 8) {
        return (uint64_t)(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24)) |
               ((uint64_t)(c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)) << 32);
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= c[e] << (4 * e);
        return w;
    }
}

// Store the codes of eight weights starting at weight k of row n.
template <int BITS>
__device__ inline void store_codes(uint8_t *qweight, int64_t n, int64_t K, int64_t k, uint64_t c) {
    if constexpr (BITS == 8)
        *reinterpret_cast<uint2 *>(qweight + n * K + k) = make_uint2((uint32_t)c, (uint32_t)(c >> 32));
    else
        *reinterpret_cast<uint32_t *>(qweight + n * (K / 2) + k / 2) = (uint32_t)c;
}

// Groups of 8 * SEG weights (SEG = 8, 16, 32 or 64 lanes): each SEG-lane
// segment of a wave quantizes one group; lane j of the segment owns the 8
// weights 8j .. 8j+7 (one 16- or 32-byte load, one 4-byte code store).  A wave
// takes kQuantPasses * (64 / SEG) consecutive groups (row-major order), with
// every pass's loads issued before any is used.
template <bool F32, int SEG, int BITS>
__global__ void __launch_bounds__(kQuantWaves * 64)
quantize_kernel(const void *__restrict__ w, int64_t N, int64_t K, uint8_t *__restrict__ qweight,
                uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros) {
    constexpr int GS = 8 * SEG, SPW = 64 / SEG;   // group size, segments per wave
    const int lane = threadIdx.x & 63, seg = lane / SEG, j = lane % SEG;
    const int64_t G = K / GS, total = N * G;
    const int64_t grp0 = ((int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6)) * kQuantPasses * SPW;
    float v[kQuantPasses][8];
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
        const int64_t grp = grp0 + SPW * p + seg;
        if (grp >= total) {   // past the last group: nothing loaded, nothing stored
#pragma unroll
            for (int e = 0; e < 8; ++e) v[p][e] = 0.0f;
            continue;
        }
        const int64_t n = grp / G, g = grp - n * G;
        load8<F32>(w, n * K + g * GS + 8 * j, v[p]);
    }
    // ranges of the wave's kQuantPasses * SPW groups (every lane of a segment
    // holds its group's)
    float lo[kQuantPasses], hi[kQuantPasses];
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
        // fminf/fmaxf skip NaN operands; min/max are exact in float32
        lo[p] = 0.0f;
        hi[p] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[p] = fminf(lo[p], v[p][e]);
            hi[p] = fmaxf(hi[p], v[p][e]);
        }
        for (int o = SEG / 2; o >= 1; o >>= 1) {   // within the segment
            lo[p] = fminf(lo[p], __shfl_xor(lo[p], o));
            hi[p] = fmaxf(hi[p], __shfl_xor(hi[p], o));
        }
    }
    // scale and zero once per group: lane l < kQuantPasses * SPW takes group
    // (pass l / SPW, segment l % SPW); the binary64 work is then done by one
    // lane per group instead of all SEG lanes of its segment
    constexpr int NG = kQuantPasses * SPW;
    static_assert(NG <= 64, "one lane per group");
    const int mp = lane / SPW < kQuantPasses ? lane / SPW : 0, ms = lane % SPW;
    float mlo = 0.0f, mhi = 0.0f;
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
        const float a = __shfl(lo[p], ms * SEG), b = __shfl(hi[p], ms * SEG);
        if (p == mp) {
            mlo = a;
            mhi = b;
        }
    }
    uint32_t msb = 0;
    double msd = 1.0, mz = 0.0;
    if (lane < NG) scale_zero<BITS>(mlo, mhi, msb, msd, mz);
    if (lane < NG) {
        const int64_t grp = grp0 + lane;   // = grp0 + SPW * mp + ms
        if (grp < total) {
            scales[grp] = (uint16_t)msb;
            zeros[grp] = (uint8_t)mz;
        }
    }
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
        const int64_t grp = grp0 + SPW * p + seg;
        const int src = SPW * p + seg;   // the lane holding this group's scale and zero
        const double sd = __shfl(msd, src), z = __shfl(mz, src);
        if (grp >= total) continue;
        const int64_t n = grp / G, g = grp - n * G;
        store_codes<BITS>(qweight, n, K, g * GS + 8 * j, codes8<BITS>(v[p], sd, z));
    }
}

// Other group sizes (multiples of 128 other than 128, 256, 512, up to a whole
// row): one wave per group, two passes over it (range, then codes), 512
// weights per wave step.
template <bool F32, int BITS>
__global__ void __launch_bounds__(kQuantWaves * 64)
quantize_long_kernel(const void *__restrict__ w, int64_t N, int64_t K, int64_t GS,
                     uint8_t *__restrict__ qweight, uint16_t *__restrict__ scales,
                     uint8_t *__restrict__ zeros) {
    const int lane = threadIdx.x & 63;
    const int64_t G = K / GS;
    const int64_t grp = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
    if (grp >= N * G) return;   // whole waves leave
    const int64_t n = grp / G, g = grp - n * G;
    const int64_t base = n * K + g * GS;
    float lo = 0.0f, hi = 0.0f;
    for (int64_t i = 8 * lane; i < GS; i += 512) {
        float v[8];
        load8<F32>(w, base + i, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo = fminf(lo, v[e]);
            hi = fmaxf(hi, v[e]);
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, o));
        hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    uint32_t sb;
    double sd, z;
    scale_zero<BITS>(lo, hi, sb, sd, z);
    for (int64_t i = 8 * lane; i < GS; i += 512) {
        float v[8];
        load8<F32>(w, base + i, v);
        store_codes<BITS>(qweight, n, K, g * GS + i, codes8<BITS>(v, sd, z));
    }
    if (lane == 0) {
        scales[n * G + g] = (uint16_t)sb;
        zeros[n * G + g] = (uint8_t)z;
    }
}

template <bool F32, int BITS>
int launch_quantize(const void *w, int64_t N, int64_t K, int64_t gs, uint8_t *qweight,
                    uint16_t *scales, uint8_t *zeros, hipStream_t st) {
    const int64_t groups = N * (K / gs);
    const unsigned threads = kQuantWaves * 64;
    if (gs != 64 && gs != 128 && gs != 256 && gs != 512) {
        const int64_t blocks = ceil_div(groups, kQuantWaves);
        if (blocks > 0x7fffffff) return QI4_ERR_SHAPE;
        quantize_long_kernel<F32, BITS><<<(unsigned)blocks, threads, 0, st>>>(w, N, K, gs, qweight, scales, zeros);
        return launch_status();
    }
    const int seg = (int)(gs / 8);
    const int64_t blocks = ceil_div(groups, (int64_t)kQuantWaves * kQuantPasses * (64 / seg));
    if (blocks > 0x7fffffff) return QI4_ERR_SHAPE;
    const dim3 g((unsigned)blocks);
    switch (seg) {
    case 8: quantize_kernel<F32, 8, BITS><<<g, threads, 0, st>>>(w, N, K, qweight, scales, zeros); break;
    case 16: quantize_kernel<F32, 16, BITS><<<g, threads, 0, st>>>(w, N, K, qweight, scales, zeros); break;
    case 32: quantize_kernel<F32, 32, BITS><<<g, threads, 0, st>>>(w, N, K, qweight, scales, zeros); break;
    case 64: quantize_kernel<F32, 64, BITS><<<g, threads, 0, st>>>(w, N, K, qweight, scales, zeros); break;
    default: return QI4_ERR_GROUP;
    }
    return launch_status();
}

}  // namespace
}  // namespace qi4

using namespace qi4;

namespace {

template <int BITS>
int quantize_entry(const void *w, int w_dtype, int64_t N, int64_t K, int group_size,
                   uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream) {
    if (!w || !qweight || !scales || !zeros) return QI4_ERR_NULL;
    if (w_dtype != QI4_F32 && w_dtype != QI4_BF16) return QI4_ERR_DTYPE;
    const int flags = BITS == 8 ? QI4_INT8 : 0;
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    const int64_t gs = effective_group(group_size, K);
    const int64_t es = w_dtype == QI4_F32 ? 4 : 2;
    if (!aligned(w, 16) || !aligned(qweight, BITS == 8 ? 8 : 4) || !aligned(scales, 2))
        return QI4_ERR_SHAPE;
    const int64_t G = K / gs, cb = code_bytes(N, K, flags);
    if (overlaps(w, N * K * es, qweight, cb) || overlaps(w, N * K * es, scales, N * G * 2) ||
        overlaps(w, N * K * es, zeros, N * G) || overlaps(qweight, cb, scales, N * G * 2) ||
        overlaps(qweight, cb, zeros, N * G) || overlaps(scales, N * G * 2, zeros, N * G))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    hipStream_t st = as_stream(stream);
    return w_dtype == QI4_F32 ? launch_quantize<true, BITS>(w, N, K, gs, qweight, scales, zeros, st)
                              : launch_quantize<false, BITS>(w, N, K, gs, qweight, scales, zeros, st);
}

}  // namespace

extern "C" int qi4_quantize(const void *w, int w_dtype, int64_t N, int64_t K, int group_size,
                            uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream) {
    return quantize_entry<4>(w, w_dtype, N, K, group_size, qweight, scales, zeros, stream);
}

extern "C" int qi4_quantize_int8(const void *w, int w_dtype, int64_t N, int64_t K,
                                 int group_size, uint8_t *qweight, uint16_t *scales,
                                 uint8_t *zeros, void *stream) {
    return quantize_entry<8>(w, w_dtype, N, K, group_size, qweight, scales, zeros, stream);
}
