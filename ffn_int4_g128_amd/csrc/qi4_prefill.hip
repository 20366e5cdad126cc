// Prefill (many tokens per expert) grouped GEMM of the MoE FFN on fp16 MFMA.
//
// At prefill sizes each expert's weights are reused by tens to thousands of
// tokens, so the product is a dense contraction near the MFMA/HBM ridge rather
// than a weight stream.  The design:
//  * activations are converted once per row to fp16 with an exact power-of-two
//    prescale (value = fp16 * 2^e, |fp16| < 2^14), so the contraction runs on
//    fp16 MFMA and the row factor 2^e is applied once in the epilogue;
//  * each wave dequantizes its own 64 weight rows per 128-wide group straight
//    into fp16 MFMA operands: (1024 + q) - (1024 + zero) with packed fp16 adds
//    (exact), times the binary16 scale (one rounding, relative error <= 2^-11),
//    so no per-group epilogue remains;
//  * a workgroup is 4 waves x 64 weight rows and 128 activation rows; the
//    activation tile of each group (32 KB) is copied from memory straight into
//    LDS (buffer loads with the LDS bit) in the exact order the MFMA operand
//    reads want, double-buffered, and shared by the 4 waves; two workgroups
//    share a CU so one computes while the other waits at its barrier;
//  * a device-side tile list (expert, first row) built from the expert
//    segments covers every routed expert plus the shared one, so load follows
//    the routing skew without a host round trip.
#include "qi4_gemm.h"
#include "qi4_host.h"
#include "qi4_prefill.h"

namespace qi4 {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;

// Out-of-range offsets (every buffer here is smaller than 2 GiB): kOob for a
// lane part, kOobS for a wave part; their sum never wraps around.
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kOobS = 0x7FFFFFFFu;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ inline f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 operands scale * (q - zero) of the 8 codes in one packed dword, in the
// element order of the packed layout (see qi4_dev.h).
__device__ inline uint4 dequant_f16(uint32_t d, uint32_t negz, uint32_t s2) {
    const uint32_t m = 0x000F000Fu, magic = 0x64006400u;   // fp16 1024 + q
    const f16x2 nz = __builtin_bit_cast(f16x2, negz), sc = __builtin_bit_cast(f16x2, s2);
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, (d & m) | magic) + nz) * sc);
    r.y = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, ((d >> 4) & m) | magic) + nz) * sc);
    r.z = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, ((d >> 8) & m) | magic) + nz) * sc);
    r.w = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, ((d >> 12) & m) | magic) + nz) * sc);
    return r;
}

// ---- row preparation: fp16 with a per-row power-of-two prescale ----------------

// src_kind 0: bf16 rows [rows][len]; 1: hi/lo bf16 pairs [rows][2][len].
__global__ void __launch_bounds__(256)
prep_rows_kernel(const uint16_t *__restrict__ src, int src_kind, int64_t len,
                 uint16_t *__restrict__ dst, int32_t *__restrict__ exps) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const uint16_t *s = src + row * len * (src_kind ? 2 : 1);
    auto value = [&](int64_t i) -> float {
        if (src_kind == 0) return bf16_to_f32(s[i]);
        return bf16_to_f32(s[i]) + bf16_to_f32(s[len + i]);
    };
    float mx = 0.f;
    for (int64_t i = threadIdx.x; i < len; i += 256) mx = fmaxf(mx, fabsf(value(i)));
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int E = 0;
    if (mx > 0.f) frexpf(mx, &E);          // mx in [2^(E-1), 2^E)
    const int sh = mx > 0.f ? 14 - E : 0;  // |v * 2^sh| < 2^14
    for (int64_t i = threadIdx.x; i < len; i += 256) {
        const _Float16 h = (_Float16)ldexpf(value(i), sh);
        dst[row * len + i] = __builtin_bit_cast(uint16_t, h);
    }
    if (threadIdx.x == 0) exps[row] = -sh;
}

// ---- tile planner ---------------------------------------------------------------

// One entry (problem, first slot) per 128-row tile of every nonempty routed
// expert (problem = index into the active list) and of the shared expert
// (problem = -1).  Single workgroup.
__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t *__restrict__ offsets, const int32_t *__restrict__ active, int64_t T,
            int has_shared, int2 *__restrict__ tiles, int32_t *__restrict__ count) {
    __shared__ int scan[1024];
    const int n_act = active[0];
    const int i = threadIdx.x;
    int mt = 0;
    if (i < n_act) {
        const int e = active[1 + i];
        mt = (offsets[e + 1] - offsets[e] + kPrefillBM - 1) / kPrefillBM;
    }
    scan[i] = mt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = i >= d ? scan[i - d] : 0;
        __syncthreads();
        scan[i] += v;
        __syncthreads();
    }
    const int base = scan[i] - mt;
    for (int k = 0; k < mt; ++k) tiles[base + k] = make_int2(i, k * kPrefillBM);
    const int total = scan[1023];
    const int sh_tiles = has_shared ? (int)((T + kPrefillBM - 1) / kPrefillBM) : 0;
    for (int k = i; k < sh_tiles; k += 1024) tiles[total + k] = make_int2(-1, k * kPrefillBM);
    if (i == 0) *count = total + sh_tiles;
}

// ---- the grouped GEMM ----------------------------------------------------------------

constexpr int kWaves = 4;
constexpr int kNB = 4;                         // 16-row weight tiles per wave
constexpr int kMS = kPrefillBM / 16;           // 16-row activation subtiles per workgroup
constexpr int kABlock = 1024;                  // one MFMA operand fragment of a wave
constexpr int kABytes = kMS * 4 * kABlock;     // activation tile of one group: 32 KB

template <int EPI>
__global__ void __launch_bounds__(kWaves * 64, 2)
prefill_kernel(const PrefillArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kABytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15, j = lane >> 4;

    const int tix = blockIdx.y;
    if (tix >= *args.tile_count) return;
    const int2 te = args.tiles[tix];
    const uint8_t *w;
    int64_t row0, n, src0 = 0;
    const int32_t *gather = nullptr;
    if (te.x >= 0) {
        const int e = args.active[1 + te.x];
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
    const int64_t m0 = te.y;

    const PackedLayout L(args.N, args.K, args.flags);
    const int64_t nt = L.nt, G = L.G;
    const int64_t tile0 = (int64_t)blockIdx.x * (kWaves * kNB) + wave * kNB;
    const __amdgpu_buffer_rsrc_t wr = rsrc(w, (uint32_t)L.bytes);
    const __amdgpu_buffer_rsrc_t ar = rsrc(args.a16, (uint32_t)(args.a_rows * args.K * 2));

    // Weight offsets: the lane part is the same for every tile and group; the
    // tile and group part is wave-uniform and goes in soffset (scalar registers).
    const uint32_t vc = (uint32_t)lane * 16u, vs = (uint32_t)r16 * 2u, vz = (uint32_t)(r16 >> 1);
    const int nt_here = (int)(nt - tile0 < kNB ? (nt - tile0 > 0 ? nt - tile0 : 0) : kNB);
    const int zshift = 4 * (r16 & 1);

    // Activation rows this lane copies into LDS: wave w fills the operand
    // fragments of 16-row subtiles 2w and 2w+1 (four 32-wide k steps each).
    uint32_t aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t slot = m0 + 16 * (2 * wave + h) + r16;
        const bool ok = slot < n;
        const int64_t slot_c = ok ? slot : 0;
        const int64_t src = gather ? (int64_t)(gather[row0 + slot_c] / args.top_k) : src0 + slot_c;
        aoff[h] = ok ? (uint32_t)((src * args.K + 8 * j) * 2) : kOob;
    }

    // Past the last group every lane loads from an out-of-range offset (a
    // select, not a sum, so an invalid row's offset cannot wrap around).
    auto fill = [&](uint8_t *buf, int g) {
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)g * 256u : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int h = i >> 2, s = i & 3;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ar, (__attribute__((address_space(3))) void *)(buf + ((2 * wave + h) * 4 + s) * kABlock),
                16, in ? aoff[h] + 64u * s : kOob, so, 0, 0);
        }
    };
    struct WStage {
        uint4 cw[kNB];
        uint32_t sc[kNB], zb[kNB];
    };
    auto load_w = [&](WStage &q, int g) {
        const bool in = g < G;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const bool ok = in && nb < nt_here;
            const int64_t tg = (tile0 + nb) * G + g;
            const uint32_t oc = ok ? (uint32_t)(tg * 1024) : kOobS;
            const uint32_t os = ok ? (uint32_t)(L.scales_off + tg * 32) : kOobS;
            const uint32_t oz = ok ? (uint32_t)(L.zeros_off + tg * 8) : kOobS;
            q.cw[nb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, vc, oc, 0));
            q.sc[nb] = __builtin_amdgcn_raw_buffer_load_b16(wr, vs, os, 0);
            q.zb[nb] = __builtin_amdgcn_raw_buffer_load_b8(wr, vz, oz, 0);
        }
    };

    f32x4 acc[kMS][kNB];
#pragma unroll
    for (int m = 0; m < kMS; ++m)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 16-row activation subtiles of this tile that hold rows (uniform): the
    // MFMAs of empty subtiles are skipped, so a small expert costs only its rows.
    const int m_used = (int)((n - m0 + 15) / 16 < kMS ? (n - m0 + 15) / 16 : kMS);

    auto compute = [&](const WStage &q, const uint8_t *buf) {
        uint32_t negz[kNB], s2[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const uint32_t z = (q.zb[nb] >> zshift) & 15u;
            // fp16 -(1024 + z) in both halves; scale in both halves
            const uint32_t nz = __builtin_bit_cast(uint16_t, (_Float16)(-(1024.0f + (float)z)));
            negz[nb] = nz * 0x00010001u;
            s2[nb] = (q.sc[nb] & 0xFFFFu) * 0x00010001u;
        }
        // Operand fragments in (k step, subtile) order through a 2-deep ring, so
        // each LDS read is issued one MFMA batch before it is needed.
        auto rd = [&](int i) {
            return *reinterpret_cast<const f16x8 *>(buf + ((i & 7) * 4 + (i >> 3)) * kABlock + lane * 16);
        };
        f16x8 a[2];
        a[0] = rd(0);
        f16x8 b[kNB];
#pragma unroll
        for (int i = 0; i < 4 * kMS; ++i) {
            const int s = i >> 3, m = i & 7;
            if (m == 0) {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const uint32_t d = s == 0 ? q.cw[nb].x : s == 1 ? q.cw[nb].y : s == 2 ? q.cw[nb].z : q.cw[nb].w;
                    b[nb] = __builtin_bit_cast(f16x8, dequant_f16(d, negz[nb], s2[nb]));
                }
            }
            if (i + 1 < 4 * kMS) a[(i + 1) & 1] = rd(i + 1);
            if (m < m_used) {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = mfma16x16x32_f16(a[i & 1], b[nb], acc[m][nb]);
            }
        }
    };

    // Pipeline: at step g the activation tile of group g + 1 is copied into the
    // other LDS buffer and its weights are requested while group g is
    // multiplied.  At the top of a step this wave waits for its requests (vmcnt
    // 0) and the barrier makes every wave's LDS copies visible and frees the
    // buffer the next copies refill.  The second workgroup on the CU computes
    // while this one waits.
    WStage wst[2];
    fill(lds_a[0], 0);
    load_w(wst[0], 0);
    for (int g = 0; g < G; g += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (g + u >= G) break;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            fill(lds_a[(u + 1) & 1], g + u + 1);
            load_w(wst[(u + 1) & 1], g + u + 1);
            compute(wst[u], lds_a[u]);
        }
    }
    // the copies requested past the last group (out of range, zero-filled)
    // must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: row factor 2^e, SiLU(gate) * up or the plain output ----
#pragma unroll
    for (int m = 0; m < kMS; ++m) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t slot = m0 + 16 * m + 4 * j + v;
            if (slot >= n) continue;
            const int64_t src = gather ? (int64_t)(gather[row0 + slot] / args.top_k) : src0 + slot;
            const int e = args.a_exp[src];
            const int64_t dst = row0 + slot;
            if constexpr (EPI == QI4_EPI_SILU_MUL) {
#pragma unroll
                for (int p = 0; p < kNB / 2; ++p) {
                    const int64_t tile = tile0 + 2 * p;
                    const int64_t oc = (tile >> 1) * 16 + r16;
                    if (tile >= nt || oc >= args.n_out) continue;
                    const float gv = ldexpf(acc[m][2 * p][v], e), uv = ldexpf(acc[m][2 * p + 1][v], e);
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    const uint32_t hi = f32_to_bf16_rne(hv);
                    const uint32_t lo = f32_to_bf16_rne(hv - bf16_to_f32(hi));
                    uint16_t *o = static_cast<uint16_t *>(args.out);
                    o[(dst * 2) * args.ldo + oc] = (uint16_t)hi;
                    o[(dst * 2 + 1) * args.ldo + oc] = (uint16_t)lo;
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    const int64_t tile = tile0 + nb;
                    if (tile >= nt) continue;
                    const int64_t oc = tile_row(tile, r16, args.N, args.flags);
                    if (oc < 0 || oc >= args.n_out) continue;
                    static_cast<float *>(args.out)[dst * args.ldo + oc] = ldexpf(acc[m][nb][v], e);
                }
            }
        }
    }
}

}  // namespace

int launch_prep_rows(const void *src, int src_kind, int64_t rows, int64_t len, uint16_t *dst,
                     int32_t *exps, hipStream_t st) {
    if (rows <= 0) return QI4_OK;
    if (rows > 0x7fffffff) return QI4_ERR_SHAPE;
    prep_rows_kernel<<<(unsigned)rows, 256, 0, st>>>(static_cast<const uint16_t *>(src), src_kind,
                                                     len, dst, exps);
    return launch_status();
}

int launch_plan(const int32_t *offsets, const int32_t *active, int64_t T, int has_shared,
                int2 *tiles, int32_t *count, hipStream_t st) {
    plan_kernel<<<1, 1024, 0, st>>>(offsets, active, T, has_shared, tiles, count);
    return launch_status();
}

int64_t prefill_max_tiles(int64_t T, int top_k, int64_t E, int has_shared) {
    const int64_t P = T * top_k;
    const int64_t act = P < E ? P : E;
    return P / kPrefillBM + act + (has_shared ? (T + kPrefillBM - 1) / kPrefillBM : 0) + 1;
}

int launch_prefill(const PrefillArgs &a, int64_t max_tiles, hipStream_t st) {
    const int64_t nt = num_tiles(a.N, a.flags);
    const int64_t gx = ceil_div(nt, kWaves * kNB);
    if (gx > 0x7fffffff || max_tiles > 65535) return QI4_ERR_SHAPE;
    dim3 grid((unsigned)gx, (unsigned)max_tiles);
    if (a.epi == QI4_EPI_SILU_MUL)
        prefill_kernel<QI4_EPI_SILU_MUL><<<grid, kWaves * 64, 0, st>>>(a);
    else
        prefill_kernel<QI4_EPI_NONE><<<grid, kWaves * 64, 0, st>>>(a);
    return launch_status();
}

}  // namespace qi4
