// Routed mixture-of-experts FFN on int4-g128 experts: router top-k, the
// token-by-expert permutation, the grouped expert GEMMs and the combine.
//
// The pages describe MoE layers whose experts hold most of the parameters while
// each token activates only a few of them (FastLLM notes, wmrh.cn, part 1), the
// number of routed experts per token as a knob (--moe_experts) and a shared
// expert that always runs (--cuda_se) (fastllm README, "other parameters").
// Here the routed experts a batch touches are found on the device (sort), and
// one launch per projection covers all of them: grid.y enumerates the touched
// experts, then the shared one split by M tiles of slots, grid.x the 16-row
// tiles of each expert's matrix.
// Only touched experts' weights are read.
#include <limits.h>

#include <mutex>

#include <type_traits>

#include "qi4_gemm.h"
#include "qi4_host.h"
#include "qi4_prefill.h"
#include "qi4_rows.h"

namespace qi4 {
namespace {

constexpr int kRouteWaves = 4;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// ---- cross-lane helpers ----------------------------------------------------------------

// Cross-lane moves without the LDS crossbar: DPP inside rows of 16 lanes, and
// the permlane swaps between rows and between the wave's halves.
// Lanes without a source, and lanes of rows left out by ROWS, read 0.
template <int CTRL, int ROWS = 0xF>
__device__ inline uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15 - i within 16
constexpr int kDppShr1 = 0x111;       // lane i <- lane i - 1 within 16 (row_shr:1)
constexpr int kDppBcast15 = 0x142;    // row r <- lane 15 of row r - 1
constexpr int kDppBcast31 = 0x143;    // rows 2, 3 <- lane 31

// Inclusive prefix sum over the wave's lanes (every lane active).
__device__ inline int wave_incl_scan(int x) {
    x += (int)dpp_u32<kDppShr1>((uint32_t)x);
    x += (int)dpp_u32<kDppShr1 + 1>((uint32_t)x);
    x += (int)dpp_u32<kDppShr1 + 3>((uint32_t)x);
    x += (int)dpp_u32<kDppShr1 + 7>((uint32_t)x);   // rows of 16 scanned
    x += (int)dpp_u32<kDppBcast15, 0xA>((uint32_t)x);   // rows 1, 3 add their left row
    x += (int)dpp_u32<kDppBcast31, 0xC>((uint32_t)x);   // rows 2, 3 add rows 0-1
    return x;
}

// (value, index) pairs: the larger value wins, equal values go to the lower index.
__device__ inline bool beats(float av, int ai, float bv, int bi) {
    return (av > bv) | ((av == bv) & (ai < bi));   // no short-circuit: no branches
}
template <int CTRL>
__device__ inline void argmax_step(float &v, int &i) {
    const float ov = __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
    const int oi = (int)dpp_u32<CTRL>((uint32_t)i);
    if (beats(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}
// Both results of a swap hold, lane by lane, the two partners of a pairing
// (lane with the other row / half); keep the better one.
__device__ inline void argmax_swap(float &v, int &i, bool rows16) {
    const uint32_t uv = __float_as_uint(v), ui = (uint32_t)i;
    uint32_t av, bv, ai, bi;
    if (rows16) {
        const auto sv = __builtin_amdgcn_permlane16_swap(uv, uv, false, false);
        const auto si = __builtin_amdgcn_permlane16_swap(ui, ui, false, false);
        av = sv[0]; bv = sv[1]; ai = si[0]; bi = si[1];
    } else {
        const auto sv = __builtin_amdgcn_permlane32_swap(uv, uv, false, false);
        const auto si = __builtin_amdgcn_permlane32_swap(ui, ui, false, false);
        av = sv[0]; bv = sv[1]; ai = si[0]; bi = si[1];
    }
    const bool a_wins = beats(__uint_as_float(av), (int)ai, __uint_as_float(bv), (int)bi);
    v = __uint_as_float(a_wins ? av : bv);
    i = (int)(a_wins ? ai : bi);
}
// Argmax over the whole wave; every lane ends with the winner.  The wave must
// be fully active.
__device__ inline void wave_argmax(float &v, int &i) {
    argmax_step<kDppXor1>(v, i);
    argmax_step<kDppXor2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    argmax_swap(v, i, true);
    argmax_swap(v, i, false);
}
// Sum over the whole wave in a fixed pattern; every lane ends with the same bits.
__device__ inline float wave_sum(float x) {
    x += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(x)));
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// ---- router logits: a bf16 MFMA GEMM, hidden -> experts -------------------------

constexpr int kRouterWaves = 16;   // waves of a workgroup; they split K

// logits[t][e] = sum_k x[t][k] * w[e][k] with x bf16 [T][H], w bf16 [E][H] and
// float32 accumulation.  A workgroup owns 16 experts x 16 MT tokens; its waves
// take consecutive 32-wide k steps, CH at a time with all their loads issued
// before the first MFMA (the k range of a wave is a few steps, so this is most
// of its memory parallelism), and their partial sums are added in LDS in wave
// order, so the result does not depend on timing.  Out-of-range rows (tokens
// past T, experts past E) and steps past the wave's range load zeros.
template <int MT>
__global__ void __launch_bounds__(kRouterWaves * 64)
router_gemm_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t T,
                   int64_t H, int E, float *__restrict__ logits) {
    constexpr int CH = MT == 4 ? 4 : 8;
    __shared__ float red[kRouterWaves * MT * 256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, j = lane >> 4;
    const int64_t e0 = (int64_t)blockIdx.x * 16, t0 = (int64_t)blockIdx.y * (16 * MT);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(T * H * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)(E * H * 2));
    const int nks = (int)(H / 32);
    const int kb = nks * wave / kRouterWaves, ke = nks * (wave + 1) / kRouterWaves;
    // lane parts of the offsets: the operand row and its 8-element k chunk
    const uint32_t wo = e0 + r16 < E ? (uint32_t)(((e0 + r16) * H + 8 * j) * 2) : kOob;
    uint32_t xo[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t t = t0 + 16 * m + r16;
        xo[m] = t < T ? (uint32_t)((t * H + 8 * j) * 2) : kOob;
    }
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = zero4;
    for (int k0 = kb; k0 < ke; k0 += CH) {
        bf16x8 bv[CH], av[CH][MT];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            // 32 bf16 per k step (wave-uniform); steps past the range load zeros
            const uint32_t ko = k0 + c < ke ? (uint32_t)(k0 + c) * 64u : kOobS;
            bv[c] = as_bf16x8(buf_b128(wr, wo, ko));
#pragma unroll
            for (int m = 0; m < MT; ++m) av[c][m] = as_bf16x8(buf_b128(xr, xo[m], ko));
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = mfma16x16x32(av[c][m], bv[c], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wave * MT + m) * 4 + v) * 64 + lane] = acc[m][v];
    __syncthreads();
    // one output per thread: tile m, register v, lane l -> token 4 (l >> 4) + v, expert l & 15
    for (int it = threadIdx.x; it < MT * 256; it += kRouterWaves * 64) {
        const int m = it >> 8, v = (it >> 6) & 3, l = it & 63;
        float sum = 0.f;
        for (int ww = 0; ww < kRouterWaves; ++ww) sum += red[((ww * MT + m) * 4 + v) * 64 + l];
        const int64_t t = t0 + 16 * m + 4 * (l >> 4) + v, e = e0 + (l & 15);
        if (t < T && e < E) logits[t * E + e] = sum;
    }
}

// Large batches: a workgroup owns 16 NE experts x 16 MT tokens (64 x 32 for
// T >= kRouterWideMinT), so each token row is read by E / (16 NE) workgroups
// instead of E / 16; its kRouterWideWaves waves split K and add their partial
// sums in LDS in wave order (deterministic, as above); 64 KiB of LDS for the
// partial sums.  T = 2048, E = 256, H = 7168 on MI355X: 79 -> 50 us for the
// projection and top-k (64 x 64 tiles: 75 us, 16 x 128: 73 us, 4 waves: 52 us).
constexpr int kRouterWideWaves = 8;
constexpr int64_t kRouterWideMinT = 256;
template <int MT, int NE>
__global__ void __launch_bounds__(kRouterWideWaves * 64)
router_gemm_wide_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t T,
                        int64_t H, int E, float *__restrict__ logits) {
    constexpr int CH = 2;
    __shared__ float red[kRouterWideWaves * MT * NE * 256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, j = lane >> 4;
    const int64_t e0 = (int64_t)blockIdx.x * 16 * NE, t0 = (int64_t)blockIdx.y * (16 * MT);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(T * H * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)(E * H * 2));
    const int nks = (int)(H / 32);
    const int kb = nks * wave / kRouterWideWaves, ke = nks * (wave + 1) / kRouterWideWaves;
    uint32_t wo[NE], xo[MT];
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int64_t e = e0 + 16 * n + r16;
        wo[n] = e < E ? (uint32_t)((e * H + 8 * j) * 2) : kOob;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t t = t0 + 16 * m + r16;
        xo[m] = t < T ? (uint32_t)((t * H + 8 * j) * 2) : kOob;
    }
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[MT][NE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NE; ++n) acc[m][n] = zero4;
    for (int k0 = kb; k0 < ke; k0 += CH) {
        bf16x8 bv[CH][NE], av[CH][MT];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const uint32_t ko = k0 + c < ke ? (uint32_t)(k0 + c) * 64u : kOobS;
#pragma unroll
            for (int n = 0; n < NE; ++n) bv[c][n] = as_bf16x8(buf_b128(wr, wo[n], ko));
#pragma unroll
            for (int m = 0; m < MT; ++m) av[c][m] = as_bf16x8(buf_b128(xr, xo[m], ko));
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NE; ++n) acc[m][n] = mfma16x16x32(av[c][m], bv[c][n], acc[m][n]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NE; ++n)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[(((wave * MT + m) * NE + n) * 4 + v) * 64 + lane] = acc[m][n][v];
    __syncthreads();
    // one output per thread: tile (m, n), register v, lane l -> token 16 m +
    // 4 (l >> 4) + v, expert 16 n + (l & 15)
    for (int it = threadIdx.x; it < MT * NE * 256; it += kRouterWideWaves * 64) {
        const int mn = it >> 8, v = (it >> 6) & 3, l = it & 63;
        float sum = 0.f;
        for (int ww = 0; ww < kRouterWideWaves; ++ww)
            sum += red[((ww * MT * NE + mn) * 4 + v) * 64 + l];
        const int m = mn / NE, n = mn % NE;
        const int64_t t = t0 + 16 * m + 4 * (l >> 4) + v, e = e0 + 16 * n + (l & 15);
        if (t < T && e < E) logits[t * E + e] = sum;
    }
}

// Router logits of decode batches (T <= kGemvMaxT): one workgroup per (expert,
// group of up to four tokens), its four waves each taking a quarter of the
// expert's row in 16-byte chunks (8 bf16, all loads of a lane issued before
// they are used), float32 products summed in k order per lane, then a
// fixed-pattern wave sum and the four waves added in order: deterministic, and
// 256 experts keep 1024 waves or more streaming the matrix where the MFMA
// kernel above has 16 workgroups.  Later token groups read the row from cache.
constexpr int kGemvTokens = 4;
constexpr int64_t kGemvMaxT = 64;
constexpr int kGemvChunks = 8;   // chunks of 8 values per lane held in flight

template <int TT>
__global__ void __launch_bounds__(256)
router_gemv_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t T,
                   int64_t H, int E, float *__restrict__ logits) {
    __shared__ float part[4][TT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * TT;
    const int nt = (int)(T - t0 < TT ? T - t0 : TT);   // tokens of this group
    x += t0 * H;
    logits += t0 * E;
    const int64_t nch = H / 8, per = (nch + 3) / 4;
    const int64_t c0 = wave * per, c1 = c0 + per < nch ? c0 + per : nch;
    const uint16_t *wr = w + (int64_t)e * H;
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
    auto dot8 = [](uint4 a, uint4 b, float s) {
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(bf16_to_f32(av[i] & 0xFFFFu), bf16_to_f32(bv[i] & 0xFFFFu), s);
            s = fmaf(bf16_to_f32(av[i] >> 16), bf16_to_f32(bv[i] >> 16), s);
        }
        return s;
    };
    for (int64_t c = c0 + lane; c < c1; c += 64 * kGemvChunks) {
        uint4 wv[kGemvChunks], xv[kGemvChunks][TT];
#pragma unroll
        for (int u = 0; u < kGemvChunks; ++u) {
            const int64_t cu = c + 64 * u;
            const bool ok = cu < c1;
            wv[u] = ok ? *reinterpret_cast<const uint4 *>(wr + 8 * cu) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < TT; ++t)
                xv[u][t] = ok && t < nt ? *reinterpret_cast<const uint4 *>(x + t * H + 8 * cu)
                                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kGemvChunks; ++u)
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[t] = dot8(wv[u], xv[u][t], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) part[wave][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = threadIdx.x;
        logits[(int64_t)t * E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    }
}

int launch_router_gemm(const uint16_t *x, const uint16_t *w, int64_t T, int64_t H, int E,
                       float *logits, hipStream_t st) {
    if (T <= kGemvMaxT) {
        const dim3 g((unsigned)E, (unsigned)ceil_div(T, kGemvTokens));
        if (T == 1) router_gemv_kernel<1><<<g, 256, 0, st>>>(x, w, T, H, E, logits);
        else if (T == 2) router_gemv_kernel<2><<<g, 256, 0, st>>>(x, w, T, H, E, logits);
        else if (T == 3) router_gemv_kernel<3><<<g, 256, 0, st>>>(x, w, T, H, E, logits);
        else router_gemv_kernel<4><<<g, 256, 0, st>>>(x, w, T, H, E, logits);
        return launch_status();
    }
    if (T >= kRouterWideMinT) {
        const int64_t gy = ceil_div(T, 16 * 2);
        if (gy > 65535) return QI4_ERR_SHAPE;
        const dim3 g((unsigned)ceil_div(E, 16 * 4), (unsigned)gy);
        router_gemm_wide_kernel<2, 4><<<g, kRouterWideWaves * 64, 0, st>>>(x, w, T, H, E, logits);
        return launch_status();
    }
    const int MT = T <= 16 ? 1 : T <= 32 ? 2 : 4;
    const int64_t gy = ceil_div(T, 16 * MT);
    if (gy > 65535) return QI4_ERR_SHAPE;
    const dim3 g((unsigned)ceil_div(E, 16), (unsigned)gy);
    const unsigned tb = kRouterWaves * 64;
    if (MT == 1) router_gemm_kernel<1><<<g, tb, 0, st>>>(x, w, T, H, E, logits);
    else if (MT == 2) router_gemm_kernel<2><<<g, tb, 0, st>>>(x, w, T, H, E, logits);
    else router_gemm_kernel<4><<<g, tb, 0, st>>>(x, w, T, H, E, logits);
    return launch_status();
}

// ---- router: one wave per token --------------------------------------------------

// One token on one (fully active) wave: k rounds of a wave argmax over the
// logits not taken yet, lane j keeping the j-th pick, then the softmax over the
// k picks.  Writes ids and weights of token t (and the ids to ids_copy if given).
template <int VPL>
__device__ inline void route_token(const float *__restrict__ logits, int64_t t, int E, int k,
                                   int lane, int32_t *__restrict__ ids, float *__restrict__ wts,
                                   int32_t *ids_copy) {
    float v[VPL];
    bool taken[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = i * 64 + lane;
        float x = e < E ? logits[t * E + e] : -INFINITY;
        if (x != x) x = -INFINITY;   // NaN ranks like -inf
        v[i] = x;
        taken[i] = e >= E;
    }
    float myv = -INFINITY;
    int myi = 0;
    for (int jj = 0; jj < k; ++jj) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = i * 64 + lane;
            if ((!taken[i]) & beats(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
        wave_argmax(bv, bi);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (bi == i * 64 + lane) taken[i] = true;
        if (lane == jj) {
            myv = bv;
            myi = bi;
        }
    }
    const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__float_as_uint(myv)));
    const float ex = lane < k ? expf(myv - l0) : 0.f;
    const float sum = wave_sum(ex);
    if (lane < k) {
        ids[t * k + lane] = myi;
        wts[t * k + lane] = ex / sum;
        if (ids_copy) ids_copy[t * k + lane] = myi;
    }
}

// The layer input's rows as fp16 with per-row exponents (prep_row), done by
// the workgroups of a routing launch past its routing ones, so the layer call
// needs no launch of its own for them.  x == nullptr: none.
struct RowPrep {
    const uint16_t *x;
    int64_t len;
    uint16_t *x16;
    int32_t *ex;
};

// One wave per token; workgroups from route_blocks on prepare row
// blockIdx.x - route_blocks of the layer input.
template <int VPL>
__global__ void __launch_bounds__(kRouteWaves * 64)
route_kernel(const float *__restrict__ logits, int64_t T, int E, int k,
             int32_t *__restrict__ ids, float *__restrict__ wts, int64_t route_blocks,
             RowPrep prep) {
    if (blockIdx.x >= route_blocks) {
        __shared__ float wmax[kRouteWaves];
        prep_row<kRouteWaves * 64>(prep.x, 0, prep.len, blockIdx.x - route_blocks, prep.x16,
                                   prep.ex, wmax);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T) return;   // whole waves leave: the rest stay fully active
    route_token<VPL>(logits, t, E, k, lane, ids, wts, nullptr);
}

// ---- stable counting sort of the (token, slot) pairs by expert ----------------------

// Lanes of this wave holding the same expert id (valid lanes only).
__device__ inline uint64_t match_expert(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// The sort on one workgroup of W waves (wave w takes the w-th chunk of the
// pairs), with its LDS tables passed in.  ids may point to global or LDS memory.
template <int W>
__device__ inline void sort_body(const int32_t *ids, int64_t npairs, int E, int nbits,
                                 int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ offsets,
                                 int32_t *__restrict__ pair_to_sorted, int32_t *__restrict__ active,
                                 int (&cnt)[W][kMaxExperts], int *off_s, int *tot_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    int64_t chunk = (npairs + W - 1) / W;
    chunk = (chunk + 63) & ~int64_t(63);
    const int64_t pb = wave * chunk;
    const int64_t pe = pb + chunk < npairs ? pb + chunk : npairs;

    for (int i = threadIdx.x; i < W * E; i += blockDim.x) cnt[i / E][i % E] = 0;
    __syncthreads();

    // histogram of this wave's chunk (ids outside [0, E) are left out)
    for (int64_t pos = pb; pos < pe; pos += 64) {
        const int64_t i = pos + lane;
        int e = i < pe ? ids[i] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        const uint64_t m = match_expert(e, valid, nbits);
        if (valid && (__ffsll((unsigned long long)m) - 1) == lane) cnt[wave][e] += __popcll(m);
    }
    __syncthreads();

    // per expert: exclusive prefix over the waves, and the total
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int w = 0; w < W; ++w) {
            const int c = cnt[w][e];
            cnt[w][e] = run;
            run += c;
        }
        tot_s[e] = run;
    }
    __syncthreads();

    // exclusive scan over the experts (wave 0), plus the list of nonempty experts
    if (wave == 0) {
        const int per = (E + 63) / 64;
        const int e0 = lane * per;
        int s = 0, a = 0;
        for (int e = e0; e < e0 + per && e < E; ++e) {
            s += tot_s[e];
            a += tot_s[e] > 0;
        }
        const int ps = wave_incl_scan(s), pa = wave_incl_scan(a);   // across lanes
        int run = ps - s, arun = pa - a;
        for (int e = e0; e < e0 + per && e < E; ++e) {
            off_s[e] = run;
            offsets[e] = run;
            if (tot_s[e] > 0) {
                if (active) active[1 + arun] = e;
                ++arun;
            }
            run += tot_s[e];
        }
        if (lane == 63) {
            off_s[E] = ps;
            offsets[E] = ps;
            if (active) active[0] = pa;
        }
    }
    __syncthreads();

    // scatter, stable within each expert: waves in pair order, lanes in pair order
    for (int64_t pos = pb; pos < pe; pos += 64) {
        const int64_t i = pos + lane;
        int e = i < pe ? ids[i] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (i < pe && !valid) pair_to_sorted[i] = -1;   // dropped: out-of-range id
        if (!valid) e = 0;
        const uint64_t m = match_expert(e, valid, nbits);
        int base = 0;
        if (valid) base = off_s[e] + cnt[wave][e];
        const int rank = __popcll(m & lt_mask);
        if (valid) {
            const int dst = base + rank;
            sorted_pairs[dst] = (int32_t)i;
            pair_to_sorted[i] = dst;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && (__ffsll((unsigned long long)m) - 1) == lane) cnt[wave][e] = base - off_s[e] + __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

template <int W>
__global__ void __launch_bounds__(W * 64)
sort_kernel(const int32_t *__restrict__ ids, int64_t npairs, int E, int nbits,
            int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ offsets,
            int32_t *__restrict__ pair_to_sorted, int32_t *__restrict__ active) {
    __shared__ int cnt[W][kMaxExperts];
    __shared__ int off_s[kMaxExperts + 1];
    __shared__ int tot_s[kMaxExperts];
    sort_body<W>(ids, npairs, E, nbits, sorted_pairs, offsets, pair_to_sorted, active, cnt, off_s,
                 tot_s);
}

// Decode batches (T <= 16 tokens): routing and sort in one workgroup of 16
// waves, wave t routing token t, the ids passed through LDS.  Saves one launch
// (measured 1.4 us of a 72 us step at T = 1); from two tokens per wave on, the
// serialized routing eats the gain.
// W waves (4 up to four tokens, else 16): fewer waves take less to zero the
// tables and to pass the barriers.
constexpr int kFusedWaves = 16;
constexpr int kFusedPairs = kFusedWaves * kMaxTopK;
// Workgroups 1 .. T (when prep.x is given) prepare the layer input's rows.
template <int VPL, int W>
__global__ void __launch_bounds__(W * 64)
route_sort_kernel(const float *__restrict__ logits, int64_t T, int E, int k, int nbits,
                  int32_t *__restrict__ ids, float *__restrict__ wts,
                  int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ offsets,
                  int32_t *__restrict__ pair_to_sorted, int32_t *__restrict__ active,
                  RowPrep prep) {
    if (blockIdx.x > 0) {
        __shared__ float wmax[W];
        prep_row<W * 64>(prep.x, 0, prep.len, blockIdx.x - 1, prep.x16, prep.ex, wmax);
        return;
    }
    __shared__ int cnt[W][kMaxExperts];
    __shared__ int off_s[kMaxExperts + 1];
    __shared__ int tot_s[kMaxExperts];
    __shared__ int32_t ids_s[W * kMaxTopK];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < T)   // whole waves: fully active
        route_token<VPL>(logits, wave, E, k, lane, ids, wts, ids_s);
    __syncthreads();
    sort_body<W>(ids_s, T * k, E, nbits, sorted_pairs, offsets, pair_to_sorted, active, cnt, off_s,
                 tot_s);
}

// ---- combine: fixed order, slots then the shared expert -------------------------------

// 16 bytes loaded with the non-temporal hint (data read once).
__device__ inline uint4 load_b128_nt(const void *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// The slot rows of a token are loaded eight at a time before any is added, so
// their latencies overlap, with the non-temporal hint (each is read once; the
// T = 2048 combine 110 -> 86 us; the same hint on the row conversions and the
// quantizer's input was no faster); the additions keep the order j = 0 ..
// k-1, then the shared expert.
__global__ void __launch_bounds__(256)
combine_kernel(const float *__restrict__ y, const float *__restrict__ wts,
               const int32_t *__restrict__ p2s, int64_t T, int k, int64_t H, int has_shared,
               uint16_t *__restrict__ out) {
    constexpr int kBatch = 8;
    const int64_t t = blockIdx.y;
    const int64_t n4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (n4 >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += kBatch) {
        float p[kBatch];
        float4 v[kBatch];
        bool use[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int j = j0 + b;
            const int64_t r = j < k ? p2s[t * k + j] : -1;   // -1: dropped slot
            use[b] = r >= 0;
            p[b] = use[b] ? wts[t * k + j] : 0.f;
            v[b] = use[b] ? __builtin_bit_cast(float4, load_b128_nt(y + r * H + n4))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (!use[b]) continue;
            acc.x += p[b] * v[b].x;
            acc.y += p[b] * v[b].y;
            acc.z += p[b] * v[b].z;
            acc.w += p[b] * v[b].w;
        }
    }
    if (has_shared) {
        const float4 v = __builtin_bit_cast(float4, load_b128_nt(y + (T * k + t) * H + n4));
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2 *>(out + t * H + n4) = o;
}

// The routed pairs whose expert runs elsewhere get the id -1: the permutation
// leaves them out and the combine skips them, so this device computes only its
// own experts' share of the layer and reads only their weights.
__global__ void __launch_bounds__(256)
mask_ids_kernel(const int32_t *__restrict__ ids, int64_t npairs, const uint8_t *__restrict__ here,
                int E, int32_t *__restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < npairs; i += (int64_t)gridDim.x * 256) {
        const int32_t e = ids[i];
        out[i] = (e >= 0 && e < E && here[e]) ? e : -1;
    }
}

// ---- host helpers ------------------------------------------------------------------------

int check_desc(const qi4_moe_desc *d) {
    if (!d) return QI4_ERR_NULL;
    // one group size for both projections: 64, a multiple of 128 dividing both
    // hidden and inter, or 0 (one group per row of each matrix)
    if (d->group_size < 0 || (d->group_size != 0 && d->group_size != 64 &&
                              (d->group_size < 128 || d->group_size % 128 != 0)))
        return QI4_ERR_GROUP;
    if ((d->flags & ~QI4_INT8) || (d->has_shared != 0 && d->has_shared != 1))
        return QI4_ERR_UNSUPPORTED;
    if (d->num_experts < 1 || d->num_experts > kMaxExperts) return QI4_ERR_SHAPE;
    if (d->hidden < 128 || d->hidden % 128 || d->inter < 128 || d->inter % 128) return QI4_ERR_SHAPE;
    if (d->hidden > (1 << 20) || d->inter > (1 << 20)) return QI4_ERR_SHAPE;
    if (d->group_size > 64 && (d->hidden % d->group_size || d->inter % d->group_size))
        return QI4_ERR_SHAPE;
    if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->num_experts) return QI4_ERR_SHAPE;
    return QI4_OK;
}

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Group sizes of the gate/up (groups along hidden) and down (along inter) matrices.
inline int gs_gate_up(const qi4_moe_desc *d) { return (int)effective_group(d->group_size, d->hidden); }
inline int gs_down(const qi4_moe_desc *d) { return (int)effective_group(d->group_size, d->inter); }
// Pack flags of the two matrices (QI4_INT8: 8-bit experts, stored as two 4-bit
// planes of twice the width, each block reading one activation block).
inline int gate_up_flags(const qi4_moe_desc *d) { return QI4_PACK_GATEUP | (d->flags & QI4_INT8); }
inline int down_flags(const qi4_moe_desc *d) { return d->flags & QI4_INT8; }
inline int a_shift_of(const qi4_moe_desc *d) { return (d->flags & QI4_INT8) ? 1 : 0; }
inline int64_t gate_up_bytes(const qi4_moe_desc *d) {
    return PackedLayout(2 * d->inter, packed_k(d->hidden, d->flags), gate_up_flags(d),
                        gs_gate_up(d)).bytes;
}
inline int64_t down_bytes(const qi4_moe_desc *d) {
    return PackedLayout(d->hidden, packed_k(d->inter, d->flags), down_flags(d), gs_down(d)).bytes;
}

// Batches of at least this many tokens run the prefill GEMM (fp16 MFMA on
// LDS-staged activation tiles); smaller ones the weight-streaming decode GEMM.
constexpr int64_t kPrefillMinT = 128;

// Capacity of the prefill deferred list: the larger of the two projections.
int64_t prefill_deferred_capacity(const qi4_moe_desc *d, const PrefillTiles &mt) {
    const int64_t a = prefill_max_deferred(2 * d->inter, QI4_PACK_GATEUP, mt);
    const int64_t b = prefill_max_deferred(d->hidden, 0, mt);
    return a > b ? a : b;
}

// Workspace regions.  W4A8 (w4a8): h holds int8 rows and x8 the int8 input,
// and every batch runs the decode GEMMs (no prefill regions).
struct MoeWorkspace {
    int64_t ids, wts, sorted, offsets, p2s, active, h, y, x16, ex, h16, eh, tiles, ntiles, deferred,
        x8, mids, total;
    MoeWorkspace(const qi4_moe_desc *d, int64_t T, bool w4a8 = false) {
        const int64_t P = T * d->top_k;
        const int64_t R = P + (d->has_shared ? T : 0);
        const bool pf = !w4a8 && T >= kPrefillMinT;
        int64_t o = 0;
        ids = o;     o += align256(P * 4);
        wts = o;     o += align256(P * 4);
        sorted = o;  o += align256(P * 4);
        offsets = o; o += align256((d->num_experts + 1) * 4);
        p2s = o;     o += align256(P * 4);
        active = o;  o += align256((d->num_experts + 1) * 4);
        h = o;       o += align256(w4a8 ? R * d->inter : R * 2 * d->inter * 2);
        y = o;       o += align256(R * d->hidden * 4);
        // fp16 rows with per-row exponents (both GEMM paths; not W4A8), then,
        // for the prefill only, the tile list
        x16 = o;     o += !w4a8 ? align256(T * d->hidden * 2) : 0;
        ex = o;      o += !w4a8 ? align256(T * 4) : 0;
        h16 = o;     o += !w4a8 ? align256(R * d->inter * 2) : 0;
        eh = o;      o += !w4a8 ? align256(R * 4) : 0;
        const PrefillTiles mt = prefill_max_tiles(T, d->top_k, d->num_experts, d->has_shared);
        tiles = o;   o += pf ? align256((mt.big + 3 * mt.small) * 8) : 0;
        ntiles = o;  o += pf ? 256 : 0;
        deferred = o; o += pf ? align256(prefill_deferred_capacity(d, mt) * 16) : 0;
        x8 = o;      o += w4a8 ? align256(T * d->hidden) : 0;
        mids = o;    o += align256(P * 4);   // ids with the experts of another device dropped
        total = o;
    }
};

int bits_for(int64_t E) {
    int b = 0;
    while ((int64_t(1) << b) < E) ++b;
    return b;
}

// prep.x given: T more workgroups prepare the layer input's rows.
int launch_route(const float *logits, int64_t T, int E, int k, int32_t *ids, float *wts,
                 hipStream_t st, RowPrep prep = {}) {
    const int64_t rb = ceil_div(T, kRouteWaves);
    const int64_t blocks = rb + (prep.x ? T : 0);
    if (blocks > 0x7fffffff) return QI4_ERR_SHAPE;
    const int vpl = (E + 63) / 64;
    const dim3 g((unsigned)blocks), b(kRouteWaves * 64);
    if (vpl <= 1) route_kernel<1><<<g, b, 0, st>>>(logits, T, E, k, ids, wts, rb, prep);
    else if (vpl <= 2) route_kernel<2><<<g, b, 0, st>>>(logits, T, E, k, ids, wts, rb, prep);
    else if (vpl <= 4) route_kernel<4><<<g, b, 0, st>>>(logits, T, E, k, ids, wts, rb, prep);
    else if (vpl <= 8) route_kernel<8><<<g, b, 0, st>>>(logits, T, E, k, ids, wts, rb, prep);
    else route_kernel<16><<<g, b, 0, st>>>(logits, T, E, k, ids, wts, rb, prep);
    return launch_status();
}

int launch_sort(const int32_t *ids, int64_t npairs, int E, int32_t *sorted, int32_t *offsets,
                int32_t *p2s, int32_t *active, hipStream_t st) {
    // 16 waves once there are enough pairs to keep them busy
    if (npairs >= 4096)
        sort_kernel<16><<<1, 16 * 64, 0, st>>>(ids, npairs, E, bits_for(E), sorted, offsets, p2s,
                                              active);
    else
        sort_kernel<8><<<1, 8 * 64, 0, st>>>(ids, npairs, E, bits_for(E), sorted, offsets, p2s,
                                               active);
    return launch_status();
}

// Routing then sort: one fused workgroup for decode batches, else the two
// kernels.  prep.x given: the same launch also prepares the layer input's rows
// (T more workgroups).
int launch_route_sort(const float *logits, int64_t T, int E, int k, int32_t *ids, float *wts,
                      int32_t *sorted, int32_t *offsets, int32_t *p2s, int32_t *active,
                      hipStream_t st, RowPrep prep = {}) {
    if (T > kFusedWaves || T * k > kFusedPairs) {
        int rc = launch_route(logits, T, E, k, ids, wts, st, prep);
        if (rc) return rc;
        return launch_sort(ids, T * k, E, sorted, offsets, p2s, active, st);
    }
    const int vpl = (E + 63) / 64, nb = bits_for(E);
    const unsigned g = 1 + (prep.x ? (unsigned)T : 0u);
    auto go = [&](auto w) {
        constexpr int W = decltype(w)::value;
        const unsigned tb = W * 64;
        if (vpl <= 1) route_sort_kernel<1, W><<<g, tb, 0, st>>>(logits, T, E, k, nb, ids, wts, sorted, offsets, p2s, active, prep);
        else if (vpl <= 2) route_sort_kernel<2, W><<<g, tb, 0, st>>>(logits, T, E, k, nb, ids, wts, sorted, offsets, p2s, active, prep);
        else if (vpl <= 4) route_sort_kernel<4, W><<<g, tb, 0, st>>>(logits, T, E, k, nb, ids, wts, sorted, offsets, p2s, active, prep);
        else if (vpl <= 8) route_sort_kernel<8, W><<<g, tb, 0, st>>>(logits, T, E, k, nb, ids, wts, sorted, offsets, p2s, active, prep);
        else route_sort_kernel<16, W><<<g, tb, 0, st>>>(logits, T, E, k, nb, ids, wts, sorted, offsets, p2s, active, prep);
    };
    if (T <= 4) go(std::integral_constant<int, 4>());
    else go(std::integral_constant<int, kFusedWaves>());
    return launch_status();
}

GemmArgs gate_up_args(const qi4_moe_desc *d, const void *x, int64_t T, const int32_t *sorted,
                      const int32_t *offsets, const int32_t *active, const void *w_gu,
                      const void *sh_gu, void *h) {
    GemmArgs a = {};
    a.w = static_cast<const uint8_t *>(w_gu);
    a.w_stride = gate_up_bytes(d);
    a.w_shared = static_cast<const uint8_t *>(sh_gu);
    a.N = 2 * d->inter;
    a.K = packed_k(d->hidden, d->flags);
    a.flags = gate_up_flags(d);
    a.group_size = gs_gate_up(d);
    a.a = x;
    a.lda = d->hidden;
    a.a_shift = a_shift_of(d);
    a.a_bytes = T * d->hidden * 2;
    a.a_f32 = 0;
    a.P = 1;
    a.moe = 1;
    a.T = T;
    a.top_k = d->top_k;
    a.sorted_pairs = sorted;
    a.offsets = offsets;
    a.active = active;
    a.routed_slots = (int)(T * d->top_k < d->num_experts ? T * d->top_k : d->num_experts);
    a.gather_tokens = 1;
    a.out = h;
    a.ldo = d->inter;
    a.out_mode = OUT_SPLIT2;
    a.epi = QI4_EPI_SILU_MUL;
    a.n_out = d->inter;
    return a;
}

GemmArgs down_args(const qi4_moe_desc *d, const void *h, int64_t T, const int32_t *offsets,
                   const int32_t *active, const void *w_dn, const void *sh_dn, float *y) {
    GemmArgs a = {};
    a.w = static_cast<const uint8_t *>(w_dn);
    a.w_stride = down_bytes(d);
    a.w_shared = static_cast<const uint8_t *>(sh_dn);
    a.N = d->hidden;
    a.K = packed_k(d->inter, d->flags);
    a.flags = down_flags(d);
    a.group_size = gs_down(d);
    a.a = h;
    a.lda = d->inter;
    a.a_shift = a_shift_of(d);
    a.a_bytes = (T * d->top_k + (d->has_shared ? T : 0)) * 2 * d->inter * 2;
    a.a_f32 = 0;
    a.P = 2;
    a.moe = 1;
    a.T = T;
    a.top_k = d->top_k;
    a.offsets = offsets;
    a.active = active;
    a.routed_slots = (int)(T * d->top_k < d->num_experts ? T * d->top_k : d->num_experts);
    a.gather_tokens = 0;
    a.out = y;
    a.ldo = d->hidden;
    a.out_mode = OUT_F32;
    a.epi = QI4_EPI_NONE;
    a.n_out = d->hidden;
    return a;
}

PrefillArgs prefill_args(const qi4_moe_desc *d, int64_t T, bool gate_up, const int32_t *sorted,
                         const int32_t *offsets, const int32_t *active, const void *w,
                         const void *w_shared, const uint16_t *a16, const int32_t *aexp,
                         const int2 *tiles, const int32_t *ntiles, int4 *deferred, void *out) {
    PrefillArgs a = {};
    const PrefillTiles mt = prefill_max_tiles(T, d->top_k, d->num_experts, d->has_shared);
    a.max_big = mt.big;
    a.max_small = mt.small;
    a.deferred = deferred;
    a.deferred_count = const_cast<int32_t *>(ntiles) + 4;
    a.max_deferred = prefill_deferred_capacity(d, mt);
    const int64_t H = d->hidden, I = d->inter;
    a.w = static_cast<const uint8_t *>(w);
    a.w_shared = static_cast<const uint8_t *>(w_shared);
    a.N = gate_up ? 2 * I : H;
    a.K = packed_k(gate_up ? H : I, d->flags);
    a.a_shift = a_shift_of(d);
    a.flags = gate_up ? gate_up_flags(d) : down_flags(d);
    a.group_size = gate_up ? gs_gate_up(d) : gs_down(d);
    a.w_stride = PackedLayout(a.N, a.K, a.flags, a.group_size).bytes;
    a.a16 = a16;
    a.a_rows = gate_up ? T : T * d->top_k + (d->has_shared ? T : 0);
    a.a_exp = aexp;
    a.gather_tokens = gate_up ? 1 : 0;
    a.sorted_pairs = sorted;
    a.offsets = offsets;
    a.active = active;
    a.top_k = d->top_k;
    a.T = T;
    a.tiles = tiles;
    a.tile_count = ntiles;
    a.out = out;
    a.ldo = gate_up ? I : H;
    a.epi = gate_up ? QI4_EPI_SILU_MUL : QI4_EPI_NONE;
    a.n_out = gate_up ? I : H;
    return a;
}

// Problems of a grouped decode launch: the routed experts' slots, then the
// shared expert split into one problem per M tile of slots (16 / P), so that
// its workgroups stream its weights side by side, each in one pass (from the
// cache after the first), rather than one workgroup per tile block looping
// over the M tiles and finishing last.
int grouped_problems(GemmArgs &a, const qi4_moe_desc *d, int64_t T) {
    if (!d->has_shared) return a.routed_slots;
    a.shared_rows = 16 / a.P;
    return a.routed_slots + (int)ceil_div(T, (int64_t)a.shared_rows);
}

// The two projections of the expert FFN on either path.  `ws` is the moe_ffn_int4
// workspace (only its prefill regions are used here).
// x_ready: the workspace already holds the input rows as fp16 (prepared by the
// routing launch).
int run_gate_up(const qi4_moe_desc *d, const void *x, int64_t T, const int32_t *sorted,
                const int32_t *offsets, const int32_t *active, const void *w_gu, const void *sh_gu,
                void *h, uint8_t *ws, hipStream_t st, bool x_ready = false) {
    int rc;
    // the input rows once as fp16 with a per-row power of two (exact), for
    // every expert's GEMM
    const MoeWorkspace L(d, T);
    uint16_t *x16 = reinterpret_cast<uint16_t *>(ws + L.x16);
    int32_t *ex = reinterpret_cast<int32_t *>(ws + L.ex);
    if (!x_ready && (rc = launch_prep_rows(x, 0, T, d->hidden, x16, ex, st))) return rc;
    if (T < kPrefillMinT) {
        GemmArgs a = gate_up_args(d, x16, T, sorted, offsets, active, w_gu, sh_gu, h);
        a.a_f16 = 1;
        a.a_exp = ex;
        return launch_qgemm(a, grouped_problems(a, d, T), T, st);
    }
    int2 *tiles = reinterpret_cast<int2 *>(ws + L.tiles);
    int32_t *nt = reinterpret_cast<int32_t *>(ws + L.ntiles);
    int4 *def = reinterpret_cast<int4 *>(ws + L.deferred);
    PrefillArgs a = prefill_args(d, T, true, sorted, offsets, active, w_gu, sh_gu, x16, ex, tiles, nt, def, h);
    if ((rc = launch_plan(offsets, active, T, d->has_shared, tiles, {a.max_big, a.max_small}, nt, st)))
        return rc;
    return launch_prefill(a, st);
}

int run_down(const qi4_moe_desc *d, const void *h, int64_t T, const int32_t *offsets,
             const int32_t *active, const void *w_dn, const void *sh_dn, float *y, uint8_t *ws,
             hipStream_t st) {
    int rc;
    // h (hi + lo bf16 pairs) once as fp16 rows with a per-row power of two
    const MoeWorkspace L(d, T);
    const int64_t R = T * d->top_k + (d->has_shared ? T : 0);
    uint16_t *h16 = reinterpret_cast<uint16_t *>(ws + L.h16);
    int32_t *eh = reinterpret_cast<int32_t *>(ws + L.eh);
    if ((rc = launch_prep_rows(h, 1, R, d->inter, h16, eh, st))) return rc;
    if (T < kPrefillMinT) {
        GemmArgs a = down_args(d, h16, T, offsets, active, w_dn, sh_dn, y);
        a.a_f16 = 1;
        a.a_exp = eh;
        a.a_bytes = R * d->inter * 2;
        a.P = 1;
        return launch_qgemm(a, grouped_problems(a, d, T), T, st);
    }
    int2 *tiles = reinterpret_cast<int2 *>(ws + L.tiles);
    int32_t *nt = reinterpret_cast<int32_t *>(ws + L.ntiles);
    int4 *def = reinterpret_cast<int4 *>(ws + L.deferred);
    PrefillArgs a = prefill_args(d, T, false, nullptr, offsets, active, w_dn, sh_dn, h16, eh, tiles, nt, def, y);
    if ((rc = launch_plan(offsets, active, T, d->has_shared, tiles, {a.max_big, a.max_small}, nt, st)))
        return rc;
    return launch_prefill(a, st);
}

int launch_combine(const qi4_moe_desc *d, const float *y, const float *wts, const int32_t *p2s,
                   int64_t T, void *out, hipStream_t st) {
    if (T > 65535) return QI4_ERR_SHAPE;   // grid.y limit; check_T enforces it
    const dim3 g((unsigned)ceil_div(d->hidden, 1024), (unsigned)T);
    combine_kernel<<<g, 256, 0, st>>>(y, wts, p2s, T, d->top_k, d->hidden, d->has_shared,
                                      static_cast<uint16_t *>(out));
    return launch_status();
}

int check_T(int64_t T, const qi4_moe_desc *d) {
    if (T < 0 || T > 65535) return QI4_ERR_SHAPE;
    const int64_t R = T * d->top_k + (d->has_shared ? T : 0);
    if (R * 2 * d->inter * 2 >= (int64_t(1) << 31) || T * d->hidden * 2 >= (int64_t(1) << 31))
        return QI4_ERR_SHAPE;
    if (gate_up_bytes(d) >= (int64_t(1) << 31) || down_bytes(d) >= (int64_t(1) << 31))
        return QI4_ERR_SHAPE;
    return QI4_OK;
}

}  // namespace
}  // namespace qi4

using namespace qi4;

extern "C" {

int moe_router_topk(const void *x, int64_t T, int64_t H, const void *w_router, int64_t E,
                    int32_t top_k, float *logits, int32_t *topk_ids, float *topk_weights,
                    void *stream) {
    if (E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E) return QI4_ERR_SHAPE;
    if (H < 32 || H % 32 != 0 || T < 0) return QI4_ERR_SHAPE;
    if (T * H * 2 >= (int64_t(1) << 31) || E * H * 2 >= (int64_t(1) << 31) ||
        ceil_div(T, 64) > 65535)
        return QI4_ERR_SHAPE;
    if (T == 0) return QI4_OK;
    if (!x || !w_router || !logits || !topk_ids || !topk_weights) return QI4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16)) return QI4_ERR_SHAPE;
    const int64_t lb = T * E * 4, ib = T * top_k * 4;
    if (overlaps(logits, lb, x, T * H * 2) || overlaps(logits, lb, w_router, E * H * 2) ||
        overlaps(topk_ids, ib, x, T * H * 2) || overlaps(topk_ids, ib, w_router, E * H * 2) ||
        overlaps(topk_weights, ib, x, T * H * 2) || overlaps(topk_weights, ib, w_router, E * H * 2) ||
        overlaps(topk_ids, ib, logits, lb) || overlaps(topk_weights, ib, logits, lb) ||
        overlaps(topk_ids, ib, topk_weights, ib))
        return QI4_ERR_ALIAS;
    int rc = check_device();
    if (rc) return rc;
    hipStream_t st = as_stream(stream);
    if ((rc = launch_router_gemm(static_cast<const uint16_t *>(x),
                                 static_cast<const uint16_t *>(w_router), T, H, (int)E, logits,
                                 st)))
        return rc;
    return launch_route(logits, T, (int)E, top_k, topk_ids, topk_weights, st);
}

int moe_route_topk(const float *logits, int64_t T, int64_t E, int32_t top_k, int32_t *topk_ids,
                   float *topk_weights, void *stream) {
    if (E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E) return QI4_ERR_SHAPE;
    if (T < 0 || T > (int64_t(1) << 31)) return QI4_ERR_SHAPE;
    if (T == 0) return QI4_OK;
    if (!logits || !topk_ids || !topk_weights) return QI4_ERR_NULL;
    if (overlaps(topk_ids, T * top_k * 4, logits, T * E * 4) ||
        overlaps(topk_weights, T * top_k * 4, logits, T * E * 4) ||
        overlaps(topk_ids, T * top_k * 4, topk_weights, T * top_k * 4))
        return QI4_ERR_ALIAS;
    int rc = check_device();
    if (rc) return rc;
    return launch_route(logits, T, (int)E, top_k, topk_ids, topk_weights, as_stream(stream));
}

int moe_route_sort(const float *logits, int64_t T, int64_t E, int32_t top_k, int32_t *topk_ids,
                   float *topk_weights, int32_t *sorted_pairs, int32_t *expert_offsets,
                   int32_t *pair_to_sorted, int32_t *active, void *stream) {
    if (E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E) return QI4_ERR_SHAPE;
    if (T < 0 || T * top_k > (int64_t(1) << 30)) return QI4_ERR_SHAPE;
    if (T == 0) return QI4_OK;
    if (!logits || !topk_ids || !topk_weights || !sorted_pairs || !expert_offsets ||
        !pair_to_sorted || !active)
        return QI4_ERR_NULL;
    const int64_t P = T * top_k, lb = T * E * 4;
    const void *outs[6] = {topk_ids, topk_weights, sorted_pairs, pair_to_sorted, expert_offsets, active};
    const int64_t sizes[6] = {P * 4, P * 4, P * 4, P * 4, (E + 1) * 4, (E + 1) * 4};
    for (int i = 0; i < 6; ++i) {
        if (overlaps(outs[i], sizes[i], logits, lb)) return QI4_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], sizes[i], outs[j], sizes[j])) return QI4_ERR_ALIAS;
    }
    int rc = check_device();
    if (rc) return rc;
    return launch_route_sort(logits, T, (int)E, top_k, topk_ids, topk_weights, sorted_pairs,
                             expert_offsets, pair_to_sorted, active, as_stream(stream));
}

int moe_sort_tokens(const int32_t *topk_ids, int64_t T, int32_t top_k, int64_t E,
                    int32_t *sorted_pairs, int32_t *expert_offsets, int32_t *pair_to_sorted,
                    int32_t *active, void *stream) {
    if (E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK) return QI4_ERR_SHAPE;
    if (T < 0 || T * top_k > (int64_t(1) << 30)) return QI4_ERR_SHAPE;
    if (!topk_ids || !sorted_pairs || !expert_offsets || !pair_to_sorted) return QI4_ERR_NULL;
    const int64_t P = T * top_k;
    if (overlaps(sorted_pairs, P * 4, topk_ids, P * 4) ||
        overlaps(pair_to_sorted, P * 4, topk_ids, P * 4) ||
        overlaps(expert_offsets, (E + 1) * 4, topk_ids, P * 4) ||
        overlaps(active, (E + 1) * 4, topk_ids, P * 4))
        return QI4_ERR_ALIAS;
    int rc = check_device();
    if (rc) return rc;
    return launch_sort(topk_ids, P, (int)E, sorted_pairs, expert_offsets, pair_to_sorted, active,
                       as_stream(stream));
}

int64_t moe_ffn_int4_workspace_bytes(const qi4_moe_desc *d, int64_t T) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    return MoeWorkspace(d, T).total;
}

int moe_expert_gate_up(const qi4_moe_desc *d, const void *x, int64_t T,
                       const int32_t *sorted_pairs, const int32_t *expert_offsets,
                       const int32_t *active, const void *w_gate_up, const void *shared_gate_up,
                       void *h, void *workspace, int64_t ws_bytes, void *stream) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    if (T == 0) return QI4_OK;
    if (!x || !sorted_pairs || !expert_offsets || !active || !w_gate_up || !h || !workspace)
        return QI4_ERR_NULL;
    if ((d->has_shared != 0) != (shared_gate_up != nullptr)) return QI4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_gate_up, 16) || !aligned(h, 4) || !aligned(workspace, 256) ||
        (shared_gate_up && !aligned(shared_gate_up, 16)))
        return QI4_ERR_SHAPE;
    if (ws_bytes < MoeWorkspace(d, T).total) return QI4_ERR_WORKSPACE;
    if ((rc = check_device())) return rc;
    return run_gate_up(d, x, T, sorted_pairs, expert_offsets, active, w_gate_up, shared_gate_up, h,
                       static_cast<uint8_t *>(workspace), as_stream(stream));
}

int moe_expert_down(const qi4_moe_desc *d, const void *h, int64_t T, const int32_t *expert_offsets,
                    const int32_t *active, const void *w_down, const void *shared_down, float *y,
                    void *workspace, int64_t ws_bytes, void *stream) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    if (T == 0) return QI4_OK;
    if (!h || !expert_offsets || !active || !w_down || !y || !workspace) return QI4_ERR_NULL;
    if ((d->has_shared != 0) != (shared_down != nullptr)) return QI4_ERR_NULL;
    if (!aligned(h, 16) || !aligned(w_down, 16) || !aligned(y, 4) || !aligned(workspace, 256) ||
        (shared_down && !aligned(shared_down, 16)))
        return QI4_ERR_SHAPE;
    if (ws_bytes < MoeWorkspace(d, T).total) return QI4_ERR_WORKSPACE;
    if ((rc = check_device())) return rc;
    return run_down(d, h, T, expert_offsets, active, w_down, shared_down, y,
                    static_cast<uint8_t *>(workspace), as_stream(stream));
}

int moe_combine(const qi4_moe_desc *d, const float *y, const float *topk_weights,
                const int32_t *pair_to_sorted, int64_t T, void *out, void *stream) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    if (T == 0) return QI4_OK;
    if (!y || !topk_weights || !pair_to_sorted || !out) return QI4_ERR_NULL;
    if (!aligned(y, 16) || !aligned(out, 8)) return QI4_ERR_SHAPE;
    const int64_t R = T * d->top_k + (d->has_shared ? T : 0);
    if (overlaps(out, T * d->hidden * 2, y, R * d->hidden * 4)) return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;
    return launch_combine(d, y, topk_weights, pair_to_sorted, T, out, as_stream(stream));
}

}  // extern "C"

namespace {

// Static int8 scale: finite, positive, with a finite float32 reciprocal.
bool good_scale(float s) { return s > 0.f && s < INFINITY && 1.0f / s < INFINITY; }

// moe_ffn_int4 and moe_ffn_w4a8 (scales given).
int moe_ffn_impl(const qi4_moe_desc *d, const void *x, int64_t T, const float *router_logits,
                 int32_t *topk_ids, float *topk_weights, const void *w_gate_up, const void *w_down,
                 const void *shared_gate_up, const void *shared_down, void *out, void *workspace,
                 int64_t ws_bytes, void *stream, const float *w4a8_scales,
                 const uint8_t *gpu_experts = nullptr) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    if (T == 0) return QI4_OK;
    if (!x || !w_gate_up || !w_down || !out || !workspace) return QI4_ERR_NULL;
    if (!router_logits && (!topk_ids || !topk_weights)) return QI4_ERR_NULL;
    if ((d->has_shared != 0) != (shared_gate_up != nullptr) ||
        (d->has_shared != 0) != (shared_down != nullptr))
        return QI4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(out, 8) ||
        !aligned(workspace, 256) || (shared_gate_up && !aligned(shared_gate_up, 16)) ||
        (shared_down && !aligned(shared_down, 16)))
        return QI4_ERR_SHAPE;
    const bool w4a8 = w4a8_scales != nullptr;
    if (w4a8) {
        if (d->flags != 0) return QI4_ERR_UNSUPPORTED;   // 4-bit experts
        if (!good_scale(w4a8_scales[0]) || !good_scale(w4a8_scales[1])) return QI4_ERR_SHAPE;
    }
    const MoeWorkspace L(d, T, w4a8);
    if (ws_bytes < L.total) return QI4_ERR_WORKSPACE;
    const int64_t H = d->hidden;
    if (overlaps(out, T * H * 2, x, T * H * 2) || overlaps(out, T * H * 2, workspace, ws_bytes) ||
        overlaps(workspace, ws_bytes, x, T * H * 2))
        return QI4_ERR_ALIAS;
    if ((rc = check_device())) return rc;

    hipStream_t st = as_stream(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const int E = (int)d->num_experts, k = d->top_k;
    int32_t *ids = topk_ids ? topk_ids : reinterpret_cast<int32_t *>(ws + L.ids);
    float *wts = topk_weights ? topk_weights : reinterpret_cast<float *>(ws + L.wts);
    int32_t *sorted = reinterpret_cast<int32_t *>(ws + L.sorted);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *p2s = reinterpret_cast<int32_t *>(ws + L.p2s);
    int32_t *active = reinterpret_cast<int32_t *>(ws + L.active);
    void *h = ws + L.h;
    float *y = reinterpret_cast<float *>(ws + L.y);

    bool x_ready = false;
    if (gpu_experts) {
        // a share of the experts: route in full (the caller's routing outputs
        // keep every pair), then sort only the pairs of this device's experts
        int32_t *mids = reinterpret_cast<int32_t *>(ws + L.mids);
        if (router_logits) {
            RowPrep prep = {};
            if (!w4a8)
                prep = {static_cast<const uint16_t *>(x), H,
                        reinterpret_cast<uint16_t *>(ws + L.x16),
                        reinterpret_cast<int32_t *>(ws + L.ex)};
            if ((rc = launch_route(router_logits, T, E, k, ids, wts, st, prep))) return rc;
            x_ready = !w4a8;
        }
        const int64_t np = T * k;
        const unsigned gm = (unsigned)(ceil_div(np, 256) < 1024 ? ceil_div(np, 256) : 1024);
        mask_ids_kernel<<<gm, 256, 0, st>>>(ids, np, gpu_experts, E, mids);
        if ((rc = launch_status())) return rc;
        if ((rc = launch_sort(mids, np, E, sorted, offsets, p2s, active, st))) return rc;
    } else if (router_logits) {
        // the bf16 path's input rows are prepared by the routing launch
        RowPrep prep = {};
        if (!w4a8)
            prep = {static_cast<const uint16_t *>(x), H, reinterpret_cast<uint16_t *>(ws + L.x16),
                    reinterpret_cast<int32_t *>(ws + L.ex)};
        if ((rc = launch_route_sort(router_logits, T, E, k, ids, wts, sorted, offsets, p2s, active,
                                    st, prep)))
            return rc;
        x_ready = !w4a8;
    } else if ((rc = launch_sort(ids, T * k, E, sorted, offsets, p2s, active, st))) {
        return rc;
    }
    if (w4a8) {
        // int8 x, then gate/up writing int8 h, then down on int8 h (decode GEMMs)
        const int64_t R = T * k + (d->has_shared ? T : 0);
        uint8_t *x8 = ws + L.x8;
        if ((rc = launch_quantize_act(x, 0, T, H, 1.0f / w4a8_scales[0], x8, st))) return rc;
        GemmArgs a = gate_up_args(d, x, T, sorted, offsets, active, w_gate_up, shared_gate_up, h);
        a.a = x8;
        a.a_bytes = T * H;
        a.a_i8 = 1;
        a.a_scale = w4a8_scales[0];
        a.out_mode = OUT_I8;
        a.out_r = 1.0f / w4a8_scales[1];
        if ((rc = launch_qgemm(a, grouped_problems(a, d, T), T, st))) return rc;
        GemmArgs b = down_args(d, h, T, offsets, active, w_down, shared_down, y);
        b.a_bytes = R * d->inter;
        b.a_i8 = 1;
        b.a_scale = w4a8_scales[1];
        b.P = 1;
        if ((rc = launch_qgemm(b, grouped_problems(b, d, T), T, st))) return rc;
        return launch_combine(d, y, wts, p2s, T, out, st);
    }
    if ((rc = run_gate_up(d, x, T, sorted, offsets, active, w_gate_up, shared_gate_up, h, ws, st,
                          x_ready)))
        return rc;
    if ((rc = run_down(d, h, T, offsets, active, w_down, shared_down, y, ws, st))) return rc;
    return launch_combine(d, y, wts, p2s, T, out, st);
}

}  // namespace

extern "C" {

int moe_ffn_int4(const qi4_moe_desc *d, const void *x, int64_t T, const float *router_logits,
                 int32_t *topk_ids, float *topk_weights, const void *w_gate_up, const void *w_down,
                 const void *shared_gate_up, const void *shared_down, void *out, void *workspace,
                 int64_t ws_bytes, void *stream) {
    return moe_ffn_impl(d, x, T, router_logits, topk_ids, topk_weights, w_gate_up, w_down,
                        shared_gate_up, shared_down, out, workspace, ws_bytes, stream, nullptr);
}

int moe_ffn_int4_share(const qi4_moe_desc *d, const void *x, int64_t T,
                       const float *router_logits, int32_t *topk_ids, float *topk_weights,
                       const void *w_gate_up, const void *w_down, const void *shared_gate_up,
                       const void *shared_down, const uint8_t *gpu_experts, void *out,
                       void *workspace, int64_t ws_bytes, void *stream) {
    if (!gpu_experts) return QI4_ERR_NULL;
    return moe_ffn_impl(d, x, T, router_logits, topk_ids, topk_weights, w_gate_up, w_down,
                        shared_gate_up, shared_down, out, workspace, ws_bytes, stream, nullptr,
                        gpu_experts);
}

int64_t moe_ffn_w4a8_workspace_bytes(const qi4_moe_desc *d, int64_t T) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    return MoeWorkspace(d, T, true).total;
}

int moe_ffn_w4a8(const qi4_moe_desc *d, const void *x, float x_scale, float h_scale, int64_t T,
                 const float *router_logits, int32_t *topk_ids, float *topk_weights,
                 const void *w_gate_up, const void *w_down, const void *shared_gate_up,
                 const void *shared_down, void *out, void *workspace, int64_t ws_bytes,
                 void *stream) {
    const float sc[2] = {x_scale, h_scale};
    return moe_ffn_impl(d, x, T, router_logits, topk_ids, topk_weights, w_gate_up, w_down,
                        shared_gate_up, shared_down, out, workspace, ws_bytes, stream, sc);
}

}  // extern "C"

// ---- the layer without a caller workspace ----------------------------------------
//
// Scratch of moe_ffn_int4_noalloc: a file-scope device array, one copy per GPU
// (part of the code object, so it lives until the process ends).  Host code
// never passes the array's name to a kernel: that name is a host-side stand-in.
// The device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is used.  Nothing in it has
// to start at zero: every region is written before it is read within a call
// (routing, permutation, fp16 rows, h, y; the prefill tile counters are reset
// by the planner).  Calls that overlap in time on one GPU share it and race.
namespace {
__device__ __align__(256) uint8_t scratch[QI4_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
    std::once_flag once;
    void *ptr = nullptr;
    int rc = QI4_ERR_HIP;
};
constexpr int kScratchDevices = 64;
ScratchAddr g_scratch[kScratchDevices];

int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return QI4_ERR_HIP;
    ScratchAddr &sa = g_scratch[dev];
    std::call_once(sa.once, [&sa] {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) {
            sa.ptr = p;
            sa.rc = QI4_OK;
        }
    });
    *out = sa.ptr;
    return sa.rc;
}
}  // namespace

extern "C" int moe_ffn_int4_noalloc(const qi4_moe_desc *d, const void *x, int64_t T,
                                    const float *router_logits, int32_t *topk_ids,
                                    float *topk_weights, const void *w_gate_up,
                                    const void *w_down, const void *shared_gate_up,
                                    const void *shared_down, void *out, void *stream) {
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_T(T, d))) return rc;
    if (MoeWorkspace(d, T).total > (int64_t)QI4_NOALLOC_SCRATCH_BYTES) return QI4_ERR_WORKSPACE;
    if (T == 0) return QI4_OK;
    if ((rc = check_device())) return rc;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return moe_ffn_impl(d, x, T, router_logits, topk_ids, topk_weights, w_gate_up, w_down,
                        shared_gate_up, shared_down, out, ws, (int64_t)QI4_NOALLOC_SCRATCH_BYTES,
                        stream, nullptr);
}

