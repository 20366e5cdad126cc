// Prefill (many tokens per expert) grouped GEMM of the MoE FFN on fp16 MFMA.
//
// At prefill sizes each expert's weights are reused by tens to thousands of
// tokens, so the product is a dense contraction near the MFMA/HBM ridge rather
// than a weight stream.  The design:
//  * activations are converted once per row to fp16 with an exact power-of-two
//    prescale (value = fp16 * 2^e, |fp16| < 2^14), so the contraction runs on
//    fp16 MFMA and the row factor 2^e is applied once in the epilogue; the
//    columns k = 2, 3, 6, 7 (mod 8) carry a further exact 2^-4;
//  * each wave dequantizes its own weight rows per 128-wide group straight
//    into fp16 MFMA operands, 16 (q - zero) scale for the columns above and
//    (q - zero) scale for the others (exact integer part, one rounding of the
//    product, relative error <= 2^-11), so no per-group epilogue remains;
//  * a device-side planner splits every expert's rows (and the shared
//    expert's) into big tiles of up to 128 rows and at most one small tile of
//    up to 16, 32 or 64 rows.  Big tiles run on MFMA-bound workgroups (4 waves
//    x 64 weight rows, two-stage pipeline, two workgroups per CU); small tiles
//    run on weight-stream-bound workgroups (8 waves x 32 weight rows,
//    four-stage pipeline, 16 waves per CU) after the big tiles, on the same
//    stream;
//  * the activation tile of each group is copied from memory straight into LDS
//    (buffer loads with the LDS bit), each 4-lane quad reading 64 contiguous
//    bytes, in a rotated order that spreads the MFMA operand reads over the
//    LDS banks, and shared by all waves of the workgroup;
//  * a workgroup whose weights hold a scale the 16x operands cannot represent
//    (|scale| >= 256, inf, NaN) hands its tile to a pass with plain operands.
#include <type_traits>

#include "qi4_gemm.h"
#include "qi4_host.h"
#include "qi4_prefill.h"
#include "qi4_rows.h"

namespace qi4 {
namespace {

// (kOob / kOobS out-of-range offsets and buffer resources: qi4_dev.h)
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return make_rsrc(base, bytes);
}

// fp16 operands scale * (q - zero) of the 8 codes in one packed dword, in the
// element order of the packed layout (see qi4_dev.h): (1024 + q) - (1024 + zero)
// with packed fp16 adds (exact), times the binary16 scale (one rounding).
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

// The same operands with elements 2, 3, 6 and 7 sixteen times larger: their
// codes sit at bits 4..7 of each half, so masking them in place gives
// 1024 + 16q and (1024 + 16q) - (1024 + 16 zero) = 16 (q - zero), exactly.
// Activations at k = 2, 3, 6, 7 (mod 8) are stored divided by 16, so the
// products are unchanged.  One shift, four and-or, four adds, four multiplies
// per 8 codes.  magic holds fp16 1024 in both halves.
__device__ inline uint4 dequant_f16_x16(uint32_t d, uint32_t negz, uint32_t negz16, uint32_t s2,
                                        uint32_t magic) {
    const f16x2 nz = __builtin_bit_cast(f16x2, negz), nz16 = __builtin_bit_cast(f16x2, negz16);
    const f16x2 sc = __builtin_bit_cast(f16x2, s2);
    const uint32_t t = d >> 8;
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, and_or(d, 0x000F000Fu, magic)) + nz) * sc);
    r.y = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, and_or(d, 0x00F000F0u, magic)) + nz16) * sc);
    r.z = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, and_or(t, 0x000F000Fu, magic)) + nz) * sc);
    r.w = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, and_or(t, 0x00F000F0u, magic)) + nz16) * sc);
    return r;
}

// ---- row preparation: fp16 with a per-row power-of-two prescale ----------------

// One workgroup per row (prep_row).
constexpr int kPrepThreads = 256;

__global__ void __launch_bounds__(kPrepThreads)
prep_rows_kernel(const uint16_t *__restrict__ src, int src_kind, int64_t len,
                 uint16_t *__restrict__ dst, int32_t *__restrict__ exps) {
    __shared__ float wmax[kPrepThreads / 64];
    prep_row<kPrepThreads>(src, src_kind, len, blockIdx.x, dst, exps, wmax);
}

// ---- tile planner ---------------------------------------------------------------

// Tiles of a problem (routed expert or the shared one) with n rows: n / 128 big
// tiles of 128 rows, then the remaining n % 128 rows as one more big tile if
// there are more than 64 of them, else as one small tile of at most 16, 32 or
// 64 rows (classes 0, 1, 2).  Big tiles are bound by the MFMAs, small ones by
// the weight stream; each list has its own kernel.  Entry: (problem, first
// slot), problem -1 for the shared expert.  counts: [0] big, [1 + c] small of
// class c, [4] deferred pairs (zeroed here).  Single workgroup; each thread
// owns two problems.
__device__ inline int small_class(int64_t rows) { return rows <= 16 ? 0 : rows <= 32 ? 1 : 2; }

__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t *__restrict__ offsets, const int32_t *__restrict__ active, int64_t T,
            int has_shared, int2 *__restrict__ big, int2 *__restrict__ small, int64_t small_cap,
            int32_t *__restrict__ counts) {
    __shared__ int sc[4][1024];   // [0] big, [1..3] small classes
    const int n_act = active[0];
    const int n_prob = n_act + (has_shared ? 1 : 0);
    const int i = threadIdx.x;
    auto rows = [&](int p) -> int64_t {
        if (p < n_act) {
            const int e = active[1 + p];
            return offsets[e + 1] - offsets[e];
        }
        return T;
    };
    int mine[4] = {0, 0, 0, 0};
    for (int q = 0; q < 2; ++q) {
        const int p = 2 * i + q;
        if (p >= n_prob) break;
        const int64_t n = rows(p), rem = n % kPrefillBM;
        mine[0] += (int)(n / kPrefillBM) + (rem > kPrefillBMSmall ? 1 : 0);
        if (rem > 0 && rem <= kPrefillBMSmall) mine[1 + small_class(rem)] += 1;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[c][i] = mine[c];
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        int v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = i >= d ? sc[c][i - d] : 0;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c) sc[c][i] += v[c];
        __syncthreads();
    }
    int pos[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pos[c] = sc[c][i] - mine[c];
    for (int q = 0; q < 2; ++q) {
        const int p = 2 * i + q;
        if (p >= n_prob) break;
        const int64_t n = rows(p), full = n / kPrefillBM, rem = n % kPrefillBM;
        const int pid = p < n_act ? p : -1;
        for (int64_t k = 0; k < full; ++k) big[pos[0]++] = make_int2(pid, (int)(k * kPrefillBM));
        if (rem > kPrefillBMSmall) {
            big[pos[0]++] = make_int2(pid, (int)(full * kPrefillBM));
        } else if (rem > 0) {
            const int c = small_class(rem);
            small[c * small_cap + pos[1 + c]++] = make_int2(pid, (int)(full * kPrefillBM));
        }
    }
    if (i == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) counts[c] = sc[c][1023];
        counts[4] = 0;
    }
}

// ---- the grouped GEMM ----------------------------------------------------------------

constexpr int kABlock = 1024;          // one MFMA operand fragment of a wave (16 rows x 32 k, fp16)
constexpr int kRowsPerWG = 256;        // weight rows (16 tiles) of one workgroup
constexpr bool kMergeSmall = true;     // see prefill_small12_kernel

// Shapes of the two kernels.  Big tiles: 128 activation rows, 4 waves of 64
// weight rows, 2 pipeline stages, two workgroups per CU (256 registers a wave).
// Small tiles: 64 activation rows, 8 waves of 32 weight rows, 4 stages (three
// groups of requests in flight), 128 registers a wave so that 16 waves share a CU.
template <int MS_, int NBW_, int W_, int S_, int OCC_>
struct Shape {
    static constexpr int MS = MS_;     // 16-row activation subtiles per tile
    static constexpr int NBW = NBW_;   // 16-row weight tiles per wave
    static constexpr int W = W_;       // waves per workgroup
    static constexpr int S = S_;       // pipeline stages
    static constexpr int OCC = OCC_;   // waves per SIMD the register budget allows
    static constexpr int kStageBytes = MS * 4 * kABlock;
    static constexpr int FPW = MS * 4 / W;   // operand fragments each wave copies per group
    static constexpr int NH = FPW >= 4 ? FPW / 4 : 1;   // distinct subtiles each wave copies
    static_assert(W * NBW * 16 == kRowsPerWG, "workgroup rows");
    static constexpr int kLds = S * kStageBytes;   // LDS of one workgroup
    static_assert(kLds <= 160 * 1024, "LDS stages");
    static_assert(FPW >= 1 && (FPW >= 4 ? FPW % 4 == 0 : 4 % FPW == 0), "copy split");
};
using BigShape = Shape<8, 4, 4, 2, 2>;
using SmallShape = Shape<4, 2, 8, 4, 4>;
// Small tiles of class C (<= 16 << C rows) stage only the 1 << C activation
// subtiles they multiply, over 3 stages: 12 / 24 / 48 KiB of LDS for classes
// 0 / 1 / 2 (class 0: 4 waves of 64 weight rows), so they leave room on each
// CU for the big-tile kernel's workgroups beside them (measured: step 2.98 ->
// 2.87-2.90 ms).  With 64-wide groups class 0 keeps the 4-stage 64-row shape
// (the 4-wave one would spill).
template <int C, int H>
using SmallShapeC = std::conditional_t<
    C == 0, std::conditional_t<H == 1, Shape<1, 4, 4, 3, 4>, SmallShape>,
    std::conditional_t<C == 1, Shape<2, 2, 8, 3, 4>, Shape<4, 2, 8, 3, 4>>>;

// s_waitcnt operand that waits until at most `vm` vector memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

// The LDS buffers of the pipeline stages, each its own variable.  The copies
// into a stage are memory requests that write LDS; a read of LDS that may
// overlap them must wait for them.  With one array for all stages the compiler
// cannot tell the stages apart and makes every step's first operand read wait
// for the copies just issued for a later group (one memory latency exposed per
// group); with one variable per stage it can, and waits only where the code
// does.  Stage index: a constant once the pipeline loop is unrolled.
struct Stages {
    uint8_t *p[4];
};
#define QI4_STAGE_LDS(SH_, VAR_)                                                               \
    __shared__ __attribute__((aligned(16))) uint8_t VAR_##0[SH_::kStageBytes];                 \
    __shared__ __attribute__((aligned(16))) uint8_t VAR_##1[SH_::S > 1 ? SH_::kStageBytes : 16]; \
    __shared__ __attribute__((aligned(16))) uint8_t VAR_##2[SH_::S > 2 ? SH_::kStageBytes : 16]; \
    __shared__ __attribute__((aligned(16))) uint8_t VAR_##3[SH_::S > 3 ? SH_::kStageBytes : 16]; \
    const Stages VAR_ = {{VAR_##0, VAR_##1, VAR_##2, VAR_##3}}

// One tile: SH::MS 16-row activation subtiles times this workgroup's 256
// weight rows, over the whole K.
// H = 2: 64-wide quantization groups (two scale/zero records per block).
template <int EPI, class SH, int MU, bool WIDE, int H>
__device__ __forceinline__ void run_tile(const PrefillArgs &args, const PackedLayout &L, const Stages &lds,
                                         int *wg_flag, int2 te, const uint8_t *w, int64_t row0,
                                         int64_t n, int64_t src0, const int32_t *gather, int64_t bx,
                                         int wave, int lane) {
    const int64_t m0 = te.y;
    constexpr int MS = SH::MS, NBW = SH::NBW, S = SH::S, FPW = SH::FPW, NH = SH::NH;
    const int r16 = lane & 15, j = lane >> 4;
    const int64_t nt = L.nt, G = L.G;
    const int64_t tile0 = bx * (kRowsPerWG / 16) + wave * NBW;
    const __amdgpu_buffer_rsrc_t wr = rsrc(w, (uint32_t)L.bytes);
    const int64_t KA = args.K >> args.a_shift;   // activation row length
    const __amdgpu_buffer_rsrc_t ar = rsrc(args.a16, (uint32_t)(args.a_rows * KA * 2));

    // Weight offsets: the lane part is the same for every tile and group; the
    // tile and group part is wave-uniform and goes in soffset (scalar registers).
    // A wave's NBW tiles are aligned inside one quad (tile0 % NBW == 0).
    const uint32_t slot0 = (uint32_t)(tile0 & (kQuadTiles - 1));
    const uint32_t vc = (uint32_t)lane * 16u, vs = (uint32_t)r16 * 8u + 2u * slot0,
                   vz = (uint32_t)r16 * 2u + (slot0 >> 1);
    const int nt_here = (int)(nt - tile0 < NBW ? (nt - tile0 > 0 ? nt - tile0 : 0) : NBW);

    // 16-row subtiles of this tile that hold rows (uniform).
    const int m_used = (int)((n - m0 + 15) / 16 < MS ? (n - m0 + 15) / 16 : MS);

    // Operand fragments this wave copies into LDS each group: fragment
    // f = FPW * wave + i is k step f % 4 of subtile f / 4 (16 rows x 64 bytes).
    // A copy request moves 16 bytes per lane to LDS at 16 * lane.  Lane l
    // copies row l / 4 of the fragment, so every 4 consecutive lanes read 64
    // contiguous bytes (the address unit coalesces them); inside the quad the
    // four 16-byte chunks are rotated by rot(row), so that the 16 lanes of each
    // k quarter of an MFMA operand read (j fixed) hit 16 different 16-byte
    // bank groups.  On this chip the operand reads still stall 4 cycles per
    // KiB (counters); reads in lane order (16 * lane) would not, but then each
    // copy request gathers 16 bytes from 16 rows per 16 lanes, which measured
    // 7-10 % slower overall.
    auto rot = [](int r) { return ((r >> 1) + (r >> 3)) & 3; };
    auto frag_sub = [&](int i) { return (FPW * wave + i) >> 2; };
    auto frag_k = [&](int i) { return (FPW * wave + i) & 3; };
    const int crow = lane >> 2, cchunk = ((lane & 3) - rot(lane >> 2)) & 3;
    uint32_t aoff[NH];   // byte offset of this lane's activation chunk, per copied subtile
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int64_t slot = m0 + 16 * frag_sub(4 * h) + crow;
        const bool ok = slot < n;
        const int64_t slot_c = ok ? slot : 0;
        const int64_t src = gather ? (int64_t)(gather[row0 + slot_c] / args.top_k) : src0 + slot_c;
        aoff[h] = ok ? (uint32_t)((src * KA + 8 * cchunk) * 2) : kOob;
    }
    // MFMA operand lane (row r16, chunk j) finds its chunk at this LDS offset
    const uint32_t rdoff = 16u * (uint32_t)(4 * r16 + ((j + rot(r16)) & 3));

    // Past the last group every lane loads from an out-of-range offset (a
    // select, not a sum, so an invalid row's offset cannot wrap around), which
    // fills zeros.  Big tiles skip the copies of empty subtiles (they wait for
    // all requests); small tiles issue every copy (rows past the end are
    // zero-filled, without a memory access) so that each group costs each
    // wave exactly kReqs requests.
    auto fill = [&](int stage, int g) {
        const bool in = g < G;
        const uint32_t so = in ? (uint32_t)(g >> args.a_shift) * 256u : 0u;
        uint8_t *buf = lds.p[stage];
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            if (S == 2 && frag_sub(i) >= m_used) continue;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ar, (__attribute__((address_space(3))) void *)(buf + (FPW * wave + i) * kABlock), 16,
                in ? aoff[i / 4 < NH ? i / 4 : 0] + 64u * (uint32_t)frag_k(i) : kOob, so, 0, 0);
        }
    };
    struct WStage {
        uint4 cw[NBW];
        uint32_t sc[H][(NBW + 1) / 2], zb[H];
    };
    // memory requests per group per wave: activation copies, codes, and a
    // scale and a zero load per half
    constexpr int kReqs = FPW + NBW + 2 * H;
    // Small tiles (the last tile of their expert) read the weight codes with
    // the non-temporal hint; big tiles leave them in the cache for the
    // expert's other tiles (T = 2048 step: 2.78 -> 2.74 ms; the hint on the
    // big tiles too measured slower).
    constexpr int kCpol = SH::MS == BigShape::MS ? 0 : kCpolNonTemporal;
    auto load_w = [&](WStage &q, int g) {
        const bool in = g < G && nt_here > 0;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const bool ok = in && nb < nt_here;
            const int64_t tg = (tile0 + nb) * G + g;
            const uint32_t oc = ok ? (uint32_t)(tg * 1024) : kOobS;
            q.cw[nb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, vc, oc, kCpol));
        }
#pragma unroll
        for (int h = 0; h < H; ++h)
            load_meta<NBW>(wr, vs, vz, in ? (uint32_t)L.scale_rec(tile0, g) + h * kQuadScaleBytes : kOobS,
                           in ? (uint32_t)L.zero_rec(tile0, g) + h * kQuadZeroBytes : kOobS, q.sc[h],
                           q.zb[h]);
    };

    f32x4 acc[MS][NBW];
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 16 (q - zero) scale can exceed binary16 once |scale| >= 256.  On the fast
    // pass the waves scan the scale records of their tiles' quads (contiguous:
    // G * 128 bytes per quad; of two waves sharing a quad, the first scans it)
    // while the prologue's requests are in flight; a workgroup that finds such
    // a scale (or inf/NaN) records its tile in the deferred list and leaves it
    // to the plain-operand pass.
    bool big = false;
    if constexpr (!WIDE) {
        const bool scans = nt_here > 0 && (tile0 & (kQuadTiles - 1)) == 0;
        const uint32_t span = scans ? (uint32_t)(G * L.srec) : 0u;
        const uint32_t base = (uint32_t)L.scale_rec(tile0, 0);
        for (uint32_t o = 0; o < span; o += 1024) {
            const uint32_t lo = o + (uint32_t)lane * 16u;
            const uint4 v = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, lo < span ? lo : kOob, base, 0));
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                big |= (u[c] & 0x7C00u) >= 0x5C00u || (u[c] & 0x7C000000u) >= 0x5C000000u;
        }
    }

    // Prologue: the first S - 1 groups' activation tiles and weights.
    WStage wst[S];
#pragma unroll
    for (int q = 0; q < S - 1; ++q) {
        fill(q, q);
        load_w(wst[q], q);
    }

    if constexpr (!WIDE) {
        if (threadIdx.x == 0) *wg_flag = 0;
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(big) != 0 && lane == 0) *wg_flag = 1;
        __syncthreads();
        if (*wg_flag) {
            if (threadIdx.x == 0) {
                const int slot = atomicAdd(args.deferred_count, 1);
                args.deferred[slot] = make_int4(te.x, te.y, (int)bx, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);   // the prologue's LDS copies land before exit
            return;
        }
    }

    const uint32_t magic = f16_magic_pair();

    // The main loop multiplies the first MU subtiles (MU * 16 >= the tile's
    // rows; rows past its end only feed output rows that are never stored), so
    // its body has no branches.
    {
        static_assert(MU >= 1 && MU <= MS, "subtiles");
        auto compute = [&](const WStage &q, int stage) {
            const uint8_t *buf = lds.p[stage];
            uint32_t negz[H][NBW], negz16[H][NBW], s2[H][NBW];
#pragma unroll
            for (int h = 0; h < H; ++h)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const uint32_t z = (q.zb[h] >> (4 * nb)) & 15u;
                    // fp16 -(1024 + z) and -(1024 + 16 z) in both halves; scale in both halves
                    negz[h][nb] = (0xE400u | z) * 0x00010001u;
                    negz16[h][nb] = (0xE400u | (z << 4)) * 0x00010001u;
                    s2[h][nb] = ((q.sc[h][nb >> 1] >> (16 * (nb & 1))) & 0xFFFFu) * 0x00010001u;
                }
            auto deq = [&](int s, f16x8 (&b)[NBW]) {
                const int h = H == 2 ? s >> 1 : 0;   // k steps 0, 1 / 2, 3: first / second 64-wide group
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const uint32_t d = s == 0 ? q.cw[nb].x : s == 1 ? q.cw[nb].y : s == 2 ? q.cw[nb].z : q.cw[nb].w;
                    if constexpr (WIDE)
                        b[nb] = __builtin_bit_cast(f16x8, dequant_f16(d, negz[h][nb], s2[h][nb]));
                    else
                        b[nb] = __builtin_bit_cast(f16x8, dequant_f16_x16(d, negz[h][nb], negz16[h][nb], s2[h][nb], magic));
                }
            };
            if constexpr (WIDE || MU < 4) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    f16x8 b[NBW];
                    deq(s, b);
#pragma unroll
                    for (int m = 0; m < MU; ++m) {
                        f16x8 a = *reinterpret_cast<const f16x8 *>(buf + (m * 4 + s) * kABlock + rdoff);
                        if constexpr (WIDE) {
                            // the activations at k = 2, 3, 6, 7 (mod 8) are stored / 16
                            const f16x8 x16 = {1, 1, 16, 16, 1, 1, 16, 16};
                            a = a * x16;
                        }
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) acc[m][nb] = mfma16x16x32_f16(a, b[nb], acc[m][nb]);
                    }
                    // nothing moves across k steps: bounds the registers in flight
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // Tiles of 4 or more subtiles: the next k step's weight operands
                // are dequantized while this step's MFMAs run, one VALU
                // instruction issued after each MFMA (the matrix core works on
                // the MFMA meanwhile).  Measured on the T = 2048 step: 2.82 ->
                // 2.73 ms (two VALU instructions per MFMA: 2.75, three: 2.76).
                f16x8 bc[NBW], bn[NBW];
                deq(0, bc);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < 3) deq(s + 1, bn);
#pragma unroll
                    for (int m = 0; m < MU; ++m) {
                        const f16x8 a =
                            *reinterpret_cast<const f16x8 *>(buf + (m * 4 + s) * kABlock + rdoff);
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            acc[m][nb] = mfma16x16x32_f16(a, bc[nb], acc[m][nb]);
                    }
                    if (s < 3) {
                        // the operand reads first, then MFMA, VALU, MFMA, VALU, ...
                        __builtin_amdgcn_sched_group_barrier(0x100, MU, 0);
#pragma unroll
                        for (int i = 0; i < MU * NBW; ++i) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) bc[nb] = bn[nb];
                }
            }
        };
        // Pipeline: at step g the activation tile and the weights of group
        // g + S - 1 are requested into the stage that group g - 1 used, while
        // group g is multiplied.  At the top of a step this wave waits until
        // group g's requests have landed (the requests issued after them are
        // those of the S - 2 groups that follow, kReqs each; with two stages,
        // none), then the barrier makes every wave's LDS copies of group g
        // visible and frees the stage of group g - 1.
        for (int g = 0; g < G; g += S) {
#pragma unroll
            for (int u = 0; u < S; ++u) {
                if (g + u >= G) break;
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kReqs * (S - 2)));
                __syncthreads();
                const int nxt = (u + S - 1) % S;   // constant once unrolled
                fill(nxt, g + u + S - 1);
                load_w(wst[nxt], g + u + S - 1);
                compute(wst[u], u);
            }
        }
    }
    // the copies requested past the last group (out of range, zero-filled)
    // must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: row factor 2^e, SiLU(gate) * up or the plain output ----
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t slot = m0 + 16 * m + 4 * j + v;
            if (slot >= n) continue;
            const int64_t src = gather ? (int64_t)(gather[row0 + slot] / args.top_k) : src0 + slot;
            const int e = args.a_exp[src];
            const int64_t dst = row0 + slot;
            if constexpr (EPI == QI4_EPI_SILU_MUL) {
#pragma unroll
                for (int p = 0; p < NBW / 2; ++p) {
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
                for (int nb = 0; nb < NBW; ++nb) {
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

// Tile list entry -> problem, then run_tile.
template <int EPI, class SH, int MU, bool WIDE, int H>
__device__ __forceinline__ void tile_entry(const PrefillArgs &args, int2 te, int64_t bx, const Stages &lds,
                                           int *wg_flag) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const PackedLayout L(args.N, args.K, args.flags, args.group_size);
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
    run_tile<EPI, SH, MU, WIDE, H>(args, L, lds, wg_flag, te, w, row0, n, src0, gather, bx, wave, lane);
}

// Workgroup ids are dealt to the 8 XCDs in turn (id mod 8): tile tix goes to
// XCD tix mod 8 and all its column blocks run there back to back, so the
// activation tile they share is fetched once into that XCD's L2.
// bid: the workgroup's index in its region of the grid (regions start at
// multiples of 8, so bid & 7 is still its XCD).
template <int EPI, class SH, int MU, int H>
__device__ __forceinline__ void fast_pass(const PrefillArgs &args, const int2 *tiles, int count,
                                          uint32_t bid, const Stages &lds, int *wg_flag) {
    const int64_t nt = num_tiles(args.N, args.flags);
    const uint32_t gx = (uint32_t)((nt * 16 + kRowsPerWG - 1) / kRowsPerWG);
    const uint32_t kx = bid >> 3;
    const int tix = (int)((kx / gx) * 8 + (bid & 7));
    if (tix >= count) return;
    tile_entry<EPI, SH, MU, false, H>(args, tiles[tix], kx % gx, lds, wg_flag);
}

template <int EPI, int H>
__global__ void __launch_bounds__(BigShape::W * 64, BigShape::OCC)
prefill_big_kernel(const PrefillArgs args) {
    QI4_STAGE_LDS(BigShape, lds);
    __shared__ int wg_flag;
    fast_pass<EPI, BigShape, BigShape::MS, H>(args, args.tiles, args.tile_count[0], blockIdx.x, lds,
                                               &wg_flag);
}

// Small tiles of class C: at most 16 << C rows, 1 << C subtiles multiplied.
template <int EPI, int C, int H>
__global__ void __launch_bounds__((SmallShapeC<C, H>::W * 64), (SmallShapeC<C, H>::OCC))
prefill_small_kernel(const PrefillArgs args) {
    using SH = SmallShapeC<C, H>;
    QI4_STAGE_LDS(SH, lds);
    __shared__ int wg_flag;
    fast_pass<EPI, SmallShapeC<C, H>, 1 << C, H>(args, args.tiles + args.max_big + C * args.max_small,
                                                  args.tile_count[1 + C], blockIdx.x, lds, &wg_flag);
}

// The 17-32- and 33-64-row classes in one launch (128-wide groups; both use
// 8 waves of 32 weight rows): the 33-64-row tiles in the first region_blocks
// workgroups, the others after them, so the first class's last workgroups
// share the chip with the second's first ones instead of leaving CUs idle at
// the end of a launch of their own.
template <int EPI>
__global__ void __launch_bounds__(8 * 64, 4)
prefill_small12_kernel(const PrefillArgs args, uint32_t region_blocks) {
    static_assert(SmallShapeC<1, 1>::W == 8 && SmallShapeC<2, 1>::W == 8, "8-wave shapes");
    // (class 1 stages are smaller and fewer or as many: the class 2 buffers serve both)
    static_assert(SmallShapeC<1, 1>::S <= SmallShapeC<2, 1>::S &&
                      SmallShapeC<1, 1>::kStageBytes <= SmallShapeC<2, 1>::kStageBytes, "stages");
    using SH = SmallShapeC<2, 1>;
    QI4_STAGE_LDS(SH, lds);
    __shared__ int wg_flag;
    const int2 *t = args.tiles + args.max_big;
    if (blockIdx.x < region_blocks)
        fast_pass<EPI, SmallShapeC<2, 1>, 4, 1>(args, t + 2 * args.max_small, args.tile_count[3],
                                               blockIdx.x, lds, &wg_flag);
    else
        fast_pass<EPI, SmallShapeC<1, 1>, 2, 1>(args, t + args.max_small, args.tile_count[2],
                                               blockIdx.x - region_blocks, lds, &wg_flag);
}

// Deferred (tile, column block) pairs, with the plain operands (big-tile shape
// also for small tiles).  A grid-stride loop over the list.
template <int EPI, int H>
__global__ void __launch_bounds__(BigShape::W * 64, BigShape::OCC)
prefill_wide_kernel(const PrefillArgs args) {
    QI4_STAGE_LDS(BigShape, lds);
    const int count = *args.deferred_count;
    for (int i = blockIdx.x; i < count; i += gridDim.x) {
        const int4 d = args.deferred[i];
        tile_entry<EPI, BigShape, BigShape::MS, true, H>(args, make_int2(d.x, d.y), d.z, lds, nullptr);
        __syncthreads();   // LDS is reused by the next entry
    }
}

}  // namespace

int launch_prep_rows(const void *src, int src_kind, int64_t rows, int64_t len, uint16_t *dst,
                     int32_t *exps, hipStream_t st) {
    if (rows <= 0) return QI4_OK;
    if (rows > 0x7fffffff) return QI4_ERR_SHAPE;
    prep_rows_kernel<<<(unsigned)rows, kPrepThreads, 0, st>>>(static_cast<const uint16_t *>(src),
                                                             src_kind, len, dst, exps);
    return launch_status();
}

int launch_plan(const int32_t *offsets, const int32_t *active, int64_t T, int has_shared,
                int2 *tiles, const PrefillTiles &m, int32_t *counts, hipStream_t st) {
    plan_kernel<<<1, 1024, 0, st>>>(offsets, active, T, has_shared, tiles, tiles + m.big, m.small,
                                    counts);
    return launch_status();
}

PrefillTiles prefill_max_tiles(int64_t T, int top_k, int64_t E, int has_shared) {
    // each problem of n rows has at most n / 128 + 1 tiles, at most one small
    const int64_t P = T * top_k;
    const int64_t act = P < E ? P : E;
    PrefillTiles m;
    m.big = P / kPrefillBM + act + (has_shared ? T / kPrefillBM + 1 : 0);
    m.small = act + (has_shared ? 1 : 0);
    return m;
}

int64_t prefill_max_deferred(int64_t N, int flags, const PrefillTiles &m) {
    const int64_t gx = ceil_div(num_tiles(N, flags) * 16, kRowsPerWG);
    return gx * (ceil_div(m.big, 8) + 3 * ceil_div(m.small, 8)) * 8;
}

// All four kernels run on the caller's stream, one after the other: the
// big-tile kernel first (the MFMA-bound bulk of the work, 128-row tiles), then
// the three small-tile classes (weight-streaming), then the pass for deferred
// tiles.  The library keeps no streams or events of its own.
namespace {
template <int EPI, int H>
int launch_prefill_epi(const PrefillArgs &a, hipStream_t st, unsigned gb, unsigned gs) {
    const unsigned tb = BigShape::W * 64;
    const unsigned ts0 = SmallShapeC<0, H>::W * 64, ts1 = SmallShapeC<1, H>::W * 64,
                   ts2 = SmallShapeC<2, H>::W * 64;
    int rc;
    prefill_big_kernel<EPI, H><<<gb, tb, 0, st>>>(a);
    if ((rc = launch_status())) return rc;
    if (H == 1 && kMergeSmall) {
        prefill_small_kernel<EPI, 0, H><<<gs, ts0, 0, st>>>(a);
        prefill_small12_kernel<EPI><<<2 * gs, 8 * 64, 0, st>>>(a, gs);
    } else {
        prefill_small_kernel<EPI, 0, H><<<gs, ts0, 0, st>>>(a);
        prefill_small_kernel<EPI, 1, H><<<gs, ts1, 0, st>>>(a);
        prefill_small_kernel<EPI, 2, H><<<gs, ts2, 0, st>>>(a);
    }
    if ((rc = launch_status())) return rc;
    // tiles deferred by either kind, after both
    prefill_wide_kernel<EPI, H><<<512, tb, 0, st>>>(a);   // two workgroups per CU
    return launch_status();
}
}  // namespace

int launch_prefill(const PrefillArgs &a, hipStream_t st) {
    const int64_t nt = num_tiles(a.N, a.flags);
    const int64_t gx = ceil_div(nt * 16, kRowsPerWG);
    const int64_t gb = gx * ceil_div(a.max_big, 8) * 8, gs = gx * ceil_div(a.max_small, 8) * 8;
    if (gb > 0x7fffffff || 2 * gs > 0x7fffffff) return QI4_ERR_SHAPE;
    if (gb + 3 * gs > a.max_deferred) return QI4_ERR_SHAPE;
    const bool h2 = halves_for(a.group_size) == 2;
    if (a.epi == QI4_EPI_SILU_MUL)
        return h2 ? launch_prefill_epi<QI4_EPI_SILU_MUL, 2>(a, st, (unsigned)gb, (unsigned)gs)
                  : launch_prefill_epi<QI4_EPI_SILU_MUL, 1>(a, st, (unsigned)gb, (unsigned)gs);
    return h2 ? launch_prefill_epi<QI4_EPI_NONE, 2>(a, st, (unsigned)gb, (unsigned)gs)
              : launch_prefill_epi<QI4_EPI_NONE, 1>(a, st, (unsigned)gb, (unsigned)gs);
}

}  // namespace qi4
