// int4-g128 weight-only GEMM for few rows of activations (decode, T <= 32 per
// problem per pass), on bf16 MFMA with float32 accumulation.
//
// The FastLLM page (section 3.1, 4-bit quantization and weight reordering)
// has each 4-bit weight dequantized on the fly inside the matrix product, with
// no separate dequantization pass, and decode time set by how fast the weights
// are read rather than by arithmetic, since every token reads all of them again.
// On CDNA4 that becomes:
//  * one 16-byte load per lane per (16-row tile, 128-wide group): a contiguous
//    kilobyte per wave, prepared by qi4_pack;
//  * the codes become MFMA operands with one AND/OR per pair: bf16 with the
//    bits 0x4300 | q is exactly 128 + q;
//  * the codes become exact fp16 operands q - zero with one and-or and one
//    packed add per pair (fp16 1024 | q is exactly 1024 + q);
//  * the activation rows become exact fp16 operands too: one power of two per
//    (row, 128-wide block) taken from the block's largest exponent, built from
//    the bf16 bits with packed integer ops (qi4_dev.h), and undone on the
//    block's sum;
//  * MFMA 16x16x32 fp16 forms each block's sum of exact products in float32
//    (a code on its zero point adds exactly 0, so no large offset is ever
//    subtracted), and the block adds scale * 2^(c - 112) * sum per output;
//  * the K range is split across the waves of a workgroup and reduced in LDS in
//    a fixed order, so results are deterministic;
//  * a workgroup may stream several consecutive tile blocks through one
//    register pipeline: the next block's first loads are in flight while the
//    previous block is reduced and stored;
//  * the scales and zero points of a quad of four tiles arrive with one load
//    each per group.
// Activations in float32 are split exactly into three bf16 terms (hi + mid +
// lo), each an MFMA row with its own block exponent; the epilogue adds the rows
// of one token back together.
#include "qi4_gemm.h"
#include "qi4_host.h"

namespace qi4 {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kA5TransposeBytes = 4096;   // per wave and M tile, activation mode 5
constexpr bool kDenseMSplit = true;   // see launch_qgemm
constexpr bool kDownWaveBlocks = true;   // see launch_qgemm
// (wave, m, nb) partial tiles the LDS reduction buffer holds: 16 (16 KiB), or
// 32 for a quad of tiles over two M tiles (the only shape that needs more; the
// others keep the smaller buffer so that LDS never caps their occupancy).
template <int NB, int MT>
constexpr int kRedSlotsFor = NB * MT >= 8 ? 32 : 16;
__host__ __device__ constexpr int red_slots(int NB, int MT) { return NB * MT >= 8 ? 32 : 16; }

// Part `part` of the exact split of v into bf16 terms v = hi + mid + lo.
__device__ inline uint32_t split_part(float v, int part) {
    const uint32_t hi = f32_to_bf16_rne(v);
    const float r1 = v - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    const uint32_t lo = f32_to_bf16_rne(r2);
    return part == 0 ? hi : part == 1 ? mid : part == 2 ? lo : 0u;
}

// bf16 fragment of part `part` of eight float32 activations.
__device__ inline uint4 split_frag(uint4 u, uint4 v, int part) {
    uint4 r;
    r.x = split_part(__uint_as_float(u.x), part) | (split_part(__uint_as_float(u.y), part) << 16);
    r.y = split_part(__uint_as_float(u.z), part) | (split_part(__uint_as_float(u.w), part) << 16);
    r.z = split_part(__uint_as_float(v.x), part) | (split_part(__uint_as_float(v.y), part) << 16);
    r.w = split_part(__uint_as_float(v.z), part) | (split_part(__uint_as_float(v.w), part) << 16);
    return r;
}

// Loads of one 128-wide group: the codes, scale and zero byte of NB tiles and
// the raw activation fragments of MT M tiles (bf16: one 16-byte load per k
// step; float32: two).
// AM: activation mode -- 0 bf16 rows, 1 float32 rows (split into bf16 terms),
// 2 int8 rows in operand order (W4A8; 32 bytes per lane per block), 3 fp16
// rows with a per-row power of two (prep_rows), 4 bf16 rows that each
// workgroup first converts into LDS as fp16 rows with a per-row power of two
// (few short rows: the whole activation matrix fits in LDS), 5 bf16 rows as in
// mode 0, loaded row-major (16 lanes per row, four rows per load, full cache
// lines) and put in operand order through 4 KiB of LDS per wave: a load in
// operand order touches 64 bytes of each of 16 rows.
template <int NB, int MT, int AM, int H>
struct Stage {
    uint4 cw[NB];
    uint32_t sc[H][(NB + 1) / 2];   // per half: binary16 scales of tiles 2i, 2i+1 in dword i
    uint32_t zb[H];                 // per half: zero of tile nb in nibble nb (+ the slot offset)
    uint4 af[MT][AM == 2 ? 2 : AM == 4 ? 1 : 4][AM == 1 ? 2 : 1];
    uint32_t ag;                    // AM 4: byte offset of the step's block in an LDS row
};



// Waves per SIMD the register allocation must allow: four for the grouped
// gate/up and down GEMMs of the MoE decode (a quad of tiles, one M tile, fp16
// rows from prep_rows).  With 64-wide groups, or with the bf16 rows converted in
// registers, they need more registers than four waves allow: no cap there (a
// cap made the converting kernel spill and run slower).
template <int NB, int MT, int AM, int EPI, int H>
constexpr int kMinWaves = (AM == 3 && MT == 1 && NB == 4 && H == 1) ? 4 : 1;

// H = 2: 64-wide groups, two scales and zeros per 128-wide block.
// WB: each wave streams its own tile blocks over the whole K and stores its
// results from registers (no reduction across waves; fp16 rows, one part per
// slot); otherwise the waves of a workgroup split K and reduce through LDS.
template <int NB, int MT, int AM, int S, int EPI, int H, bool WB = false>
__global__ void __launch_bounds__(kMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(kMinWaves<NB, MT, AM, EPI, H>)))
qgemm_kernel(const GemmArgs args) {
    constexpr bool AF32 = AM == 1, AI8 = AM == 2, AF16 = AM == 3, ALDS = AM == 4;
    static_assert(!WB || AF16, "wave-owned blocks: fp16 rows only");
    __shared__ float red[kRedSlotsFor<NB, MT> * 256];
    // AM 4: [rows][lda] fp16 activation rows, 16 zero bytes, float
    // [lda / 128][rows padded to 16] (each block's factor; lds_act_bytes)
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int W = blockDim.x >> 6;
    const int r16 = lane & 15;   // operand row / output column within the tile
    const int j = lane >> 4;     // k quarter of the operand, row block of the result

    // ---- which problem this workgroup serves
    const uint8_t *w;
    int64_t row0, n, src0 = 0;
    const int32_t *gather = nullptr;
    if (!args.moe) {
        // one dense problem; with m_rows, grid.y splits its rows
        w = args.w;
        row0 = args.m_rows > 0 ? (int64_t)blockIdx.y * args.m_rows : 0;
        n = args.m_rows > 0 && args.T - row0 > args.m_rows ? args.m_rows : args.T - row0;
        src0 = row0;
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
            // shared expert: problem py - routed_slots takes its shared_rows
            // slots starting there
            w = args.w_shared;
            const int64_t sr = args.shared_rows > 0 ? args.shared_rows : args.T;
            const int64_t cs = (int64_t)(py - args.routed_slots) * sr;
            row0 = args.T * args.top_k + cs;
            n = args.T - cs < sr ? args.T - cs : sr;
            src0 = args.gather_tokens ? cs : row0;
        }
    }
    if (n <= 0) return;

    const PackedLayout L(args.N, args.K, args.flags, args.group_size);
    const int64_t nt = L.nt, G = L.G;
    // Tile blocks of this workgroup: R consecutive blocks of NB tiles, streamed
    // back to back through one register pipeline, so a block's first loads are
    // in flight while the previous block is reduced and stored, and the
    // problem lookup above is paid once per R blocks.
    const int R = WB ? 1 : args.blocks_per_wg;   // (WB: one block per wave)
    const int64_t owner = WB ? (int64_t)blockIdx.x * W + wave : (int64_t)blockIdx.x;
    const int64_t tile0 = owner * R * NB;
    const int64_t nblk_all = (nt + NB - 1) / NB;
    const int64_t blk0 = owner * R;
    const int nblk = (int)(nblk_all - blk0 < R ? nblk_all - blk0 : R);
    if (WB && nblk <= 0) return;   // (no barriers on this path)
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)L.bytes);
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(args.a, (uint32_t)args.a_bytes);

    // Weight offsets: the lane part is the same for every tile and group; the
    // tile and group part is wave-uniform and goes in soffset.
    const uint32_t vc = (uint32_t)lane * 16u, vs = (uint32_t)r16 * 8u, vz = (uint32_t)r16 * 2u;

    // The waves split the groups; every wave runs the same number of steps per
    // block (ngp, a multiple of S) so that all reach each block's reduction
    // together.  Steps past a wave's range load out-of-range offsets (zero
    // codes, scales and activations), so computing them adds exactly 0.
    const int gb = WB ? 0 : (int)((G * wave) / W), ge = WB ? (int)G : (int)((G * (wave + 1)) / W);
    const int ngp = WB ? (((int)G + S - 1) / S) * S : (((int)((G + W - 1) / W) + S - 1) / S) * S;
    const int steps = nblk * ngp;
    const int P = args.P;                   // 1, 2 or 4
    const int plog = P == 4 ? 2 : P == 2 ? 1 : 0;
    const int spt = 16 >> plog;             // slots per M tile
    const int64_t chunk = (int64_t)MT * spt;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    constexpr int ES = AF32 ? 4 : AI8 ? 1 : 2;   // bytes per activation element
    // source row of A (a token when gathering, else a slot) of a problem slot
    auto src_row = [&](int64_t slot) -> int64_t {
        if (!gather) return src0 + slot;
        const uint32_t pr = (uint32_t)gather[row0 + slot];
        return args.top_k == 1 ? pr : __umulhi(pr, args.topk_magic);
    };

    // AM 4: the n activation rows (bf16) once into LDS as fp16 rows, each
    // 128-wide block of a row with its own power of two (the conversion of the
    // rows converted in registers, bf16_to_f16_scaled: the block's largest
    // magnitude lands in [2^14, 2^15), columns k = 2, 3, 6, 7 (mod 8) a further
    // 2^-4, as the weight operands there are 16x), and the block's factor
    // 2^(c - 112) as a float in fac[block][row] (rows padded to 16, padding 0).
    // The 16 chunks of 8 values of a block are held by 16 consecutive lanes,
    // which find the block's maximum among themselves; no barrier until the end.
    // Called once the first weight loads are in flight.
    const int64_t xrow_bytes = args.lda * 2;
    const uint32_t zoff = (uint32_t)(n * xrow_bytes);
    const int64_t fpad = (n + 15) & ~int64_t(15);   // rows of fac per block
    float *const fac = reinterpret_cast<float *>(xlds + zoff + 16);
    auto fill_lds = [&]() {
        const int64_t cpr = args.lda / 8, nch = n * cpr;   // (nch a multiple of 16)
        for (int64_t i = threadIdx.x; i < (args.lda / 128) * (fpad - n); i += blockDim.x)
            fac[(i / (fpad - n)) * fpad + n + i % (fpad - n)] = 0.f;
        if (threadIdx.x < 4) reinterpret_cast<uint32_t *>(xlds + zoff)[threadIdx.x] = 0u;
        const uint16_t *xg = static_cast<const uint16_t *>(args.a);
        for (int64_t b0 = 0; b0 < nch; b0 += 2 * (int64_t)blockDim.x) {   // (uniform)
            uint4 v[2];
            int64_t cu[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                cu[u] = b0 + u * (int64_t)blockDim.x + threadIdx.x;
                const int64_t r = cu[u] / cpr;
                v[u] = cu[u] < nch ? *reinterpret_cast<const uint4 *>(xg + r * args.lda + 8 * (cu[u] - r * cpr))
                                   : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t mx = pk_max_u16(pk_max_u16(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                         pk_max_u16(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu));
                mx = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {   // every lane of the wave takes part
                    const uint32_t t = (uint32_t)__shfl_xor((int)mx, o);
                    mx = t > mx ? t : mx;
                }
                const uint32_t E = mx >> 7, c = E > 29u ? E - 29u : 0u;
                if (cu[u] < nch) {
                    const int64_t r = cu[u] / cpr, k8 = 8 * (cu[u] - r * cpr);
                    *reinterpret_cast<f16x8 *>(xlds + r * xrow_bytes + 2 * k8) =
                        bf16_to_f16_scaled(v[u], (c << 7) * 0x00010001u, ((c + 4) << 7) * 0x00010001u);
                    if ((cu[u] & 15) == 0) fac[(k8 >> 7) * fpad + r] = __int_as_float((int)((c + 15u) << 23));
                }
            }
        }
        __syncthreads();
    };

    for (int64_t c0 = 0; c0 < n; c0 += chunk) {
        // M tiles of this chunk that hold at least one slot (uniform per workgroup)
        const int64_t mt_left = (n - c0 + spt - 1) >> (4 - plog);
        const int m_used = (int)(mt_left < MT ? mt_left : MT);

        f32x4 res[MT][NB];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) res[m][nb] = zero4;

        // S register stages: while one step is multiplied, the loads of the
        // next S - 1 steps are in flight.
        Stage<NB, MT, AM, H> st[S];
        uint32_t abase[MT];
        uint32_t acol[MT][4];   // AM 5: the lane's row-major chunk of each load (see load_a)
        int apart[MT];
        // Load cursor (wave-uniform): block lr, step li of that block, and the
        // byte offsets of that step's codes (first tile of the block), scale and
        // zero records, and activation group.  Offsets advance by a constant
        // per step and are re-based once per block.
        const uint32_t tstride = (uint32_t)G * kTileGroupBytes;   // next tile, same group
        int lr = 0, li = 0;
        uint32_t loc = 0, los = 0, loz = 0, loa = 0;
        int lnt = 0;   // tiles of block lr inside the matrix (0..NB)
        const int ash = args.a_shift;
        auto rebase = [&]() {
            const int64_t tile = tile0 + (int64_t)lr * NB;
            const uint32_t slot = (uint32_t)(tile & (kQuadTiles - 1));
            loc = (uint32_t)((tile * G + gb) * kTileGroupBytes);
            los = (uint32_t)L.scale_rec(tile, gb) + 2u * slot;
            loz = (uint32_t)L.zero_rec(tile, gb) + (slot >> 1);
            loa = (uint32_t)(gb >> ash) * 128u * ES;
            lnt = lr < nblk ? (int)(nt - tile < NB ? nt - tile : NB) : 0;
        };
        // The codes are read once per call: non-temporal loads, except in
        // activation mode 5, where the M tiles of a tile block run in
        // workgroups gx apart in dispatch order (on one XCD when gx is a
        // multiple of 8), so the later ones can find the codes in the L2
        // (13824 -> 5120 at T = 32: 35.8 -> 34.2 us, 5120 -> 13824 26.1 ->
        // 24.8 us).
        auto load_w = [&](Stage<NB, MT, AM, H> &q) {
            const bool in = lnt > 0 && gb + li < ge;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                q.cw[nb] = AM == 5 ? buf_b128(wr, vc, in && nb < lnt ? loc + nb * tstride : kOobS)
                                   : buf_b128_stream(wr, vc, in && nb < lnt ? loc + nb * tstride : kOobS);
#pragma unroll
            for (int h = 0; h < H; ++h)
                load_meta<NB>(wr, vs, vz, in ? los + h * kQuadScaleBytes : kOobS,
                              in ? loz + h * kQuadZeroBytes : kOobS, q.sc[h], q.zb[h]);
        };
        auto load_a = [&](Stage<NB, MT, AM, H> &q) {
            const bool in = lnt > 0 && gb + li < ge;
            if constexpr (ALDS) {   // the rows are in LDS: only the block offset
                q.ag = in ? loa : 0u;
                return;
            }
            const uint32_t oa = in ? loa : kOobS;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if constexpr (AM == 5) {
                    // row-major: 16 lanes read one row's 256 bytes of the block,
                    // a load covers four rows (transposed in compute)
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) q.af[m][s4][0] = buf_b128(ar, acol[m][s4], oa);
                } else if constexpr (AI8) {
                    q.af[m][0][0] = buf_b128(ar, abase[m], oa);
                    q.af[m][1][0] = buf_b128(ar, abase[m] + 16u, oa);
                } else {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        q.af[m][s4][0] = buf_b128(ar, abase[m] + 32u * s4 * ES, oa);
                        if constexpr (AF32) q.af[m][s4][AF32 ? 1 : 0] = buf_b128(ar, abase[m] + 32u * s4 * ES + 16, oa);
                    }
                }
            }
        };
        auto advance = [&]() {
            loc += kTileGroupBytes;
            los += H * kQuadScaleBytes;
            loz += H * kQuadZeroBytes;
            // the next block reads the next activation block (8-bit planes:
            // after each odd block)
            if (((gb + li) | (ash ^ 1)) & 1) loa += 128u * ES;
            if (++li == ngp) {
                li = 0;
                ++lr;
                rebase();
            }
        };
        auto compute = [&](const Stage<NB, MT, AM, H> &q, int zshift) {
          if constexpr (AI8) {
            // W4A8: codes as int8 operands (no offset), exact int32 sums per
            // block; acc - xz = sum_k a * (q - zero) exactly, then the scale.
            // The k order inside a lane's 16 bytes is the one the activation
            // quantizer writes: low nibbles of a dword (k offsets 0, 4, 1, 5),
            // then its high nibbles (2, 6, 3, 7), dwords s = 2kk, 2kk + 1.
            const i32x4 zero_i = {0, 0, 0, 0};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint4 d = q.cw[nb];
                const uint32_t mk = 0x0F0F0F0Fu;
                const i32x4 b0 = {(int)(d.x & mk), (int)((d.x >> 4) & mk), (int)(d.y & mk),
                                  (int)((d.y >> 4) & mk)};
                const i32x4 b1 = {(int)(d.z & mk), (int)((d.z >> 4) & mk), (int)(d.w & mk),
                                  (int)((d.w >> 4) & mk)};
                i32x4 bz[H];
                float sc[H];
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const int zz = (int)(((q.zb[h] >> (zshift + 4 * nb)) & 15u) * 0x01010101u);
                    bz[h] = i32x4{zz, zz, zz, zz};
                    sc[h] = f16_bits_to_f32((uint16_t)(q.sc[h][nb >> 1] >> (16 * (nb & 1))));
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= m_used) break;
                    const i32x4 a0 = __builtin_bit_cast(i32x4, q.af[m][0][0]);
                    const i32x4 a1 = __builtin_bit_cast(i32x4, q.af[m][1][0]);
                    if constexpr (H == 1) {
                        i32x4 acc = mfma_i8(a0, b0, zero_i);
                        i32x4 xz = mfma_i8(a0, bz[0], zero_i);
                        acc = mfma_i8(a1, b1, acc);
                        xz = mfma_i8(a1, bz[0], xz);
#pragma unroll
                        for (int v = 0; v < 4; ++v) res[m][nb][v] += sc[0] * (float)(acc[v] - xz[v]);
                    } else {
                        const i32x4 acc0 = mfma_i8(a0, b0, zero_i), xz0 = mfma_i8(a0, bz[0], zero_i);
                        const i32x4 acc1 = mfma_i8(a1, b1, zero_i), xz1 = mfma_i8(a1, bz[H - 1], zero_i);
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            res[m][nb][v] += sc[0] * (float)(acc0[v] - xz0[v]) +
                                             sc[H - 1] * (float)(acc1[v] - xz1[v]);
                    }
                }
            }
          } else {
            // Exact operands: the codes as fp16 q - zero (16x at k-offsets 2, 3,
            // 6, 7), the activation rows as fp16 times a power of two: one per
            // (row, block) converted here from bf16 (qi4_dev.h) or by the
            // workgroup into LDS (AM 4), or one per row from prep_rows (AM 3,
            // applied at the store).  The products are
            // exact and a code on its zero point adds exactly 0.  One MFMA chain
            // per tile and block (two with 64-wide groups), then the scale (times
            // 2^(c - 112) for the blocks converted here) per output row.
            const uint32_t magic = f16_magic_pair();
            uint4 raw[MT][4];
            if constexpr (AM == 5) {
                // the row-major chunks through this wave's 4 KiB of LDS per M
                // tile into operand order (lane 16 j + r: row r, bytes 64 s +
                // 16 j of the block for k step s).  Chunk c of row r sits at
                // 16 (c ^ r) of the row's 256 bytes, so that the 16 lanes of a
                // write (one row) and of a read (one chunk of 16 rows) touch
                // 16 different 16-byte bank groups.  One wave's LDS operations
                // run in order; the fences keep the compiler from moving them.
                uint8_t *tw = xlds + (uint32_t)(wave * MT * kA5TransposeBytes);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= m_used) break;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int rw = (lane >> 4) + 4 * s4;
                        *reinterpret_cast<uint4 *>(tw + m * kA5TransposeBytes + rw * 256 + 16 * ((lane & 15) ^ rw)) =
                            q.af[m][s4][0];
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= m_used) break;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        raw[m][s4] = *reinterpret_cast<const uint4 *>(
                            tw + m * kA5TransposeBytes + r16 * 256 + 16 * ((4 * s4 + j) ^ r16));
                }
            }
            uint32_t cc[MT], cc4[MT];
            float f[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (AF16 || ALDS || m >= m_used) break;
                if constexpr (AF32) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        raw[m][s4] = split_frag(q.af[m][s4][0], q.af[m][s4][1], apart[m]);
                } else if constexpr (AM == 0) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) raw[m][s4] = q.af[m][s4][0];
                }
                const uint32_t c = row_block_offset(bf16_absmax_bits(raw[m]));
                cc[m] = (c << 7) * 0x00010001u;
                cc4[m] = ((c + 4) << 7) * 0x00010001u;
                // 2^(c - 112) of the rows this lane's results belong to: result
                // register v of lane 16 j + col is operand row 4 j + v
                const int fb = (int)((c + 15u) << 23);
#pragma unroll
                for (int v = 0; v < 4; ++v) f[m][v] = __int_as_float(__shfl(fb, 4 * j + v));
            }
            if constexpr (ALDS) {
                // the block factors of this lane's result rows 4 j .. 4 j + 3
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= m_used) break;
                    const float4 t = *reinterpret_cast<const float4 *>(
                        fac + (int64_t)(q.ag >> 8) * fpad + c0 + m * spt + 4 * j);
                    f[m][0] = t.x;
                    f[m][1] = t.y;
                    f[m][2] = t.z;
                    f[m][3] = t.w;
                }
            }
            // activation operands of the 4 k steps, shared by the tiles
            f16x8 a[MT][4];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m >= m_used) break;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    a[m][s] = ALDS ? *reinterpret_cast<const f16x8 *>(
                                         xlds + (abase[m] != kOob ? abase[m] + q.ag + 64u * s : zoff))
                            : AF16 ? __builtin_bit_cast(f16x8, q.af[m][s][0])
                                   : bf16_to_f16_scaled(raw[m][s], cc[m], cc4[m]);
            }
            // tile by tile: one accumulator (per M tile and half) live at a time
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc[MT][H];
                uint32_t negz[H], negz16[H];
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const uint32_t z = (q.zb[h] >> (zshift + 4 * nb)) & 15u;
                    negz[h] = f16_negz(z);
                    negz16[h] = f16_negz16(z);
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[m][h] = zero4;
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int h = H == 2 ? s >> 1 : 0;   // 64-wide groups: k steps 0, 1 / 2, 3
                    const uint32_t d = s == 0 ? q.cw[nb].x : s == 1 ? q.cw[nb].y : s == 2 ? q.cw[nb].z : q.cw[nb].w;
                    const f16x8 b = __builtin_bit_cast(f16x8, codes_minus_zero_f16(d, negz[h], negz16[h], magic));
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        if (m >= m_used) break;
                        acc[m][h] = mfma16x16x32_f16(a[m][s], b, acc[m][h]);
                    }
                }
                const float s0 = f16_bits_to_f32((uint16_t)(q.sc[0][nb >> 1] >> (16 * (nb & 1))));
                const float s1 = f16_bits_to_f32((uint16_t)(q.sc[H - 1][nb >> 1] >> (16 * (nb & 1))));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= m_used) break;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float g = s0 * acc[m][0][v];
                        if constexpr (H == 2) g += s1 * acc[m][H - 1][v];
                        if constexpr (AF16) res[m][nb][v] += g;
                        else res[m][nb][v] += f[m][v] * g;
                    }
                }
            }
          }
        };

        // ---- reduction of the waves' partial sums of block r in a fixed
        // order, epilogue and store
        auto finish_block = [&](int r) {
          if constexpr (!WB) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[((wave * MT + m) * NB + nb) * 256 + v * 64 + lane] = res[m][nb][v];
            __syncthreads();
          }

            const int64_t tile_b = tile0 + (int64_t)r * NB;
            const int pairs = EPI == QI4_EPI_SILU_MUL ? NB / 2 : NB;
            auto store = [&](int64_t slot, int64_t oc, float val, float uval) {
                if constexpr (AI8) {   // the activations' scale
                    val *= args.a_scale;
                    uval *= args.a_scale;
                }
                if constexpr (AF16) {   // the row's power of two
                    const int e = args.a_exp[src_row(slot)];
                    val = ldexpf(val, e);
                    uval = ldexpf(uval, e);
                }
                if (EPI == QI4_EPI_SILU_MUL) val = val / (1.0f + expf(-val)) * uval;
                const int64_t dst = row0 + slot;
                if (args.out_mode == OUT_F32) {
                    static_cast<float *>(args.out)[dst * args.ldo + oc] = val;
                } else if (args.out_mode == OUT_BF16) {
                    static_cast<uint16_t *>(args.out)[dst * args.ldo + oc] = (uint16_t)f32_to_bf16_rne(val);
                } else if (AI8 && args.out_mode == OUT_I8) {   // (int8 rows only from W4A8)
                    // the activation quantizer's decision and byte order (k offset e
                    // of a dword at 2 (e & 3) + (e >> 2))
                    const float qv = fminf(fmaxf(rintf(val * args.out_r), -127.0f), 127.0f);
                    const int64_t pos = (oc & ~int64_t(127)) + 32 * ((oc >> 3) & 3) +
                                        8 * ((oc >> 5) & 3) + 2 * (oc & 3) + ((oc >> 2) & 1);
                    static_cast<int8_t *>(args.out)[dst * args.ldo + pos] = (int8_t)(int)qv;
                } else {
                    const uint32_t hi = f32_to_bf16_rne(val);
                    const uint32_t lo = f32_to_bf16_rne(val - bf16_to_f32(hi));
                    uint16_t *o = static_cast<uint16_t *>(args.out);
                    o[(dst * 2) * args.ldo + oc] = (uint16_t)hi;
                    o[(dst * 2 + 1) * args.ldo + oc] = (uint16_t)lo;
                }
            };
            auto out_col = [&](int nbA, int col) -> int64_t {
                const int64_t tile = tile_b + nbA;
                if (EPI == QI4_EPI_SILU_MUL) return (tile >> 1) * 16 + col;
                return tile < nt ? tile_row(tile, col, args.N, args.flags) : -1;
            };
            if constexpr (WB) {
                // this wave's results, straight from its registers: lane
                // 16 j + col holds rows 4 j + v of column col of each tile
                // (one part per slot).  The column index passes through an
                // empty asm statement, so the compiler computes the store
                // addresses here rather than holding them across the loop.
                int col = r16;
                __asm__ volatile("" : "+v"(col));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
#pragma unroll
                    for (int pi = 0; pi < pairs; ++pi) {
                        const int nbA = EPI == QI4_EPI_SILU_MUL ? 2 * pi : pi;
                        const int64_t oc = out_col(nbA, col);
                        if (oc < 0 || oc >= args.n_out) continue;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int64_t slot = c0 + (int64_t)m * 16 + 4 * j + v;
                            if (slot >= n) continue;
                            store(slot, oc, res[m][nbA][v],
                                  EPI == QI4_EPI_SILU_MUL ? res[m][EPI == QI4_EPI_SILU_MUL ? nbA + 1 : nbA][v] : 0.f);
                        }
                    }
                }
            } else if constexpr (NB == 4) {
                // grouped expert GEMMs: one thread per result lane, its four rows
                // together (the register budget of these kernels is tight)
                const int items = MT * pairs * 64;
                for (int it = threadIdx.x; it < items; it += blockDim.x) {
                    const int l = it & 63;
                    const int rest = it >> 6;
                    const int pi = rest % pairs;
                    const int m = rest / pairs;
                    const int nbA = EPI == QI4_EPI_SILU_MUL ? 2 * pi : pi;
                    float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int ww = 0; ww < W; ++ww) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            a4[v] += red[((ww * MT + m) * NB + nbA) * 256 + v * 64 + l];
                            if (EPI == QI4_EPI_SILU_MUL)
                                b4[v] += red[((ww * MT + m) * NB + nbA + 1) * 256 + v * 64 + l];
                        }
                    }
                    const int64_t oc = out_col(nbA, l & 15);
                    if (oc < 0 || oc >= args.n_out) continue;
                    const int rbase = 4 * (l >> 4);
                    // (static register indices: v0 and p are unrolled, P is 1, 2 or 4)
#pragma unroll
                    for (int v0 = 0; v0 < 4; ++v0) {
                        if ((v0 & (P - 1)) != 0) continue;
                        const int64_t slot = c0 + (int64_t)m * spt + ((rbase + v0) >> plog);
                        if (((rbase + v0) >> plog) >= spt || slot >= n) continue;
                        float val = 0.f, uval = 0.f;
#pragma unroll
                        for (int p = 0; v0 + p < 4; ++p) {
                            if (p >= P) break;
                            val += a4[v0 + p];
                            uval += b4[v0 + p];
                        }
                        store(slot, oc, val, uval);
                    }
                }
            } else {
            // one thread per output element (M tile, tile or gate/up pair, slot,
            // column); slots past the end are skipped before any LDS read.  The
            // sums run over the waves, then over a slot's P parts.
            const int items = MT * pairs * spt * 16;
            for (int it = threadIdx.x; it < items; it += blockDim.x) {
                const int col = it & 15;
                int rest = it >> 4;
                const int sq = rest & (spt - 1);
                rest >>= 4 - plog;
                const int pi = rest % pairs;
                const int m = rest / pairs;
                const int64_t slot = c0 + (int64_t)m * spt + sq;
                if (slot >= n) continue;
                const int nbA = EPI == QI4_EPI_SILU_MUL ? 2 * pi : pi;
                const int64_t oc = out_col(nbA, col);
                if (oc < 0 || oc >= args.n_out) continue;
                const float *ra = red + ((m * NB + nbA) * 256);
                float val = 0.f, uval = 0.f;
                for (int p = 0; p < P; ++p) {
                    const int rr = sq * P + p;   // result row: register rr & 3 of lane group rr >> 2
                    const int idx = (rr & 3) * 64 + 16 * (rr >> 2) + col;
                    float a = 0.f, b = 0.f;
                    for (int ww = 0; ww < W; ++ww) {
                        a += ra[ww * MT * NB * 256 + idx];
                        if (EPI == QI4_EPI_SILU_MUL) b += ra[ww * MT * NB * 256 + 256 + idx];
                    }
                    val += a;
                    uval += b;
                }
                store(slot, oc, val, uval);
            }
            }
            if constexpr (!WB) __syncthreads();
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) res[m][nb] = zero4;
        };

        // weights first: they come from HBM; the activation rows need the
        // slot -> row lookups, and come from cache
        rebase();
#pragma unroll
        for (int q = 0; q < S; ++q) {
            load_w(st[q]);
            advance();
        }
        if constexpr (ALDS) {
            if (c0 == 0) fill_lds();
        }
        // ---- byte offset of this lane's activation row (operand row r16 of each M tile)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int64_t slot = c0 + (int64_t)m * spt + (r16 >> plog);
            const int part = r16 & (P - 1);
            const bool ok = (r16 < spt * P) && slot < n;
            const int64_t slot_c = ok ? slot : 0;
            const int64_t src = src_row(slot_c);
            const int64_t row = AF32 ? src : src * P + part;
            apart[m] = part;
            // (int8 rows: a lane's 32 bytes of a block sit at 32 j; AM 4: an
            // offset into the LDS rows)
            abase[m] = ok ? (uint32_t)(row * args.lda * ES + (AI8 ? 32 * j : 8 * j * ES)) : kOob;
            if constexpr (AM == 5) {   // (one part per slot) rows (lane >> 4) + 4 s4 of the tile
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int64_t sl = c0 + (int64_t)m * spt + (lane >> 4) + 4 * s4;
                    acol[m][s4] = sl < n ? (uint32_t)(src_row(sl) * args.lda * 2 + 16 * (lane & 15)) : kOob;
                }
            }
        }
        lr = 0;
        li = 0;
        rebase();
#pragma unroll
        for (int q = 0; q < S; ++q) {
            load_a(st[q]);
            advance();
        }
        // (lr, li) now points S steps ahead of the step being computed, which
        // is step ci of block cr
        int cr = 0, ci = 0;
        for (int s0 = 0; s0 < steps; s0 += S) {
            const int zshift = NB == 1 ? 4 * (int)((tile0 + (int64_t)cr * NB) & 1) : 0;
#pragma unroll
            for (int q = 0; q < S; ++q) {
                compute(st[q], zshift);
                // the refill of this stage is issued after its compute: hoisting
                // the loads above it would keep both copies live
                __builtin_amdgcn_sched_barrier(0);
                load_w(st[q]);
                load_a(st[q]);
                advance();
            }
            ci += S;   // S divides ngp: a block ends at an iteration boundary
            if (ci == ngp) {
                if constexpr (!WB) finish_block(cr);
                ci = 0;
                ++cr;
            }
        }
        // WB: the wave's one block, after its loop (kept out of the loop so that
        // the compiler does not hold the store addresses across it)
        if constexpr (WB) finish_block(0);
    }
}

// float32 activations (split into bf16 parts in registers) run on blocks of
// at most two tiles: their fragments take twice the registers.
template <int NB, int MT, int S, int H>
int launch_cfg_h(const GemmArgs &a, dim3 grid, int threads, hipStream_t st) {
    if (a.a_f32 && NB > 2) return QI4_ERR_UNSUPPORTED;
    // AM 4: the fp16 rows, 16 zero bytes and the block factors in dynamic LDS;
    // AM 5: 4 KiB per wave and M tile for the transposition
    const size_t dyn = a.a_lds ? (size_t)lds_act_bytes(a.T, a.lda) : 0;
    const size_t dyn5 = (size_t)(threads / 64) * MT * kA5TransposeBytes;
    if (a.epi == QI4_EPI_SILU_MUL) {
        if constexpr (NB % 2 == 0) {
            if (a.a_i8)
                qgemm_kernel<NB, MT, 2, S, QI4_EPI_SILU_MUL, H><<<grid, threads, 0, st>>>(a);
            else if (a.a_f16)
                qgemm_kernel<NB, MT, 3, S, QI4_EPI_SILU_MUL, H><<<grid, threads, 0, st>>>(a);
            else if (a.a_lds)
                qgemm_kernel<NB, MT, 4, S, QI4_EPI_SILU_MUL, H><<<grid, threads, dyn, st>>>(a);
            else if (NB <= 2 && a.a_f32)
                qgemm_kernel<NB <= 2 ? NB : 2, MT, 1, 2, QI4_EPI_SILU_MUL, H><<<grid, threads, 0, st>>>(a);
            else if (MT == 1 && a.a_tr)
                qgemm_kernel<NB, 1, 5, S, QI4_EPI_SILU_MUL, H><<<grid, threads, dyn5, st>>>(a);
            else
                qgemm_kernel<NB, MT, 0, S, QI4_EPI_SILU_MUL, H><<<grid, threads, 0, st>>>(a);
        } else {
            return QI4_ERR_UNSUPPORTED;
        }
    } else if (a.a_i8) {
        qgemm_kernel<NB, MT, 2, S, QI4_EPI_NONE, H><<<grid, threads, 0, st>>>(a);
    } else if (a.a_f16) {
        qgemm_kernel<NB, MT, 3, S, QI4_EPI_NONE, H><<<grid, threads, 0, st>>>(a);
    } else if (a.a_lds) {
        qgemm_kernel<NB, MT, 4, S, QI4_EPI_NONE, H><<<grid, threads, dyn, st>>>(a);
    } else if (NB <= 2 && a.a_f32) {
        qgemm_kernel<NB <= 2 ? NB : 2, MT, 1, 2, QI4_EPI_NONE, H><<<grid, threads, 0, st>>>(a);
    } else if (MT == 1 && a.a_tr) {
        qgemm_kernel<NB, 1, 5, S, QI4_EPI_NONE, H><<<grid, threads, dyn5, st>>>(a);
    } else {
        qgemm_kernel<NB, MT, 0, S, QI4_EPI_NONE, H><<<grid, threads, 0, st>>>(a);
    }
    return launch_status();
}

template <int NB, int MT, int S>
int launch_cfg(const GemmArgs &a, dim3 grid, int threads, hipStream_t st) {
    return halves_for(a.group_size) == 2 ? launch_cfg_h<NB, MT, S, 2>(a, grid, threads, st)
                                         : launch_cfg_h<NB, MT, S, 1>(a, grid, threads, st);
}

}  // namespace

// Launch shape, from sweeps on MI355X over the decode workloads (dense Llama-7B
// and 5120/13824 shapes, DeepSeek-V3-shaped experts at T = 1, 8, 32):
//  * W waves split K; about ten 128-wide groups per wave for a single matrix
//    (all eight waves for one row with one tile per workgroup);
//  * a single matrix takes NB = 2 tiles per workgroup (the gate/up pair)
//    unless it has fewer than 320 tiles and needs more workgroups (NB = 1);
//    from 9 rows on, a whole quad (NB = 4) when that still gives >= 192
//    workgroups: the activation fragments, re-read per block of tiles, are
//    then shared by four tiles (5120 -> 13824 at T = 32: 30.4 -> 23.7 us);
//    the grouped expert GEMMs take a whole quad (NB = 4); the down
//    projection with fp16 rows gives each wave a quad of its own over the
//    whole K once there are 3000 quads or more, else splits K over the waves
//    (two quads per workgroup, R = 2, from 12000 quads on);
//  * one M tile per pass (16 activation rows), two for a single matrix with
//    more rows.
int launch_qgemm(const GemmArgs &args, int n_problems, int64_t max_slots, hipStream_t st) {
    if (n_problems <= 0 || max_slots <= 0) return QI4_OK;
    const int64_t nt = num_tiles(args.N, args.flags);
    const int64_t G = args.K / kGroup;
    const int spt = 16 / args.P;
    // Expert problems mostly hold a few slots each: one M tile per pass keeps
    // registers low; a problem with more slots (the shared expert) takes more
    // passes.  A single matrix with more than 16 rows uses two M tiles.
    int MT = (n_problems == 1 && max_slots > spt) ? 2 : 1;
    const bool silu = args.epi == QI4_EPI_SILU_MUL;
    // (a single matrix takes two tiles per workgroup from 320 tiles up: cold-cache
    // sweeps of 4096..22016-row matrices put the crossover between 256 and 320)
    int NB = (silu || ceil_div(nt, 2) * n_problems >= 160) ? 2 : 1;
    int W, R = 1;   // R: tile blocks streamed back to back by one workgroup (or wave)
    bool wb = false;   // waves own tile blocks (qgemm_kernel's WB)
    if (n_problems > 1) {
        // grouped expert GEMMs: four tiles (one quad) per block; gate/up over
        // four waves; down as below
        NB = 4;
        if (silu) {
            W = 4;
        } else if (kDownWaveBlocks && args.a_f16 && args.P == 1 &&
                   ceil_div(nt, NB) * n_problems >= 3000) {
            // (fp16 rows) each wave streams a whole quad over K and stores it
            // without a reduction across waves, two waves per workgroup:
            // DeepSeek-V3 down at T = 32 5.41 -> 5.75 TB/s, T = 4 and 8
            // 1-2 % faster; fewer quads (T <= 2) keep K split over the waves
            W = 2;
            wb = true;
        } else if (ceil_div(nt, NB) * n_problems >= 12000) {
            W = 4;
            R = 2;
        } else {
            W = 2;
        }
    } else {
        // (W4A8 rows split over grid.y: a quad per workgroup down to 64 quads,
        // 13824 -> 5120 at T = 32 32.7 -> 28.8 us; bf16 rows there got slower)
        if (max_slots > 8 && !args.a_f32 &&
            (ceil_div(nt, 4) >= 192 || (args.a_i8 && max_slots > spt && ceil_div(nt, 4) >= 64)))
            NB = 4;
        W = 1;
        while (W < kMaxWaves && G / (2 * W) >= 8) W *= 2;
        // one row, one tile per workgroup: all eight waves (Llama-7B O
        // projection 4096 -> 4096: 10.6 -> 9.0 us cold; with two tiles per
        // workgroup the SiLU launch got slower)
        if (args.a_lds && max_slots == 1 && NB == 1) W = kMaxWaves;
    }
    // a dense matrix whose rows span two M tiles and whose activations are
    // converted in registers: one M tile per workgroup, grid.y over the M
    // tiles (twice the workgroups, each converting half the rows).  The
    // workgroups of one tile block are gx apart in dispatch order: on the same
    // XCD when gx is a multiple of 8, where the later ones find the weights in
    // that XCD's L2.
    int64_t gy = n_problems;
    GemmArgs a = args;
    a.m_rows = 0;
    a.a_tr = 0;
    if (!args.moe && MT == 2 && !args.a_lds && kDenseMSplit) {
        MT = 1;
        a.m_rows = spt;
        gy = ceil_div(max_slots, (int64_t)spt);
        // bf16 rows: loaded row-major and transposed through LDS (activation
        // mode 5; 13824 -> 5120 at T = 32: 42.7 -> 35.9 us, 8-bit codes 77.0 ->
        // 63.8 us).  Not below 17 rows: with one M tile of rows per call the
        // extra LDS round trip cost 1 us at T = 4 and 8.
        if (!a.a_f32 && !a.a_i8 && !a.a_f16) a.a_tr = 1;
    }
    while (W > 1 && W * MT * NB > red_slots(NB, MT)) W /= 2;
    // activation mode 5: the transposition buffers and the reduction buffer
    // within 64 KiB
    if (a.a_tr)
        while (W > 1 && W * MT * kA5TransposeBytes + red_slots(NB, MT) * 1024 > 65536) W /= 2;
    a.blocks_per_wg = R;
    // pair / top_k as a multiply-high: with m = floor((2^32 - 1) / k) + 1,
    // floor(p * m / 2^32) = floor(p / k) whenever p * k < 2^32 (pairs are below
    // 2^31 / 32 and top_k is at most 32); k = 1 (m = 2^32) is taken apart
    a.topk_magic = a.top_k > 1 ? (uint32_t)(0xFFFFFFFFull / (uint32_t)a.top_k + 1ull) : 0u;
    const int64_t gx = wb ? ceil_div(ceil_div(ceil_div(nt, NB), R), W) : ceil_div(ceil_div(nt, NB), R);
    if (gx > 0x7fffffff || gy > 65535) return QI4_ERR_SHAPE;
    dim3 grid((unsigned)gx, (unsigned)gy);
    const int threads = W * 64;
    if (wb) {
        if (halves_for(a.group_size) == 2)
            qgemm_kernel<4, 1, 3, 2, QI4_EPI_NONE, 2, true><<<grid, threads, 0, st>>>(a);
        else
            qgemm_kernel<4, 1, 3, 2, QI4_EPI_NONE, 1, true><<<grid, threads, 0, st>>>(a);
        return launch_status();
    }
    if (MT == 1) {
        if (NB == 4) return launch_cfg<4, 1, 2>(a, grid, threads, st);
        if (NB == 2) return launch_cfg<2, 1, 2>(a, grid, threads, st);
        return launch_cfg<1, 1, 2>(a, grid, threads, st);
    }
    if (NB == 4) return launch_cfg<4, 2, 2>(a, grid, threads, st);
    if (NB == 2) return launch_cfg<2, 2, 2>(a, grid, threads, st);
    return launch_cfg<1, 2, 2>(a, grid, threads, st);
}

}  // namespace qi4

using namespace qi4;

namespace {

// W4A8 activations: one thread per 8 consecutive values of a row, k0 = 128 b +
// 32 s + 8 j.  a = clamp(rint(x * r), -127, 127) with the float32 product (ties
// to even; NaN gives -127), stored at row * K + 128 b + 32 j + 8 s in the order
// of the weight operand's bytes: k0 + 0, 4, 1, 5, 2, 6, 3, 7.
template <bool F32>
__global__ void __launch_bounds__(256)
quantize_act_kernel(const void *__restrict__ x, int64_t T, int64_t K, float r,
                    uint8_t *__restrict__ out) {
    const int64_t chunks = T * K / 8, cpr = K / 8;
    for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
        const int64_t row = c / cpr, k0 = 8 * (c - row * cpr);
        float v[8];
        if constexpr (F32) {
            const float4 u0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + row * K + k0);
            const float4 u1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + row * K + k0 + 4);
            v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
            v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
        } else {
            const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + row * K + k0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
                v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
            }
        }
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = fminf(fmaxf(rintf(v[e] * r), -127.0f), 127.0f);
            b[e] = (uint32_t)(int)q & 0xFFu;
        }
        const uint32_t lo = b[0] | (b[4] << 8) | (b[1] << 16) | (b[5] << 24);
        const uint32_t hi = b[2] | (b[6] << 8) | (b[3] << 16) | (b[7] << 24);
        const int64_t kb = k0 & ~int64_t(127), s = (k0 >> 5) & 3, j = (k0 >> 3) & 3;
        *reinterpret_cast<uint2 *>(out + row * K + kb + 32 * j + 8 * s) = make_uint2(lo, hi);
    }
}

// W4A8 extras of a linear call: the activations' scale and the workspace that
// receives the int8 activations.
struct W4A8 {
    float scale;
    void *ws;
    int64_t ws_bytes;
};

// qlinear_int4 / qlinear_int8 (flags holds QI4_INT8 for the latter) /
// qlinear_w4a8 (w4a8 given).
int qlinear_impl(const void *x, int x_dtype, int64_t T, int64_t K, const void *packed_w,
                 int64_t N, int group_size, int flags, void *y, int y_dtype, int epilogue,
                 void *stream, const W4A8 *w4a8 = nullptr) {
    int rc = check_matrix(N, K, group_size, flags);
    if (rc) return rc;
    if (x_dtype != QI4_F32 && x_dtype != QI4_BF16) return QI4_ERR_DTYPE;
    if (y_dtype != QI4_F32 && y_dtype != QI4_BF16) return QI4_ERR_DTYPE;
    if (epilogue != QI4_EPI_NONE && epilogue != QI4_EPI_SILU_MUL) return QI4_ERR_DTYPE;
    if (epilogue == QI4_EPI_SILU_MUL && !(flags & QI4_PACK_GATEUP)) return QI4_ERR_UNSUPPORTED;
    if (T < 0 || T > (int64_t(1) << 31)) return QI4_ERR_SHAPE;
    if (T == 0) return QI4_OK;
    if (!x || !packed_w || !y) return QI4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed_w, 16) || !aligned(y, 4)) return QI4_ERR_SHAPE;
    const int64_t n_out = epilogue == QI4_EPI_SILU_MUL ? N / 2 : N;
    const int64_t xb = T * K * (x_dtype == QI4_F32 ? 4 : 2);
    const int64_t yb = T * n_out * (y_dtype == QI4_F32 ? 4 : 2);
    const int gs = (int)effective_group(group_size, K);
    const int64_t Kp = packed_k(K, flags);
    const int64_t wb = PackedLayout(N, Kp, flags, gs).bytes;
    if (wb >= (int64_t(1) << 31) || xb >= (int64_t(1) << 31)) return QI4_ERR_SHAPE;
    if (overlaps(y, yb, x, xb) || overlaps(y, yb, packed_w, wb)) return QI4_ERR_ALIAS;
    float r = 0.f;
    if (w4a8) {
        const float sx = w4a8->scale;
        r = 1.0f / sx;
        if (!(sx > 0.f) || !(sx < INFINITY) || !(r < INFINITY))   // finite, positive, finite 1/s
            return QI4_ERR_SHAPE;
        if (!w4a8->ws) return QI4_ERR_NULL;
        if (w4a8->ws_bytes < T * K) return QI4_ERR_WORKSPACE;
        if (!aligned(w4a8->ws, 16)) return QI4_ERR_SHAPE;
        if (overlaps(w4a8->ws, T * K, x, xb) || overlaps(w4a8->ws, T * K, y, yb) ||
            overlaps(w4a8->ws, T * K, packed_w, wb))
            return QI4_ERR_ALIAS;
    }
    if ((rc = check_device())) return rc;
    if (w4a8) {
        if ((rc = launch_quantize_act(x, x_dtype == QI4_F32, T, K, r,
                                      static_cast<uint8_t *>(w4a8->ws), as_stream(stream))))
            return rc;
    }

    GemmArgs a = {};
    a.w = static_cast<const uint8_t *>(packed_w);
    a.N = N;
    a.K = Kp;
    a.flags = flags;
    a.group_size = gs;
    a.a = x;
    a.lda = K;
    a.a_shift = (flags & QI4_INT8) ? 1 : 0;
    a.a_bytes = xb;
    a.a_f32 = x_dtype == QI4_F32;
    a.P = a.a_f32 ? 4 : 1;
    if (w4a8) {   // the GEMM reads the int8 rows
        a.a = w4a8->ws;
        a.a_bytes = T * K;
        a.a_f32 = 0;
        a.a_i8 = 1;
        a.a_scale = w4a8->scale;
        a.P = 1;
    }
    a.moe = 0;
    a.T = T;
    // few short bf16 rows: each workgroup converts them into LDS once
    if (!w4a8 && !a.a_f32 && T * K * 2 + 16 + 4 * T <= kLdsActBytes) a.a_lds = 1;
    a.out = y;
    a.ldo = n_out;
    a.out_mode = y_dtype == QI4_F32 ? OUT_F32 : OUT_BF16;
    a.epi = epilogue;
    a.n_out = n_out;
    return launch_qgemm(a, 1, T, as_stream(stream));
}

}  // namespace

extern "C" int qlinear_int4(const void *x, int x_dtype, int64_t T, int64_t K,
                            const void *packed_w, int64_t N, int group_size, int flags, void *y,
                            int y_dtype, int epilogue, void *stream) {
    if (flags & QI4_INT8) return QI4_ERR_UNSUPPORTED;   // an 8-bit matrix: qlinear_int8
    return qlinear_impl(x, x_dtype, T, K, packed_w, N, group_size, flags, y, y_dtype, epilogue,
                        stream);
}

extern "C" int qlinear_int8(const void *x, int x_dtype, int64_t T, int64_t K,
                            const void *packed_w, int64_t N, int group_size, int flags, void *y,
                            int y_dtype, int epilogue, void *stream) {
    return qlinear_impl(x, x_dtype, T, K, packed_w, N, group_size, flags | QI4_INT8, y, y_dtype,
                        epilogue, stream);
}

int qi4::launch_quantize_act(const void *x, int x_f32, int64_t T, int64_t K, float r,
                             uint8_t *out, hipStream_t st) {
    const int64_t chunks = T * K / 8;
    if (chunks <= 0) return QI4_OK;
    const unsigned g = (unsigned)(chunks / 256 + 1 < 65536 ? chunks / 256 + 1 : 65536);
    if (x_f32) quantize_act_kernel<true><<<g, 256, 0, st>>>(x, T, K, r, out);
    else quantize_act_kernel<false><<<g, 256, 0, st>>>(x, T, K, r, out);
    return launch_status();
}

extern "C" int64_t qlinear_w4a8_workspace_bytes(int64_t T, int64_t K) {
    if (T < 0 || K < 128 || K % 128 || T > (int64_t(1) << 31) || K > (int64_t(1) << 30))
        return QI4_ERR_SHAPE;
    return (T * K + 255) & ~int64_t(255);
}

extern "C" int qlinear_w4a8(const void *x, int x_dtype, float x_scale, int64_t T, int64_t K,
                            const void *packed_w, int64_t N, int group_size, int flags, void *y,
                            int y_dtype, int epilogue, void *workspace, int64_t ws_bytes,
                            void *stream) {
    if (flags & QI4_INT8) return QI4_ERR_UNSUPPORTED;   // 4-bit weights only
    const W4A8 w{x_scale, workspace, ws_bytes};
    return qlinear_impl(x, x_dtype, T, K, packed_w, N, group_size, flags, y, y_dtype, epilogue,
                        stream, &w);
}

extern "C" int qlinear_int4_g128(const void *x, int x_dtype, int64_t T, int64_t K,
                                 const void *packed_w, int64_t N, int flags, void *y,
                                 int y_dtype, int epilogue, void *stream) {
    return qlinear_int4(x, x_dtype, T, K, packed_w, N, 128, flags, y, y_dtype, epilogue, stream);
}
