// Row preparation shared by the kernels that turn activation rows into fp16
// with a per-row power-of-two prescale (the operands of the fp16 MFMA GEMMs).
#pragma once

#include "qi4_dev.h"

namespace qi4 {

// src_kind 0: bf16 rows [rows][len]; 1: hi/lo bf16 pairs [rows][2][len] (the
// value is hi + lo).  One workgroup of THREADS lanes per row: each thread loads
// its chunks of 8 consecutive elements (16-byte accesses) once into registers,
// the workgroup takes the row's largest magnitude, and the same registers are
// converted and stored, so a row costs one round trip to memory however long
// it is (rows of up to THREADS * 8 * kPrepChunks elements; longer rows run the
// loop below again from memory).  len is a multiple of 128, rows 16-byte
// aligned.  Output: dst[row] = fp16(v * 2^sh) with sh = 14 - E for the row's
// largest magnitude in [2^(E-1), 2^E) (so every |value| < 2^14), except that
// k = 2, 3, 6, 7 (mod 8) carry an extra 2^-4 (the decode and prefill weight
// operands hold 16 (q - z) there); exps[row] = -sh.  wmax: THREADS / 64 floats
// of LDS.  Every thread of the workgroup must call this (it holds a barrier).
constexpr int kPrepChunks = 8;

template <int THREADS>
__device__ inline void prep_row(const uint16_t *__restrict__ src, int src_kind, int64_t len,
                                int64_t row, uint16_t *__restrict__ dst,
                                int32_t *__restrict__ exps, float *wmax) {
    const int tid = threadIdx.x;
    const uint16_t *s = src + row * len * (src_kind ? 2 : 1);
    const int64_t nch = len / 8;
    auto load8 = [&](int64_t i, float (&v)[8]) {   // elements i .. i + 7
        const uint4 a = *reinterpret_cast<const uint4 *>(s + i);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            v[2 * c] = bf16_to_f32(w[c] & 0xFFFFu);
            v[2 * c + 1] = bf16_to_f32(w[c] >> 16);
        }
        if (src_kind) {
            const uint4 b = *reinterpret_cast<const uint4 *>(s + len + i);
            const uint32_t u[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                v[2 * c] += bf16_to_f32(u[c] & 0xFFFFu);
                v[2 * c + 1] += bf16_to_f32(u[c] >> 16);
            }
        }
    };
    float v[kPrepChunks][8];
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < kPrepChunks; ++q) {
        const int64_t ch = tid + (int64_t)q * THREADS;
        if (ch < nch) {
            load8(8 * ch, v[q]);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[q][e]));
        }
    }
    for (int64_t ch = tid + (int64_t)kPrepChunks * THREADS; ch < nch; ch += THREADS) {
        float w[8];
        load8(8 * ch, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(w[e]));
    }
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) mx = fmaxf(mx, wmax[w]);
    int E = 0;
    if (mx > 0.f) frexpf(mx, &E);          // mx in [2^(E-1), 2^E)
    const int sh = mx > 0.f ? 14 - E : 0;  // |v * 2^sh| < 2^14
    auto store8 = [&](int64_t i, const float (&w)[8]) {
        uint32_t o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int se = (c & 1) ? sh - 4 : sh;
            const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(w[2 * c], se));
            const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(w[2 * c + 1], se));
            o[c] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(dst + row * len + i) = make_uint4(o[0], o[1], o[2], o[3]);
    };
#pragma unroll
    for (int q = 0; q < kPrepChunks; ++q) {
        const int64_t ch = tid + (int64_t)q * THREADS;
        if (ch < nch) store8(8 * ch, v[q]);
    }
    for (int64_t ch = tid + (int64_t)kPrepChunks * THREADS; ch < nch; ch += THREADS) {
        float w[8];
        load8(8 * ch, w);
        store8(8 * ch, w);
    }
    if (tid == 0) exps[row] = -sh;
}

}  // namespace qi4
