// Prefill grouped GEMM (fp16 MFMA, LDS-staged activation tiles) and its helpers.
#pragma once

#include "qi4_dev.h"

namespace qi4 {

constexpr int kPrefillBM = 128;   // activation rows per workgroup tile

struct PrefillArgs {
    const uint8_t *w;          // routed expert 0 (packed), stride w_stride
    int64_t w_stride;
    const uint8_t *w_shared;   // shared expert or nullptr
    int64_t N, K;
    int flags;
    const uint16_t *a16;       // fp16 activation rows [a_rows][K]; value = a16 * 2^a_exp[row]
    int64_t a_rows;
    const int32_t *a_exp;
    int gather_tokens;         // rows of a16 are tokens (gate/up) or slots (down)
    const int32_t *sorted_pairs, *offsets, *active;
    int top_k;
    int64_t T;
    const int2 *tiles;         // (problem, first slot); problem -1 = shared expert
    const int32_t *tile_count;
    void *out;
    int64_t ldo;
    int epi;                   // SiLU(gate)*up -> hi/lo bf16 rows, or plain float32 rows
    int64_t n_out;
};

// rows of bf16 (src_kind 0) or hi/lo bf16 pairs (src_kind 1) -> fp16 rows and exponents
int launch_prep_rows(const void *src, int src_kind, int64_t rows, int64_t len, uint16_t *dst,
                     int32_t *exps, hipStream_t st);
int launch_plan(const int32_t *offsets, const int32_t *active, int64_t T, int has_shared,
                int2 *tiles, int32_t *count, hipStream_t st);
int64_t prefill_max_tiles(int64_t T, int top_k, int64_t E, int has_shared);
int launch_prefill(const PrefillArgs &a, int64_t max_tiles, hipStream_t st);

}  // namespace qi4
