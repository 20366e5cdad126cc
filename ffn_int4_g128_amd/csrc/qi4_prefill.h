// Prefill grouped GEMM (fp16 MFMA, LDS-staged activation tiles) and its helpers.
#pragma once

#include "qi4_dev.h"

namespace qi4 {

constexpr int kPrefillBM = 128;       // activation rows of a big tile
constexpr int kPrefillBMSmall = 64;   // activation rows of a small tile

struct PrefillArgs {
    const uint8_t *w;          // routed expert 0 (packed), stride w_stride
    int64_t w_stride;
    const uint8_t *w_shared;   // shared expert or nullptr
    int64_t N, K;              // rows and packed reduction length of each matrix
    int a_shift;               // weight block b reads activation block b >> a_shift
                               // (1: 8-bit matrices, two 4-bit planes per block)
    int flags;
    int group_size;            // quantization group size (64, or a multiple of 128)
    const uint16_t *a16;       // fp16 activation rows [a_rows][K >> a_shift];
                               // value = a16 * 2^a_exp[row]
    int64_t a_rows;
    const int32_t *a_exp;
    int gather_tokens;         // rows of a16 are tokens (gate/up) or slots (down)
    const int32_t *sorted_pairs, *offsets, *active;
    int top_k;
    int64_t T;
    const int2 *tiles;         // big tiles [max_big], then 3 classes of small tiles [max_small]
                               // each: (problem, first slot), problem -1 = shared expert
    int64_t max_big, max_small;
    const int32_t *tile_count; // [0] big tiles, [1..3] small tiles by class, [4] deferred pairs
    int32_t *deferred_count;   // = tile_count + 4
    int4 *deferred;            // (problem, first slot, column block, 0) [max_deferred]
    int64_t max_deferred;
    void *out;
    int64_t ldo;
    int epi;                   // SiLU(gate)*up -> hi/lo bf16 rows, or plain float32 rows
    int64_t n_out;
};

// rows of bf16 (src_kind 0) or hi/lo bf16 pairs (src_kind 1) -> fp16 rows and exponents
int launch_prep_rows(const void *src, int src_kind, int64_t rows, int64_t len, uint16_t *dst,
                     int32_t *exps, hipStream_t st);
struct PrefillTiles {
    int64_t big, small;   // capacity of the big list and of each small-tile list
};
int launch_plan(const int32_t *offsets, const int32_t *active, int64_t T, int has_shared,
                int2 *tiles, const PrefillTiles &m, int32_t *counts, hipStream_t st);
PrefillTiles prefill_max_tiles(int64_t T, int top_k, int64_t E, int has_shared);
// capacity of the deferred list for an N-row matrix
int64_t prefill_max_deferred(int64_t N, int flags, const PrefillTiles &m);
int launch_prefill(const PrefillArgs &a, hipStream_t st);

}  // namespace qi4
