// The int4-g128 GEMM core shared by the dense linear layer and the grouped
// expert GEMMs of the MoE FFN.
#pragma once

#include "qi4_dev.h"

namespace qi4 {

// OUT_I8: int8 rows in MFMA operand order (W4A8 h), q = clamp(rint(v * out_r))
enum OutMode { OUT_F32 = 0, OUT_BF16 = 1, OUT_SPLIT2 = 2, OUT_I8 = 3 };

// One launch computes out[dst(s)][n] = epi(sum_k A[src(s)][k] * W[n][k]) for the
// "slots" s of one or more problems (a problem = one weight matrix and the rows
// of A that use it).  blockIdx.y picks the problem, blockIdx.x a block of tiles.
struct GemmArgs {
    // weights (packed)
    const uint8_t *w;          // dense matrix, or routed expert 0 (each matrix < 2^31 bytes)
    int64_t w_stride;          // bytes between routed experts
    const uint8_t *w_shared;   // shared expert (moe) or nullptr
    int64_t N, K;              // rows and packed reduction length of each matrix
    int flags;                 // QI4_PACK_GATEUP or 0
    int group_size;            // quantization group size (64, or a multiple of 128)
    // activations
    const void *a;             // bf16 bits, or float32 when a_f32
    int64_t lda;               // elements per A source row
    int64_t a_bytes;           // bytes of the whole A buffer (< 2^31)
    int a_f32;                 // float32 rows, split into 4 bf16 terms in registers
    int a_i8;                  // int8 rows in MFMA operand order (W4A8), lda in bytes
    int a_f16;                 // fp16 rows from prep_rows: value = fp16 * 2^a_exp[row], with
                               // k = 2, 3, 6, 7 (mod 8) stored times 2^-4
    const int32_t *a_exp;      // a_f16: per-row exponent
    int a_lds;                 // bf16 rows converted into LDS by each workgroup (dense
                               // calls whose T * K * 2 bytes fit kLdsActBytes)
    int a_tr;                  // bf16 rows converted in registers, loaded row-major and
                               // put in operand order through LDS (set by the launch)
    float a_scale;             // W4A8: the activations' scale, applied at the store
    int P;                     // A rows per slot: parts summed at the end (1, 2 or 4)
    int a_shift;               // weight block b reads activation block b >> a_shift
                               // (1: an 8-bit matrix, two 4-bit planes per block)
    // problems
    int moe;                   // 0: one dense problem with T slots
    int64_t T;                 // tokens
    int top_k;
    uint32_t topk_magic;       // set by launch_qgemm: pair / top_k = umulhi(pair, topk_magic)
    const int32_t *sorted_pairs;  // moe gate/up: slot -> pair -> token
    const int32_t *offsets;       // moe: expert segment starts (E + 1)
    const int32_t *active;        // moe: [count, experts...]
    int routed_slots;             // moe: problem slots for routed experts in grid.y
    int shared_rows;              // moe: slots of each shared-expert problem (those after
                                  // the routed ones in grid.y); 0: all T in one
    int gather_tokens;            // moe: A rows are tokens (gate/up) rather than slots (down)
    // output
    void *out;
    int64_t ldo;               // elements per output row
    int out_mode;              // OutMode
    float out_r;               // OUT_I8: reciprocal of the output's int8 scale
    int epi;                   // QI4_EPI_NONE or QI4_EPI_SILU_MUL
    int64_t n_out;             // valid output columns
    // set by launch_qgemm
    int blocks_per_wg;         // consecutive tile blocks one workgroup streams
    int64_t m_rows;            // dense: rows per workgroup along grid.y (0: all T in one)
};

// Largest activation matrix (bytes of its fp16 rows) a dense call converts into
// LDS per workgroup; larger ones convert in registers per (row, block).
constexpr int64_t kLdsActBytes = 32 * 1024;

// Dynamic LDS of such a call: the fp16 rows, 16 zero bytes, and a float factor
// per (128-wide block, row), rows padded to a multiple of 16.
constexpr int64_t lds_act_bytes(int64_t T, int64_t lda) {
    return T * lda * 2 + 16 + (lda / 128) * ((T + 15) & ~int64_t(15)) * 4;
}

// Launch the GEMM for `n_problems` problems (grid.y); `max_slots` bounds the
// slots of any one problem and picks the M tiling.  Returns a QI4 status.
int launch_qgemm(const GemmArgs &args, int n_problems, int64_t max_slots, hipStream_t stream);

// W4A8 activations: rows x [T][K] (bf16, or float32 when x_f32) -> int8 rows in
// the operand order the AM = 2 GEMM reads, a = clamp(rint(x * r), -127, 127).
int launch_quantize_act(const void *x, int x_f32, int64_t T, int64_t K, float r, uint8_t *out,
                        hipStream_t stream);

}  // namespace qi4
