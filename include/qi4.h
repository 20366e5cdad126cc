/*
 * qi4.h -- C ABI of libqi4: int4 group-quantized (groups of 128 along K by
 * default, one binary16 scale and one 4-bit zero point per group) linear layer
 * and routed mixture-of-experts FFN for AMD MI355X (gfx950).
 *
 * What is computed follows these pages:
 *  - FastLLM: zero-dependency CPU inference framework (pgsm.cn), section 3.1
 *    (4-bit quantization and weight reordering): weights are 4-bit codes in
 *    groups of 128 sharing one scale and one zero point, kept group after group
 *    in memory so the product reads them contiguously, and each weight is
 *    dequantized on the fly inside the product rather than in a separate pass;
 *    section 2.3: the matrix multiply is a core operator below the model layer.
 *    Section 4.2 "model conversion and format": the group size defaults to 128;
 *    64 and 256 are allowed; codes are 4 or 8 bits wide (--quant-bit).
 *  - fastllm README (gittoolsai.com), "other parameters": --moe_experts sets
 *    how many routed experts each token uses; --cuda_se runs the shared expert
 *    on the GPU.  "Inference precision": int4g is the grouped int4 type, int4
 *    the plain one (read here as one scale and zero per row: group_size 0),
 *    int8 the 8-bit type (flag QI4_INT8 below).
 *  - FastLLM notes (wmrh.cn), part 1: a MoE layer holds many experts but each
 *    token activates only a few of them.
 * Dequantization is w = scale * (q - zero).  Expert FFN is
 * h = SiLU(x.Wg^T) * (x.Wu^T), y = h.Wd^T; SiLU(v) = v / (1 + e^-v).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Calls only enqueue work on `stream` and return; they never synchronize,
 *    never allocate and never free.  The caller owns every buffer.
 *  - Errors are return codes (QI4_OK == 0, negative on error).  All argument
 *    checks run on the host before anything is enqueued: on an error return
 *    nothing was launched and no output was touched.  A failed launch returns
 *    QI4_ERR_HIP.  No C++ exception crosses this ABI.
 *  - Outputs must not overlap inputs (QI4_ERR_ALIAS where checked).
 *  - group_size is 64, a multiple of 128 that divides K (256, ...), or 0 for one
 *    group per row (per-channel int4); anything else is QI4_ERR_GROUP, and a
 *    group size that does not divide K is QI4_ERR_SHAPE.  K must be a multiple
 *    of 128 (QI4_ERR_SHAPE).  A packed matrix is read with the group size it
 *    was packed with.  The device must be gfx950 (QI4_ERR_UNSUPPORTED
 *    otherwise).
 *  - Calls are reentrant.  The only global state is a cached per-device
 *    architecture check; every kernel of a call runs on `stream`.
 *
 * Canonical (interchange) format of a quantized matrix W [N][K] (out x in), with
 * Gs = group size (K when group_size is 0):
 *    qweight uint8  [N][K/2]    code of (n, k) in byte k/2, even k in the low nibble
 *    scales  uint16 [N][K/Gs]   IEEE binary16 bit patterns
 *    zeros   uint8  [N][K/Gs]   zero point, 0..15
 * A [gate; up] matrix of an FFN has N = 2*I rows: rows [0, I) gate, [I, 2I) up.
 * With the flag QI4_INT8 (8-bit codes) the canonical format is instead
 *    qweight uint8  [N][K]      one code 0..255 per byte
 *    zeros   uint8  [N][K/Gs]   zero point, 0..255
 * (scales as above), and w = scale * (q - zero) likewise.
 *
 * Packed (device) format, produced by qi4_pack: rows are cut into 16-row tiles
 * (with QI4_PACK_GATEUP, tile 2m holds gate rows 16m.. and tile 2m+1 the up rows
 * with the same index, so a tile pair yields 16 outputs of SiLU(gate)*up).
 * Let nt = number of tiles, G = K/128 (128-wide blocks of K), nq = ceil(nt/4)
 * "quads" of four consecutive tiles (tile t is slot t%4 of quad t/4), and
 * h = 2 for 64-wide groups (a block holds two groups), else 1.  Three regions
 * follow each other:
 *    codes  nt*G*1024 bytes    [tile][block][lane 0..63][16 bytes]
 *    scales nq*G*h*128 bytes   [quad][block][half][row 0..15][slot 0..3] binary16
 *    zeros  nq*G*h*32 bytes    [quad][block][half][row 0..15][2 bytes], slot s in nibble s
 * and the total is rounded up to a multiple of 256 bytes.  With groups of 128
 * or more, the records of every block of a group repeat that group's values.
 * Lane 16*j + r of a tile/block holds row r's codes for k in
 * 128*g + 32*s + 8*j + [0, 8) in its dword s (s = 0..3), so one 16-byte load per
 * lane brings a wave exactly one block of 16 rows.  Missing rows (N not a multiple
 * of 16) are packed as zeros.  An 8-bit matrix (QI4_INT8) is stored as the
 * 4-bit packed matrix of width 2K whose block 2b holds the high nibbles q >> 4
 * of block b with zero z >> 4 and scale binary16(16 * scale), and block 2b + 1
 * the low nibbles q & 15 with zero z & 15 and the scale itself:
 * 16 s (q_hi - z_hi) + s (q_lo - z_lo) = s (q - z) exactly, and every GEMM
 * reads the activations of block b for both.  16 * scale must be a binary16,
 * so 8-bit scales need |scale| <= 4094 (a larger one gives an infinite product).
 * The layout is private to this library: only qi4_pack writes it and only the
 * calls below read it.
 */
#ifndef QI4_H
#define QI4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QI4_ABI_VERSION 1

enum {
    QI4_OK = 0,
    QI4_ERR_NULL = -1,        /* a required pointer is NULL                          */
    QI4_ERR_SHAPE = -2,       /* a size is out of range or K % 128 != 0               */
    QI4_ERR_DTYPE = -3,       /* unknown dtype or epilogue code                       */
    QI4_ERR_GROUP = -4,       /* group_size not 0, 64 or a multiple of 128            */
    QI4_ERR_WORKSPACE = -5,   /* workspace too small                                  */
    QI4_ERR_ALIAS = -6,       /* an output overlaps an input                          */
    QI4_ERR_UNSUPPORTED = -7, /* device is not gfx950, or flags/epilogue combination */
    QI4_ERR_HIP = -8          /* a HIP runtime call or launch failed                  */
};

enum { QI4_F32 = 0, QI4_BF16 = 1 };          /* activation / output element types */
enum { QI4_EPI_NONE = 0, QI4_EPI_SILU_MUL = 1 };
enum { QI4_PACK_GATEUP = 1,                  /* pack flag: pair gate/up tiles      */
       QI4_INT8 = 2 };                        /* format flag: 8-bit codes           */

/* ABI version of the loaded library (QI4_ABI_VERSION). */
int qi4_abi_version(void);

/* Static, host-side, human-readable name of a status code. Never NULL. */
const char *qi4_status_string(int status);

/* Bytes of the packed format for an N x K matrix; negative status on bad
   arguments (N < 1, K < 128, K % 128, an unsupported group_size or one that
   does not divide K, unknown flags, or QI4_PACK_GATEUP with odd N). */
int64_t qi4_packed_bytes(int64_t N, int64_t K, int group_size, int flags);

/* Canonical -> packed (the offline reorder: each group of 16 rows becomes one
   contiguous kilobyte per wave load).  Exact: qi4_unpack inverts it bit for
   bit.  `packed` must hold qi4_packed_bytes(N, K, group_size, flags) bytes. */
int qi4_pack(const uint8_t *qweight, const uint16_t *scales, const uint8_t *zeros,
             int64_t N, int64_t K, int group_size, int flags, void *packed, void *stream);

/* Packed -> canonical; the exact inverse of qi4_pack (4-bit zero values beyond
   15 cannot occur). */
int qi4_unpack(const void *packed, int64_t N, int64_t K, int group_size, int flags,
               uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream);

/* Dequantize a packed matrix to float32 w [N][K] in canonical row order:
   w = float(scale) * (q - zero).  Exact (the product of a binary16 scale and an
   integer in [-255, 255] is representable in binary32). */
int qi4_dequant_f32(const void *packed, int64_t N, int64_t K, int group_size, int flags,
                    float *w, void *stream);

/* Load-time quantizer: w [N][K] (float32 or bf16 per w_dtype, 16-byte aligned;
 * qweight 4-byte aligned) -> canonical qweight, scales, zeros (the format above), in
 * groups of group_size (0: one per row).  The fastllm README (gittoolsai.com), section "model export": loading
 * with an int4 dtype quantizes online at every load, which is slow; this is that
 * step on the GPU.  Per group (asymmetric min/max, 0 always inside the range):
 *   lo = min(0, min w), hi = max(0, max w)
 *   scale = binary16 nearest (ties to even) of (hi - lo) / 15; 1.0 if that is 0
 *   zero  = clamp(rint(-lo / scale), 0, 15)
 *   q     = clamp(rint(w / scale) + zero, 0, 15)     rint: half to even
 * evaluated in binary64 (inputs widen exactly, divisions correctly rounded).
 * Weights must be finite (NaN is skipped by the min/max, its code unspecified).
 * Outputs must not overlap w or each other (QI4_ERR_ALIAS). */
int qi4_quantize(const void *w, int w_dtype, int64_t N, int64_t K, int group_size,
                 uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream);

/* The same quantizer with 8-bit codes (the --quant-bit 8 option of the FastLLM
 * page, section 4.2): 255 in place of 15 in every formula above, output in the
 * QI4_INT8 canonical format (qweight [N][K], 8-byte aligned; zeros 0..255). */
int qi4_quantize_int8(const void *w, int w_dtype, int64_t N, int64_t K, int group_size,
                      uint8_t *qweight, uint16_t *scales, uint8_t *zeros, void *stream);

/* The linear layer: y[t][n'] = epilogue( sum_k x[t][k] * dequant(W)[n][k] ), with
 * dequant(W)[n][k] = scale * (q - zero) for the 128-wide group of k in row n
 * (FastLLM page, section 3.1: 4-bit weights in groups of 128 with a scale and a
 * zero point, dequantized inside the product; decode reads every weight again
 * for every token, which makes this call bound by the weight stream).
 *   x        [T][K] of x_dtype (QI4_BF16 or QI4_F32), row-major, contiguous
 *   packed_w packed N x K matrix (flags as given to qi4_pack)
 *   y        [T][N'] of y_dtype (QI4_BF16 or QI4_F32);
 *            N' = N for QI4_EPI_NONE, N/2 for QI4_EPI_SILU_MUL
 *   epilogue QI4_EPI_SILU_MUL needs flags == QI4_PACK_GATEUP and gives
 *            y[t][i] = SiLU(g) * u with g, u the rows i and N/2 + i of [gate; up].
 * Accumulation is float32; the result is rounded once to y_dtype.  T == 0 is a
 * valid no-op.  float32 activations are used exactly (split into bf16 terms).
 * x must be finite: a row holding an inf or NaN gives unspecified (possibly
 * finite) values in that row of y, and leaves the other rows as they are. */
int qlinear_int4_g128(const void *x, int x_dtype, int64_t T, int64_t K,
                      const void *packed_w, int64_t N, int flags,
                      void *y, int y_dtype, int epilogue, void *stream);

/* The same linear layer for a matrix packed with any supported group_size (64,
 * a multiple of 128 dividing K, or 0 for one group per row); qlinear_int4_g128
 * is this call with group_size 128.  Section 4.2 of the FastLLM page above
 * allows group sizes 64 and 256 besides 128. */
int qlinear_int4(const void *x, int x_dtype, int64_t T, int64_t K,
                 const void *packed_w, int64_t N, int group_size, int flags,
                 void *y, int y_dtype, int epilogue, void *stream);

/* The same linear layer for an 8-bit matrix (packed with QI4_INT8 in flags; the
 * flag may be given or left out here).  The fastllm README lists int8 among the
 * weight types; the FastLLM page (section 4.2) converts with --quant-bit 8. */
int qlinear_int8(const void *x, int x_dtype, int64_t T, int64_t K,
                 const void *packed_w, int64_t N, int group_size, int flags,
                 void *y, int y_dtype, int epilogue, void *stream);

/* W4A8: the linear layer with int8 activations (the FastDeploy page,
 * x-techcon, names W4A8 static quantization: 4-bit weights, 8-bit activations
 * with a scale fixed ahead of time).  One static scale x_scale per tensor
 * (finite, > 0, with a finite float32 reciprocal, else QI4_ERR_SHAPE):
 *   r = float32(1 / x_scale)   (computed on the host in float32)
 *   a = clamp(rint(x * r), -127, 127)   float32 product, ties to even, NaN -> -127
 *   y = epilogue( x_scale * sum_k a_k * dequant(W)[n][k] )
 * The inner sums run on int8 MFMA in exact int32 per 128-wide block (the zero
 * point subtracted exactly), then the binary16 scale in float32.
 *   workspace  device, >= qlinear_w4a8_workspace_bytes(T, K) bytes, 16-byte
 *              aligned; receives the int8 activations (QI4_ERR_WORKSPACE if
 *              smaller); must not overlap x, y or packed_w.
 * 4-bit matrices only (QI4_INT8 in flags is QI4_ERR_UNSUPPORTED); other
 * arguments as qlinear_int4. */
int64_t qlinear_w4a8_workspace_bytes(int64_t T, int64_t K);
int qlinear_w4a8(const void *x, int x_dtype, float x_scale, int64_t T, int64_t K,
                 const void *packed_w, int64_t N, int group_size, int flags,
                 void *y, int y_dtype, int epilogue, void *workspace, int64_t ws_bytes,
                 void *stream);

/* ---------------------------------------------------------------------------
 * Routed mixture-of-experts FFN (decode and prefill).
 * Routed expert e uses packed gate/up block w_gate_up + e * qi4_packed_bytes(2I, H,
 * group_size, QI4_PACK_GATEUP | flags) and packed down block w_down + e *
 * qi4_packed_bytes(H, I, group_size, flags), flags = desc.flags.  The shared expert (has_shared != 0) has the same two shapes and is
 * added with weight 1.
 * ------------------------------------------------------------------------- */
typedef struct {
    int64_t num_experts;   /* E, routed experts (1..1024)                      */
    int64_t hidden;        /* H, multiple of 128                                */
    int64_t inter;         /* I, expert intermediate size, multiple of 128      */
    int32_t top_k;         /* routed experts per token (1..min(E, 32))           */
    int32_t group_size;    /* 64, a multiple of 128 dividing H and I, or 0      */
    int32_t has_shared;    /* 0 or 1                                            */
    int32_t flags;         /* 0 (4-bit experts) or QI4_INT8 (8-bit experts)      */
} qi4_moe_desc;            /* host struct                                       */

/* Router: for each token the top_k largest logits in descending order (ties to
 * the lower expert index) and softmax weights over those top_k only (the
 * FastLLM notes, wmrh.cn, part 1: each token activates a few of a MoE layer's
 * experts; the fastllm README's --moe_experts sets how many).
 *   logits [T][E] float32;  topk_ids [T][top_k] int32;  topk_weights [T][top_k] float32
 * Logits must not be NaN. */
int moe_route_topk(const float *logits, int64_t T, int64_t E, int32_t top_k,
                   int32_t *topk_ids, float *topk_weights, void *stream);

/* moe_route_topk followed by moe_sort_tokens (active required), in one call;
 * for batches of at most 16 tokens one workgroup does both, passing the ids
 * through on-chip memory (one launch instead of two).  Same outputs. */
int moe_route_sort(const float *logits, int64_t T, int64_t E, int32_t top_k, int32_t *topk_ids,
                   float *topk_weights, int32_t *sorted_pairs, int32_t *expert_offsets,
                   int32_t *pair_to_sorted, int32_t *active, void *stream);

/* Router projection and top-k in one call: the step before the routing above,
 * logits[t][e] = sum_k x[t][k] * w_router[e][k] with x bf16 [T][H] and
 * w_router bf16 [E][H] (row e = expert e), no bias, float32 accumulation in a
 * fixed order (deterministic), written to `logits` [T][E] float32; then the
 * moe_route_topk selection on those logits.  The pages route each token to a
 * few of many experts (FastLLM notes, wmrh.cn, part 1; --moe_experts in the
 * fastllm README); the projection itself is read as a plain linear layer.
 * H must be a multiple of 32, x and w_router 16-byte aligned; outputs must not
 * overlap the inputs or each other (QI4_ERR_ALIAS). */
int moe_router_topk(const void *x, int64_t T, int64_t H, const void *w_router, int64_t E,
                    int32_t top_k, float *logits, int32_t *topk_ids, float *topk_weights,
                    void *stream);

/* Token-by-expert permutation (stable counting sort of the T*top_k pairs
 * p = t*top_k + j by expert), so that each touched expert's weights are read
 * once for all of its tokens (the MoE layer activates few experts per token:
 * FastLLM notes, wmrh.cn, part 1):
 *   sorted_pairs   [T*top_k]  pairs grouped by expert ascending, tokens ascending
 *   expert_offsets [E+1]      segment starts; expert_offsets[E] = T*top_k
 *   pair_to_sorted [T*top_k]  inverse permutation
 *   active         [E+1] or NULL: active[0] = number of experts with a nonempty
 *                  segment, active[1..] those experts ascending
 * Ids must lie in [0, E); a pair with an id outside it is left out of the
 * permutation (pair_to_sorted = -1, and expert_offsets[E] counts only the pairs
 * kept; moe_combine skips it).  Deterministic. */
int moe_sort_tokens(const int32_t *topk_ids, int64_t T, int32_t top_k, int64_t E,
                    int32_t *sorted_pairs, int32_t *expert_offsets, int32_t *pair_to_sorted,
                    int32_t *active, void *stream);

/* Bytes of workspace moe_ffn_int4 needs for T tokens (negative status on bad
   descriptor). */
int64_t moe_ffn_int4_workspace_bytes(const qi4_moe_desc *d, int64_t T);

/* Stage calls.  moe_ffn_int4 below is route -> sort -> gate_up -> down -> combine
 * with exactly these kernels; they are exported for callers that route
 * elsewhere or time one stage.  Let P = T*top_k routed pairs and R = P + T*has_shared.
 * Row s < P of the intermediates belongs to sorted position s (see
 * moe_sort_tokens); row P + t belongs to token t's shared expert.
 *   h  [R][2][I] bf16 bits: SiLU(gate)*up as an unevaluated sum hi + lo of two
 *      bf16 numbers (hi = bf16(h), lo = bf16(h - hi)), about 16 significant bits
 *   y  [R][H] float32: each expert's down-projection output, before weighting
 * `active` is the array moe_sort_tokens fills.  `workspace` is a buffer of
 * moe_ffn_int4_workspace_bytes(d, T) bytes (256-byte aligned); the stage calls use
 * it for fp16 copies of their input rows (each row as fp16 times an exact power of
 * two) and, for batches of 128 or more tokens, the tile lists of the prefill
 * kernels.  h and y may lie inside it only if they do not overlap those regions;
 * passing separate buffers is simplest. */
int moe_expert_gate_up(const qi4_moe_desc *d, const void *x, int64_t T,
                       const int32_t *sorted_pairs, const int32_t *expert_offsets,
                       const int32_t *active, const void *w_gate_up,
                       const void *shared_gate_up, void *h, void *workspace, int64_t ws_bytes,
                       void *stream);
int moe_expert_down(const qi4_moe_desc *d, const void *h, int64_t T,
                    const int32_t *expert_offsets, const int32_t *active,
                    const void *w_down, const void *shared_down, float *y,
                    void *workspace, int64_t ws_bytes, void *stream);
/* out[t] = sum_j topk_weights[t][j] * y[pair_to_sorted[t*top_k+j]] (+ y[P+t]),
   summed in that order in float32, rounded once to bf16. */
int moe_combine(const qi4_moe_desc *d, const float *y, const float *topk_weights,
                const int32_t *pair_to_sorted, int64_t T, void *out, void *stream);

/* The MoE expert FFN layer (the fastllm README's MoE options: --moe_experts
 * routed experts per token, --cuda_se the shared expert; FastLLM notes, wmrh.cn,
 * part 1), with every expert int4 group-quantized as in qlinear_int4_g128:
 * out[t] = sum_j p[t][j] * FFN_{ids[t][j]}(x_t) + FFN_shared(x_t).
 *   x    [T][H] bf16 bits;  out [T][H] bf16 bits
 *   router_logits [T][E] float32, or NULL: then topk_ids/topk_weights
 *                 ([T][top_k] int32 / float32) supply the routing.  When the
 *                 logits are given, topk_ids/topk_weights may be NULL, or receive
 *                 the routing the call computed.
 *   shared_gate_up / shared_down: NULL iff has_shared == 0.
 *   workspace: moe_ffn_int4_workspace_bytes(d, T) bytes, 256-byte aligned.
 * The combine runs in a fixed order (slots 0..top_k-1, then the shared expert),
 * so results are deterministic.  x must be finite (as for qlinear_int4_g128: a
 * token whose row holds an inf or NaN gets unspecified values). */
int moe_ffn_int4(const qi4_moe_desc *d, const void *x, int64_t T,
                 const float *router_logits, int32_t *topk_ids, float *topk_weights,
                 const void *w_gate_up, const void *w_down,
                 const void *shared_gate_up, const void *shared_down,
                 void *out, void *workspace, int64_t ws_bytes, void *stream);

/* This device's share of the layer, for a layer whose experts are split
 * between devices (the fastllm README's --moe_device places a share of the MoE
 * work on the GPU and the rest on the CPU; the tencentcloud guide's single-GPU
 * plus CPU configuration splits it as {'cuda':1,'cpu':19}):
 *   out[t] = sum over j with gpu_experts[ids[t][j]] != 0 of p[t][j] * FFN_{ids[t][j]}(x_t)
 *            + FFN_shared(x_t) if d->has_shared.
 * gpu_experts: device uint8 [E], nonzero for the routed experts computed here;
 * only their weights are read (the others' blocks of w_gate_up / w_down may
 * hold anything).  The routing is computed (or given) in full, and when the
 * logits are given topk_ids / topk_weights, if not NULL, receive all of it, so
 * the other device can compute the remaining experts; the outputs of the two
 * shares add up to moe_ffn_int4's output.  Arguments, workspace
 * (moe_ffn_int4_workspace_bytes) and errors otherwise as moe_ffn_int4;
 * gpu_experts NULL is QI4_ERR_NULL. */
int moe_ffn_int4_share(const qi4_moe_desc *d, const void *x, int64_t T,
                       const float *router_logits, int32_t *topk_ids, float *topk_weights,
                       const void *w_gate_up, const void *w_down,
                       const void *shared_gate_up, const void *shared_down,
                       const uint8_t *gpu_experts, void *out, void *workspace, int64_t ws_bytes,
                       void *stream);

/* W4A8 MoE layer: moe_ffn_int4 with int8 activations in both projections (the
 * FastDeploy page, x-techcon, applies W4A8 static quantization to MoE layers).
 * Static scales, as in qlinear_w4a8: the layer input x is quantized with
 * x_scale, and h = SiLU(g) * u (computed in float32 from the int8 x) with
 * h_scale, a_h = clamp(rint(h * float32(1 / h_scale)), -127, 127), before the
 * down projection; both scales finite, > 0, with finite float32 reciprocals
 * (else QI4_ERR_SHAPE).  4-bit experts only (desc.flags 0, else
 * QI4_ERR_UNSUPPORTED).  Every batch size runs the weight-streaming grouped
 * GEMMs (int8 MFMA); workspace >= moe_ffn_w4a8_workspace_bytes(d, T).  Other
 * arguments, outputs and errors as moe_ffn_int4. */
int64_t moe_ffn_w4a8_workspace_bytes(const qi4_moe_desc *d, int64_t T);
int moe_ffn_w4a8(const qi4_moe_desc *d, const void *x, float x_scale, float h_scale, int64_t T,
                 const float *router_logits, int32_t *topk_ids, float *topk_weights,
                 const void *w_gate_up, const void *w_down,
                 const void *shared_gate_up, const void *shared_down,
                 void *out, void *workspace, int64_t ws_bytes, void *stream);

/* moe_ffn_int4 for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, results (bit for bit), routing outputs
 * and errors as moe_ffn_int4, minus the workspace: the call uses a scratch
 * array of QI4_NOALLOC_SCRATCH_BYTES (48 MiB) that the library holds on each
 * GPU it runs on until the process ends, and never allocates or frees.  A
 * layer whose moe_ffn_int4_workspace_bytes(d, T) exceeds that size returns
 * QI4_ERR_WORKSPACE before anything is enqueued (the DeepSeek-V3 shape, 7168 x
 * 2048 with 256 + 1 experts and top-8, fits up to T = 128).  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller. */
#define QI4_NOALLOC_SCRATCH_BYTES (48ll << 20)
int moe_ffn_int4_noalloc(const qi4_moe_desc *d, const void *x, int64_t T,
                         const float *router_logits, int32_t *topk_ids, float *topk_weights,
                         const void *w_gate_up, const void *w_down,
                         const void *shared_gate_up, const void *shared_down,
                         void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QI4_H */
