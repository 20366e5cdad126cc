/*
 * qi4 oracle -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, obviously correct fp64 CPU implementation of what the int4
 * group-quantized linear layer and the routed MoE expert FFN compute.  Only the
 * test-suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant generator with the GPU library
 * (ffn_int4_g128_amd/csrc); neither includes nor links the other.
 *
 * Sources (cited by page title and section):
 *  [P3] FastLLM: zero-dependency CPU inference framework (pgsm.cn),
 *       section 3.1 (4-bit quantization and weight reordering): 4-bit weights in
 *       groups of 128 that share one scale and one zero point; each weight is
 *       dequantized to float32 and then enters the matrix product;
 *       section 4.2 "model conversion and format": --quant-bit 4/8,
 *       --group-size default 128, 64/256 allowed.
 *  [P1] fastllm README (gittoolsai.com), "other parameters": --moe_experts
 *       (number of routed experts per token), --cuda_se (shared expert);
 *       "inference precision": int4g / int4 / int8 weight types.
 *  [P2] FastLLM notes (wmrh.cn), part 1: MoE layers hold huge parameter counts
 *       but each token activates only a few experts.
 *  Where the pages are silent the plain readings used are:
 *   R1  even k in the low nibble of byte k/2;
 *   R3  W is [N][K] (out x in), group g covers k in [g*G, g*G+G) of one row;
 *   R5  w = scale * (q - zero)  (the dequantization formula of the workloads);
 *   R8  gate/up weight = rows [0,I) gate, rows [I,2I) up;
 *   R9  top-k by value descending, ties to the lower expert index;
 *   R10 combine weights = softmax over the selected k logits only;
 *   R11 the shared expert is added with weight 1;
 *   R12 token permutation: expert ascending, then token ascending;
 *   R19 reference quantizer: asymmetric min/max with 0 inside the range;
 *   R29 8-bit weights (--quant-bit 8): one byte per code, q in 0..255, same
 *       groups, binary16 scale and a zero in 0..255, w = scale * (q - zero).
 *   R30 W4A8 (FastDeploy page, x-techcon: "W4A8 static quantization"): the
 *       activations are quantized to int8 with one static (caller-given) scale
 *       s_x per tensor, symmetric: a = clamp(rint(x * r), -127, 127) with
 *       r = float32(1 / s_x) and the product rounded to float32 (the decision
 *       is taken in float32), rint half to even; the layer then computes
 *       y = sum_k (a_k * s_x) * w_k with the weights as before.
 *
 * `bits` (4 or 8) selects the code width everywhere: 4-bit codes pack two per
 * byte (qweight [N][K/2]), 8-bit codes one per byte (qweight [N][K]).
 *
 * Everything is computed in double.  Scales arrive as IEEE binary16 bit
 * patterns and are decoded exactly.  Activations arrive already widened to
 * double (bf16 and fp32 both widen exactly).
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORACLE_ABI 5
int qi4o_abi_version(void) { return ORACLE_ABI; }

/* ---- IEEE binary16 <-> double ----------------------------------------- */

/* Exact decode of a binary16 bit pattern: value = (-1)^s * 2^(e-15) * (1 + m/1024),
   subnormal when e == 0: (-1)^s * 2^-14 * (m/1024). */
double qi4o_f16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even.  Used only by
   the reference quantizer (scale storage).  Works on the real value: find the
   binade, scale the significand to an integer and round it half-to-even. */
uint16_t qi4o_f64_to_f16(double v)
{
    uint16_t sign = 0;
    if (isnan(v)) return 0x7e00;
    if (v < 0 || (v == 0 && signbit(v))) { sign = 0x8000; v = -v; }
    if (v == 0) return sign;
    if (isinf(v)) return sign | 0x7c00;
    int e;
    frexp(v, &e);               /* v = f * 2^e, f in [0.5, 1) -> v in [2^(e-1), 2^e) */
    int exp_unb = e - 1;        /* v in [2^exp_unb, 2^(exp_unb+1)) */
    if (exp_unb < -14) exp_unb = -14;      /* subnormal range shares the 2^-24 quantum */
    double quantum = ldexp(1.0, exp_unb - 10);
    double r = v / quantum;     /* exact: division by a power of two */
    double fl = floor(r);
    double frac = r - fl;
    double n;
    if (frac > 0.5) n = fl + 1;
    else if (frac < 0.5) n = fl;
    else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1;
    double rv = n * quantum;
    if (rv >= 65520.0) return sign | 0x7c00;   /* rounds to infinity */
    /* re-encode the rounded value */
    if (rv < ldexp(1.0, -14)) {
        return sign | (uint16_t)(rv / ldexp(1.0, -24));
    }
    int e2;
    frexp(rv, &e2);
    int eu = e2 - 1;
    uint16_t m = (uint16_t)(rv / ldexp(1.0, eu - 10) - 1024.0);
    return sign | (uint16_t)((eu + 15) << 10) | m;
}

/* ---- the quantized format ----------------------------------------------- */

/* [P3 s3.1] one 4-bit code per weight, two codes per byte (R1: even k low);
   [P3 s4.2] with 8-bit quantization one code per byte (R29). */
static inline int q_at(const uint8_t *qweight, int64_t K, int64_t n, int64_t k, int bits)
{
    if (bits == 8) return qweight[n * K + k];
    uint8_t b = qweight[n * (K / 2) + k / 2];
    return (k & 1) ? (b >> 4) : (b & 15);
}

/* Bytes of the codes of one N x K matrix. */
static inline int64_t code_bytes(int64_t N, int64_t K, int bits)
{
    return bits == 8 ? N * K : N * (K / 2);
}

/* Dequantize one weight: w = scale * (q - zero) with the scale and zero of the
   group that holds k ([P3 s3.1]; formula R5). */
static inline double w_at(const uint8_t *qweight, const uint16_t *scales,
                          const uint8_t *zeros, int64_t K, int64_t G, int bits,
                          int64_t n, int64_t k)
{
    int64_t ng = K / G;
    int64_t g = k / G;
    double s = qi4o_f16_to_f64(scales[n * ng + g]);
    int z = zeros[n * ng + g];
    int q = q_at(qweight, K, n, k, bits);
    return s * (double)(q - z);
}

static int bad_shape(int64_t N, int64_t K, int64_t G, int bits)
{
    return N < 0 || K <= 0 || G <= 0 || (K % G) != 0 || (K % 2) != 0 ||
           (bits != 4 && bits != 8);
}

/* Unpack the codes: q[n][k] in 0..15 (4-bit) or 0..255 (8-bit). */
int qi4o_unpack(const uint8_t *qweight, int64_t N, int64_t K, int bits, uint8_t *q)
{
    if (N < 0 || K <= 0 || (K % 2) || (bits != 4 && bits != 8)) return -2;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            q[n * K + k] = (uint8_t)q_at(qweight, K, n, k, bits);
    return 0;
}

/* Dequantize the whole matrix: w[n][k] = scale(n, k/G) * (q(n,k) - zero(n, k/G)). */
int qi4o_dequant(const uint8_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                 int64_t N, int64_t K, int64_t G, int bits, double *w)
{
    if (bad_shape(N, K, G, bits)) return -2;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            w[n * K + k] = w_at(qweight, scales, zeros, K, G, bits, n, k);
    return 0;
}

/* ---- the linear layer ------------------------------------------------- */

/* y[t][n] = sum_k x[t][k] * w[n][k]  (dequantize, then multiply; [P3 s3.1]),
   k ascending, fp64 accumulator starting at 0.  S[t][n] = sum_k |x[t][k]*w[n][k]|
   is the magnitude the tolerance is stated against.  S may be NULL. */
int qi4o_linear(const double *x, int64_t T, int64_t K,
                const uint8_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                int64_t N, int64_t G, int bits, double *y, double *S, int threads)
{
    if (bad_shape(N, K, G, bits) || T < 0) return -2;
    if (threads < 1) threads = 1;
    for (int64_t t = 0; t < T; t++) {
        const double *xt = x + t * K;
#pragma omp parallel for num_threads(threads) schedule(static)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = xt[k] * w_at(qweight, scales, zeros, K, G, bits, n, k);
                acc += p;
                mag += fabs(p);
            }
            y[t * N + n] = acc;
            if (S) S[t * N + n] = mag;
        }
    }
    return 0;
}

/* ---- W4A8: int8 activations (R30) ---------------------------------------- */

/* a[t][k] = clamp(rint(x[t][k] * r), -127, 127): the product is a float32
   product (one rounding), rint rounds half to even; NaN gives -127. */
int qi4o_quantize_act(const float *x, int64_t n, float r, int8_t *a)
{
    if (n < 0) return -2;
    for (int64_t i = 0; i < n; i++) {
        volatile float p = x[i] * r;   /* float32 product, not widened */
        float q = rintf(p);
        if (!(q >= -127.0f)) q = -127.0f;
        if (q > 127.0f) q = 127.0f;
        a[i] = (int8_t)q;
    }
    return 0;
}

/* xhat[i] = a[i] * s_x in double (exact: an 8-bit integer times a float32). */
int qi4o_dequant_act(const int8_t *a, int64_t n, float s_x, double *xhat)
{
    if (n < 0) return -2;
    for (int64_t i = 0; i < n; i++) xhat[i] = (double)a[i] * (double)s_x;
    return 0;
}

/* ---- SiLU(gate) * up ---------------------------------------------------- */

/* SiLU(v) = v / (1 + exp(-v)), written the plain way in double. */
double qi4o_silu(double v) { return v / (1.0 + exp(-v)); }

/* SiLU has one minimum, at the root g* of its derivative
   sigma(g) * (1 + g * (1 - sigma(g))) (about -1.2785): it decreases before g* and
   increases after.  Found once by bisection on [-2, -1], where the derivative
   changes sign. */
static double silu_argmin(void)
{
    static double gstar = 0.0;
    if (gstar == 0.0) {
        double lo = -2.0, hi = -1.0;
        for (int it = 0; it < 200 && hi - lo > 0.0; it++) {
            double mid = 0.5 * (lo + hi);
            if (mid == lo || mid == hi) break;
            double sg = 1.0 / (1.0 + exp(-mid));
            double d = sg * (1.0 + mid * (1.0 - sg));
            if (d < 0.0) lo = mid; else hi = mid;
        }
        gstar = 0.5 * (lo + hi);
    }
    return gstar;
}

/* The largest |SiLU(g + d) - SiLU(g)| over |d| <= a.  SiLU is unimodal, so on
   [g - a, g + a] its extreme values sit at the two ends or at its minimum g*. */
static double silu_dev(double g, double a)
{
    double s0 = qi4o_silu(g);
    double d1 = fabs(qi4o_silu(g + a) - s0), d2 = fabs(qi4o_silu(g - a) - s0);
    double d = d1 > d2 ? d1 : d2;
    double gs = silu_argmin();
    if (g - a <= gs && gs <= g + a) {
        double d3 = fabs(s0 - qi4o_silu(gs));
        if (d3 > d) d = d3;
    }
    return d;
}

/* h[t][i] = SiLU(g[t][i]) * u[t][i] where [g; u] = x . W_gu^T, W_gu rows
   [0,I) = gate, [I,2I) = up (R8).  tol_h (may be NULL) bounds |h' - h| for any
   g' = g + dg, u' = u + du with |dg| <= c*S_g and |du| <= c*S_u (the per-linear
   tolerance of each projection, S = sum|w*x|):
     h' - h = (SiLU(g') - SiLU(g)) * u' + SiLU(g) * du, so
     tol_h = D * (|u| + c*S_u) + |SiLU(g)| * c*S_u
   with D the largest |SiLU(g + d) - SiLU(g)| over |d| <= c*S_g (R14).  As c
   shrinks this is c * (|SiLU'(g)| * |u| * S_g + |SiLU(g)| * S_u). */
int qi4o_gate_up_silu(const double *x, int64_t T, int64_t K,
                      const uint8_t *qweight, const uint16_t *scales, const uint8_t *zeros,
                      int64_t I, int64_t G, int bits, double c, double *h, double *tol_h,
                      int threads)
{
    int64_t N = 2 * I;
    if (bad_shape(N, K, G, bits) || T < 0) return -2;
    double *gu = (double *)malloc(sizeof(double) * (size_t)(T * N + 1));
    double *S = (double *)malloc(sizeof(double) * (size_t)(T * N + 1));
    if (!gu || !S) { free(gu); free(S); return -9; }
    int rc = qi4o_linear(x, T, K, qweight, scales, zeros, N, G, bits, gu, S, threads);
    if (rc == 0) {
        for (int64_t t = 0; t < T; t++)
            for (int64_t i = 0; i < I; i++) {
                double g = gu[t * N + i], u = gu[t * N + I + i];
                h[t * I + i] = qi4o_silu(g) * u;
                if (tol_h) {
                    double ag = c * S[t * N + i], au = c * S[t * N + I + i];
                    tol_h[t * I + i] = silu_dev(g, ag) * (fabs(u) + au) + fabs(qi4o_silu(g)) * au;
                }
            }
    }
    free(gu); free(S);
    return rc;
}

/* ---- router: top-k and softmax over the selected ------------------------ */

/* For each token: the k largest logits, in descending order, ties broken toward
   the lower expert index (R9); p = softmax over the selected k only (R10).
   The number of routed experts per token is the --moe_experts knob of [P1]. */
int qi4o_topk_softmax(const float *logits, int64_t T, int64_t E, int k,
                      int32_t *ids, double *p)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -2;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!taken) return -9;
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                /* strictly greater wins, so on a tie the earlier (lower) index stays */
                if (best < 0 || (double)l[e] > (double)l[best]) best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        double lmax = (double)l[ids[t * k + 0]];
        double den = 0.0;
        for (int j = 0; j < k; j++) den += exp((double)l[ids[t * k + j]] - lmax);
        for (int j = 0; j < k; j++) p[t * k + j] = exp((double)l[ids[t * k + j]] - lmax) / den;
    }
    free(taken);
    return 0;
}

/* ---- token-by-expert permutation ---------------------------------------- */

/* The routed (token, slot) pairs grouped by expert: for e ascending, for t
   ascending, the pair t*k+j with ids[t][j] == e (R12).  offsets[e] is where
   expert e's segment starts, offsets[E] = T*k; pair_to_sorted is the inverse.
   Returns -3 if an id is out of range. */
int qi4o_sort(const int32_t *ids, int64_t T, int k, int64_t E,
              int32_t *sorted_pairs, int32_t *offsets, int32_t *pair_to_sorted)
{
    if (T < 0 || E <= 0 || k <= 0) return -2;
    for (int64_t i = 0; i < T * k; i++)
        if (ids[i] < 0 || ids[i] >= E) return -3;
    int64_t pos = 0;
    for (int64_t e = 0; e < E; e++) {
        offsets[e] = (int32_t)pos;
        for (int64_t t = 0; t < T; t++)
            for (int j = 0; j < k; j++)
                if (ids[t * k + j] == e) {
                    sorted_pairs[pos] = (int32_t)(t * k + j);
                    pair_to_sorted[t * k + j] = (int32_t)pos;
                    pos++;
                }
    }
    offsets[E] = (int32_t)pos;
    return 0;
}

/* ---- the MoE expert FFN -------------------------------------------------- */

/* One expert on one token: h = SiLU(W_g x) * (W_u x), y = W_d h, in double.
   A (may be NULL) bounds |y' - y| when h is off by at most tol_h and the down
   projection adds its own error of at most c * sum|W_d * h'| (h' the h it was
   given): A[n] = sum_i |W_d[n][i]| * (tol_h[i] + c * (|h_i| + tol_h[i])). */
static int expert_ffn(const double *xt, int64_t H, int64_t I, int64_t Ggu, int64_t Gdn,
                      int bits, double c, const uint8_t *gq, const uint16_t *gs, const uint8_t *gz,
                      const uint8_t *dq, const uint16_t *ds, const uint8_t *dz,
                      double *y, double *A, double *h, double *tol_h, int threads)
{
    int rc = qi4o_gate_up_silu(xt, 1, H, gq, gs, gz, I, Ggu, bits, c, h, tol_h, threads);
    if (rc) return rc;
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t n = 0; n < H; n++) {
        double acc = 0.0, a = 0.0;
        for (int64_t i = 0; i < I; i++) {
            double w = w_at(dq, ds, dz, I, Gdn, bits, n, i);
            acc += w * h[i];
            a += fabs(w) * (tol_h[i] + c * (fabs(h[i]) + tol_h[i]));
        }
        y[n] = acc;
        if (A) A[n] = a;
    }
    return 0;
}

/* out[t] = sum_{j<k} p[t][j] * FFN_{ids[t][j]}(x_t) + FFN_shared(x_t)   (R10, R11)
 *
 * Routed expert e uses gate/up block gu_*[e] (2I x H, groups along H) and down
 * block dn_*[e] (H x I, groups along I); G = 0 means one group per row of each
 * matrix (H for gate/up, I for down: the plain, per-channel int4 that the
 * fastllm README names beside the grouped int4g).  The shared expert (sh_*) is skipped
 * when sh_gu_q is NULL.  tol (may be NULL) bounds the output's error when every
 * linear is off by at most c times its sum|w*x| and every combine weight by at
 * most eps_p: sum_j (|p_j|*A_{e_j} + eps_p*(|y_{e_j}| + A_{e_j})) + A_shared
 * (reading R14).
 * Tokens are processed one by one; threads split output rows of each linear. */
int qi4o_moe(const double *x, int64_t T, int64_t H, int64_t I, int64_t E, int k,
             const int32_t *ids, const double *p,
             const uint8_t *gu_q, const uint16_t *gu_s, const uint8_t *gu_z,
             const uint8_t *dn_q, const uint16_t *dn_s, const uint8_t *dn_z,
             const uint8_t *sh_gu_q, const uint16_t *sh_gu_s, const uint8_t *sh_gu_z,
             const uint8_t *sh_dn_q, const uint16_t *sh_dn_s, const uint8_t *sh_dn_z,
             int64_t G, int bits, double c, double eps_p, double *out, double *tol,
             int threads)
{
    const int64_t Ggu = G ? G : H, Gdn = G ? G : I;
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || G < 0 || H % Ggu || I % Gdn) return -2;
    if (bits != 4 && bits != 8) return -2;
    if (threads < 1) threads = 1;
    const int64_t gu_qb = code_bytes(2 * I, H, bits), gu_mb = 2 * I * (H / Ggu);
    const int64_t dn_qb = code_bytes(H, I, bits), dn_mb = H * (I / Gdn);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    double *A = (double *)malloc(sizeof(double) * (size_t)H);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    double *th = (double *)malloc(sizeof(double) * (size_t)I);
    if (!y || !A || !h || !th) { free(y); free(A); free(h); free(th); return -9; }
    int rc = 0;
    for (int64_t t = 0; t < T && rc == 0; t++) {
        const double *xt = x + t * H;
        double *ot = out + t * H;
        double *tt = tol ? tol + t * H : NULL;
        for (int64_t n = 0; n < H; n++) { ot[n] = 0.0; if (tt) tt[n] = 0.0; }
        for (int j = 0; j < k && rc == 0; j++) {
            int64_t e = ids[t * k + j];
            if (e < 0 || e >= E) { rc = -3; break; }
            double pj = p[t * k + j];
            rc = expert_ffn(xt, H, I, Ggu, Gdn, bits, c,
                            gu_q + e * gu_qb, gu_s + e * gu_mb, gu_z + e * gu_mb,
                            dn_q + e * dn_qb, dn_s + e * dn_mb, dn_z + e * dn_mb,
                            y, A, h, th, threads);
            for (int64_t n = 0; n < H; n++) {
                ot[n] += pj * y[n];
                if (tt) tt[n] += fabs(pj) * A[n] + eps_p * (fabs(y[n]) + A[n]);
            }
        }
        if (rc == 0 && sh_gu_q) {
            rc = expert_ffn(xt, H, I, Ggu, Gdn, bits, c, sh_gu_q, sh_gu_s, sh_gu_z,
                            sh_dn_q, sh_dn_s, sh_dn_z, y, A, h, th, threads);
            for (int64_t n = 0; n < H; n++) {
                ot[n] += y[n];
                if (tt) tt[n] += A[n];
            }
        }
    }
    free(y); free(A); free(h); free(th);
    return rc;
}

/* ---- W4A8 MoE (R30 applied to both projections) -------------------------- */

/* One expert with int8 activations: h = SiLU(g) * u from xhat (already the
   dequantized int8 input); the decision a_h = clamp(rint(float32(float32(h) * r_h)),
   -127, 127) with r_h = float32(1 / s_h), hhat = a_h * s_h; y = hhat . W_d^T.
   A[n] = sum_k |W_d[n][k] * hhat_k| (for the per-linear factor c) and
   B[n] = s_h * sum_k |W_d[n][k]| over the k whose decision is not certain: the
   range h +- amb_k (amb = the bound on |h' - h| of qi4o_gate_up_silu for a
   relative error c_amb in g and u, plus the float32 roundings of h and of
   h * r_h) maps to two different clamped codes. */
static int expert_ffn_w4a8(const double *xhat, int64_t H, int64_t I, int64_t Ggu, int64_t Gdn,
                           float s_h, double c_amb, const uint8_t *gq, const uint16_t *gs,
                           const uint8_t *gz, const uint8_t *dq, const uint16_t *ds,
                           const uint8_t *dz, double *y, double *A, double *B, double *h,
                           double *amb, double *hq, int *unsure, int threads)
{
    int rc = qi4o_gate_up_silu(xhat, 1, H, gq, gs, gz, I, Ggu, 4, c_amb, h, amb, threads);
    if (rc) return rc;
    const float r = 1.0f / s_h;
    for (int64_t i = 0; i < I; i++) {
        volatile float hf = (float)h[i];
        volatile float pr = hf * r;
        float q = rintf(pr);
        if (!(q >= -127.0f)) q = -127.0f;
        if (q > 127.0f) q = 127.0f;
        hq[i] = (double)q * (double)s_h;
        const double m = amb[i] + fabs(h[i]) * ldexp(1.0, -22);
        double lo = rint((h[i] - m) * (double)r), hi = rint((h[i] + m) * (double)r);
        lo = lo < -127 ? -127 : (lo > 127 ? 127 : lo);
        hi = hi < -127 ? -127 : (hi > 127 ? 127 : hi);
        unsure[i] = lo != hi;
    }
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t n = 0; n < H; n++) {
        double acc = 0.0, a = 0.0, b = 0.0;
        for (int64_t i = 0; i < I; i++) {
            double w = w_at(dq, ds, dz, I, Gdn, 4, n, i);
            acc += w * hq[i];
            a += fabs(w * hq[i]);
            if (unsure[i]) b += fabs(w) * (double)s_h;
        }
        y[n] = acc;
        A[n] = a;
        B[n] = b;
    }
    return 0;
}

/* out[t] = sum_j p[t][j] * FFN8_{ids[t][j]}(xhat_t) + FFN8_shared(xhat_t) with
   xhat = the int8 activations of x (scale s_x, qi4o_quantize_act) times s_x and
   FFN8 the expert above; 4-bit weights as in qi4o_moe.  Per expert the error of
   y is at most D = B + c * (A + B): the uncertain h decisions (one step each,
   B; the gate/up error enters only through those, bounded by c_amb) and the
   down projection's own c * sum|W_d * h'| for h' within one step of hhat on the
   uncertain decisions.  tol = sum_j (|p_j| D_j + eps_p (|y_j| + D_j)) + D_sh. */
int qi4o_moe_w4a8(const float *x, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                  const int32_t *ids, const double *p,
                  const uint8_t *gu_q, const uint16_t *gu_s, const uint8_t *gu_z,
                  const uint8_t *dn_q, const uint16_t *dn_s, const uint8_t *dn_z,
                  const uint8_t *sh_gu_q, const uint16_t *sh_gu_s, const uint8_t *sh_gu_z,
                  const uint8_t *sh_dn_q, const uint16_t *sh_dn_s, const uint8_t *sh_dn_z,
                  int64_t G, float s_x, float s_h, double c, double c_amb, double eps_p,
                  double *out, double *tol, int threads)
{
    const int64_t Ggu = G ? G : H, Gdn = G ? G : I;
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || G < 0 || H % Ggu || I % Gdn) return -2;
    if (!(s_x > 0.0f) || !(s_h > 0.0f)) return -2;
    if (threads < 1) threads = 1;
    const int64_t gu_qb = code_bytes(2 * I, H, 4), gu_mb = 2 * I * (H / Ggu);
    const int64_t dn_qb = code_bytes(H, I, 4), dn_mb = H * (I / Gdn);
    double *xh = (double *)malloc(sizeof(double) * (size_t)H);
    int8_t *ax = (int8_t *)malloc((size_t)H);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    double *A = (double *)malloc(sizeof(double) * (size_t)H);
    double *B = (double *)malloc(sizeof(double) * (size_t)H);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    double *amb = (double *)malloc(sizeof(double) * (size_t)I);
    double *hq = (double *)malloc(sizeof(double) * (size_t)I);
    int *un = (int *)malloc(sizeof(int) * (size_t)I);
    int rc = 0;
    if (!xh || !ax || !y || !A || !B || !h || !amb || !hq || !un) rc = -9;
    for (int64_t t = 0; t < T && rc == 0; t++) {
        qi4o_quantize_act(x + t * H, H, 1.0f / s_x, ax);
        qi4o_dequant_act(ax, H, s_x, xh);
        double *ot = out + t * H;
        double *tt = tol ? tol + t * H : NULL;
        for (int64_t n = 0; n < H; n++) { ot[n] = 0.0; if (tt) tt[n] = 0.0; }
        for (int j = 0; j < k && rc == 0; j++) {
            int64_t e = ids[t * k + j];
            if (e < 0 || e >= E) { rc = -3; break; }
            double pj = p[t * k + j];
            rc = expert_ffn_w4a8(xh, H, I, Ggu, Gdn, s_h, c_amb,
                                 gu_q + e * gu_qb, gu_s + e * gu_mb, gu_z + e * gu_mb,
                                 dn_q + e * dn_qb, dn_s + e * dn_mb, dn_z + e * dn_mb,
                                 y, A, B, h, amb, hq, un, threads);
            for (int64_t n = 0; n < H; n++) {
                double D = B[n] + c * (A[n] + B[n]);
                ot[n] += pj * y[n];
                if (tt) tt[n] += fabs(pj) * D + eps_p * (fabs(y[n]) + D);
            }
        }
        if (rc == 0 && sh_gu_q) {
            rc = expert_ffn_w4a8(xh, H, I, Ggu, Gdn, s_h, c_amb, sh_gu_q, sh_gu_s, sh_gu_z,
                                 sh_dn_q, sh_dn_s, sh_dn_z, y, A, B, h, amb, hq, un, threads);
            for (int64_t n = 0; n < H; n++) {
                ot[n] += y[n];
                if (tt) tt[n] += B[n] + c * (A[n] + B[n]);
            }
        }
    }
    free(xh); free(ax); free(y); free(A); free(B); free(h); free(amb); free(hq); free(un);
    return rc;
}

/* ---- reference quantizer (round-trip checks only) ----------------------- */

/* Asymmetric min/max quantizer per group (R19) with L = 2^bits - 1 levels
   (15 or 255): lo = min(min w, 0), hi = max(max w, 0), scale = fp16((hi - lo)/L)
   (1 if that is 0), zero = clamp(rint(-lo/scale), 0, L),
   q = clamp(rint(w/scale) + zero, 0, L); rint rounds half to even.  The scale is
   rounded to binary16 before it is used, so dequantizing with the stored scale
   reproduces what q was chosen against. */
int qi4o_quantize(const double *w, int64_t N, int64_t K, int64_t G, int bits,
                  uint8_t *qweight, uint16_t *scales, uint8_t *zeros)
{
    if (bad_shape(N, K, G, bits)) return -2;
    const double L = (double)((1 << bits) - 1);
    int64_t ng = K / G;
    memset(qweight, 0, (size_t)code_bytes(N, K, bits));
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < ng; g++) {
            const double *wg = w + n * K + g * G;
            double lo = 0.0, hi = 0.0;
            for (int64_t i = 0; i < G; i++) {
                if (wg[i] < lo) lo = wg[i];
                if (wg[i] > hi) hi = wg[i];
            }
            uint16_t sb = qi4o_f64_to_f16((hi - lo) / L);
            double s = qi4o_f16_to_f64(sb);
            if (s == 0.0) { sb = 0x3c00; s = 1.0; }
            double zf = nearbyint(-lo / s);
            if (zf < 0) zf = 0;
            if (zf > L) zf = L;
            int z = (int)zf;
            scales[n * ng + g] = sb;
            zeros[n * ng + g] = (uint8_t)z;
            for (int64_t i = 0; i < G; i++) {
                double qf = nearbyint(wg[i] / s) + z;
                if (qf < 0) qf = 0;
                if (qf > L) qf = L;
                int64_t k = g * G + i;
                uint8_t q = (uint8_t)qf;
                if (bits == 8) qweight[n * K + k] = q;
                else qweight[n * (K / 2) + k / 2] |= (k & 1) ? (uint8_t)(q << 4) : q;
            }
        }
    return 0;
}
