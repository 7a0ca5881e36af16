/*
 * fp64 CPU oracle of the DeepSeekMoE layer forward.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load or call this file; the layer itself never
 * does, and this file shares no code, header or table with the HIP library.
 *
 * What it computes, step by step, for every requested token t (all
 * arithmetic in IEEE double, plain sequential loops, bf16 inputs widened
 * exactly):
 *
 *   1. affinity  a_e = sum_j x[t,j] * C[e,j]
 *      The token-to-centroid inner product of the generic top-K MoE gate
 *      ("DeepSeekMoE 深度解读报告", section 3.1, Eq. 3-5 as described there).
 *   2. score     softmax gate (default): l_e = a_e + b_e (b_e = 0 without
 *      bias) and s_e = exp(l_e - max l) / sum_f exp(l_f - max l), over the
 *      N*m routed experts only; shared experts never enter the gate (same
 *      page, sections 2.3 and 3.1).  The selection key is s_e.
 *      sigmoid gate (ORACLE_SIGMOID): s_e = 1 / (1 + exp(-a_e)) and the
 *      selection key is s_e + b_e: the bias steers which experts are chosen
 *      but not their weights (the auxiliary-loss-free routing remark of the
 *      youleyou page, "DeepSeek MoE模型优化与未来演进及字节超稀疏内存技术",
 *      and the sigmoid gate of the V3 line in the report's closing notes).
 *   3. selection K rounds of argmax of the key over the experts not yet
 *      taken, strict '>' so that the lower index wins a tie.  gate_k =
 *      s_{e_k}; the other experts get 0 (section 3.1: keep the top scores,
 *      zero the rest).  With ORACLE_RENORM the K gates are divided by their
 *      sum, taken in selection order; for the softmax gate this equals a
 *      softmax over the K selected logits, the routing code of the eliteato
 *      DeepSeek-V2 explainer (section 3.1).  margin = key_(K) - key_(K+1),
 *      +inf when K == E or K == 0.
 *   4. expert    FFN_W(x) = W2 (silu(W1 x) * (W3 x)), silu(z) = z/(1+e^-z),
 *      W1, W3 of shape [inter, d] and W2 of shape [d, inter], no bias
 *      (the Expert module printed on the youleyou page, "DeepSeek MoE模型优化
 *      与未来演进及字节超稀疏内存技术").
 *   5. output    out = x + sum_{s<K_s} FFN_{shared s}(x) + sum_k gate_k FFN_{e_k}(x)
 *      (shared experts isolated and always active, section 2.3 / 3.1 of the
 *      report; the residual term is dropped when ORACLE_NO_RESIDUAL is set).
 *
 * Fine-grained segmentation (section 2.2) enters only through the shape:
 * E = N*m routed experts, each of inter-dim I = I_std/m.
 *
 * 8-bit routed weights (oracle_forward_fp8): each routed weight matrix is
 * given as OCP FP8 E4M3 codes q with one float scale per output row, the
 * weight being e4m3(q) * scale[row]; the shared experts stay bf16.  This is
 * the per-channel quantisation of routed experts, shared experts kept at
 * 16 bits, that the eliteato DeepSeek-V2 explainer recommends (section 5.5).
 * e4m3() follows the OCP 8-bit floating point definition: sign bit 7,
 * exponent field bits 6-3 with bias 7, mantissa field bits 2-0; exponent
 * field 0 holds the subnormals m/8 * 2^-6, and 0x7F / 0xFF are NaN.  Every
 * finite value and every product with a float scale is exact in double.
 *
 * 8-bit activations (ORACLE_ACT8, with 8-bit routed weights the layer's
 * products can then run on 8-bit multipliers): each token's row x gets the
 * power-of-two scale 2^e, e the smallest integer with max_j |x_j| <= 448 *
 * 2^e (448 being E4M3's largest finite value; e = 0 for an all-zero row),
 * and the codes q_j = nearest E4M3 value of x_j * 2^-e, ties to the even
 * code.  The routed experts' W1 x and W3 x take the dequantised row
 * e4m3(q_j) * 2^e.  Their down projection's input is treated the same way:
 * h = silu(W1 x) * W3 x is first rounded to bf16 (nearest, ties to even;
 * the 16-bit format the layer holds h in between its two products), then
 * each (token, expert) row of h gets its own power-of-two scale and
 * nearest-even codes by the same rule, and W2 takes the dequantised row.
 * The shared experts keep 16-bit activations throughout.  The pages only
 * advise low-bit routed experts with per-channel or per-group scales
 * (eliteato DeepSeek-V2 explainer, section 5.5); per-row power-of-two scales
 * are the plainest reading that keeps every quantised value, and its
 * product with any weight, exact, and quantising both inputs of the routed
 * products lets all of them run on 8-bit multipliers.
 *
 * Tokens are independent; OpenMP runs them on separate threads without
 * changing any token's order of operations.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NO_RESIDUAL 1u
#define ORACLE_RENORM 2u
#define ORACLE_SIGMOID 4u
#define ORACLE_ACT8 8u

typedef struct {
    int32_t T, d, E, I, K, Ks, Is;
    uint32_t flags;
} oracle_shape;

static double widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Steps 1-3 for one token.  x_t: [d] widened.  probs: [E] out (the scores
 * s_e), key: [E] scratch (the selection keys). */
static void route_token(const oracle_shape* s, const double* x_t,
                        const uint16_t* C, const float* bias,
                        double* key, double* probs, uint8_t* taken,
                        int32_t* idx, double* gate, double* margin) {
    const int d = s->d, E = s->E, K = s->K;
    const int sigmoid = (s->flags & ORACLE_SIGMOID) != 0;
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        const uint16_t* c = C + (size_t)e * d;
        for (int j = 0; j < d; ++j) acc += x_t[j] * widen(c[j]);
        const double b = bias ? (double)bias[e] : 0.0;
        if (sigmoid) {
            probs[e] = 1.0 / (1.0 + exp(-acc));
            key[e] = probs[e] + b;
        } else {
            probs[e] = acc + b;              /* the logit, until the softmax below */
        }
    }
    if (!sigmoid) {
        double mx = probs[0];
        for (int e = 1; e < E; ++e)
            if (probs[e] > mx) mx = probs[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            probs[e] = exp(probs[e] - mx);
            z += probs[e];
        }
        for (int e = 0; e < E; ++e) {
            probs[e] /= z;
            key[e] = probs[e];
        }
    }

    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || key[e] > key[best])) best = e;
        taken[best] = 1;
        idx[k] = best;
        gate[k] = probs[best];
    }
    if (s->flags & ORACLE_RENORM) {
        double z = 0.0;
        for (int k = 0; k < K; ++k) z += gate[k];
        for (int k = 0; k < K; ++k) gate[k] /= z;
    }
    if (K == 0 || K == E) {
        *margin = INFINITY;
    } else {
        int next = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (next < 0 || key[e] > key[next])) next = e;
        *margin = key[idx[K - 1]] - key[next];
    }
}

/* OCP FP8 E4M3 code -> value (see the header). */
double oracle_e4m3(uint8_t q) {
    const int sign = q >> 7, e = (q >> 3) & 15, m = q & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Scale exponent of a row of 8-bit activations: the smallest integer e
 * with amax <= 448 * 2^e (0 when amax is 0). */
int32_t oracle_act8_exponent(double amax) {
    if (!(amax > 0.0)) return 0;
    int e = (int)ceil(log2(amax / 448.0));
    while (ldexp(448.0, e) < amax) ++e;
    while (ldexp(448.0, e - 1) >= amax) --e;
    return e;
}

/* The E4M3 code nearest to y (|y| <= 448), ties to the even code: the
 * non-negative finite codes 0x00..0x7E scanned in increasing value. */
uint8_t oracle_e4m3_nearest(double y) {
    const double a = fabs(y);
    int best = 0;
    double bd = INFINITY;
    for (int q = 0; q <= 0x7E; ++q) {
        const double dd = fabs(oracle_e4m3((uint8_t)q) - a);
        if (dd < bd || (dd == bd && (q & 1) == 0)) {
            bd = dd;
            best = q;
        }
    }
    return (uint8_t)(signbit(y) ? (best | 0x80) : best);
}

/* 8-bit activations of n rows (bf16 bits [n, d]): codes [n, d] and the
 * scale exponents [n]. */
void oracle_quantize_act8(const uint16_t* x_rows, int32_t n, int32_t d, uint8_t* codes,
                          int32_t* exps) {
    for (int32_t i = 0; i < n; ++i) {
        double amax = 0.0;
        for (int j = 0; j < d; ++j) {
            const double v = fabs(widen(x_rows[(size_t)i * d + j]));
            if (v > amax) amax = v;
        }
        const int e = oracle_act8_exponent(amax);
        exps[i] = e;
        for (int j = 0; j < d; ++j)
            codes[(size_t)i * d + j] = oracle_e4m3_nearest(ldexp(widen(x_rows[(size_t)i * d + j]), -e));
    }
}

/* v rounded to the nearest bf16 value, ties to the even significand (v
 * finite and below bf16's overflow threshold); returned as bf16 bits.
 * bf16 keeps 8 significant bits for |v| >= 2^-126 and a fixed step of
 * 2^-133 below. */
uint16_t oracle_bf16_nearest(double v) {
    double r;
    if (v == 0.0) {
        r = v;
    } else if (fabs(v) >= ldexp(1.0, -126)) {
        int e2;
        const double f = frexp(v, &e2);            /* |f| in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(f, 8)), e2 - 8);
    } else {
        r = ldexp(nearbyint(ldexp(v, 133)), -133);
    }
    const float fr = (float)r;                     /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &fr, 4);
    return (uint16_t)(u >> 16);
}

/* The 256 code values, filled from oracle_e4m3() before a forward with
 * 8-bit weights reads them (a lookup in place of a decode per use). */
static double e4m3_value[256];

static void e4m3_fill(void) {
    for (int q = 0; q < 256; ++q) e4m3_value[q] = oracle_e4m3((uint8_t)q);
}

/* One weight matrix of `cols` columns: bf16 bit patterns, or 8-bit codes
 * with one float scale per row. */
typedef struct {
    const uint16_t* bf16;
    const uint8_t* q;
    const float* scale;
} wmat;

static double wat(const wmat* w, int row, int cols, int col) {
    const size_t i = (size_t)row * cols + col;
    return w->bf16 ? widen(w->bf16[i]) : e4m3_value[w->q[i]] * (double)w->scale[row];
}

/* Step 4: y = W2 (silu(W1 x) * W3 x) for one token. h: [inter] scratch.
 * hq (bf16 bits [inter]) and q (codes [inter]) non-NULL: 8-bit activations
 * into W2, h rounded to bf16 and quantised as one row (see the header). */
static void expert_ffn(int d, int inter, const wmat* w1, const wmat* w3, const wmat* w2,
                       const double* x_t, double* h, double* y, uint16_t* hq, uint8_t* q) {
    for (int i = 0; i < inter; ++i) {
        double a = 0.0, b = 0.0;
        for (int j = 0; j < d; ++j) {
            a += wat(w1, i, d, j) * x_t[j];
            b += wat(w3, i, d, j) * x_t[j];
        }
        h[i] = silu(a) * b;
    }
    if (hq) {
        int32_t e;
        for (int i = 0; i < inter; ++i) hq[i] = oracle_bf16_nearest(h[i]);
        oracle_quantize_act8(hq, 1, inter, q, &e);
        for (int i = 0; i < inter; ++i) h[i] = ldexp(oracle_e4m3(q[i]), e);
    }
    for (int o = 0; o < d; ++o) {
        double acc = 0.0;
        for (int i = 0; i < inter; ++i) acc += wat(w2, o, inter, i) * h[i];
        y[o] = acc;
    }
}

/* Routing only (steps 1-3) for n_tokens tokens; x_rows holds their rows
 * ([n_tokens, d], bf16).  probs_out may be NULL, else [n_tokens, E]: the
 * scores s_e of step 2. */
int32_t oracle_route(const oracle_shape* s, const uint16_t* x_rows, int32_t n_tokens,
                     const uint16_t* C, const float* bias,
                     int32_t* idx_out, double* gate_out, double* margin_out,
                     double* probs_out, int32_t nthreads) {
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
#pragma omp parallel num_threads(nthreads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* xt = malloc(sizeof(double) * (size_t)s->d);
        double* lg = malloc(sizeof(double) * (size_t)s->E);
        double* pr = malloc(sizeof(double) * (size_t)s->E);
        uint8_t* tk = malloc((size_t)s->E);
#pragma omp for schedule(dynamic, 1)
        for (int32_t i = 0; i < n_tokens; ++i) {
            for (int j = 0; j < s->d; ++j) xt[j] = widen(x_rows[(size_t)i * s->d + j]);
            route_token(s, xt, C, bias, lg, pr, tk, idx_out + (size_t)i * s->K,
                        gate_out + (size_t)i * s->K, margin_out + i);
            if (probs_out) memcpy(probs_out + (size_t)i * s->E, pr, sizeof(double) * (size_t)s->E);
        }
        free(xt); free(lg); free(pr); free(tk);
    }
    return used;
}

/* Full forward (steps 1-5) for n_tokens tokens whose rows are x_rows.
 * rw1/rw3/rw2: the E routed experts' matrices, sw1/sw3/sw2: the Ks shared
 * experts'.  forced_idx ([n_tokens, K] or NULL) replaces the selection of
 * step 3; gates are then the scores of the forced experts (renormalised over
 * them with ORACLE_RENORM).  out, shared_part, routed_part: [n_tokens, d]. */
static int32_t forward_impl(const oracle_shape* s, const uint16_t* x_rows, int32_t n_tokens,
                            const uint16_t* C, const float* bias,
                            const wmat* rw1, const wmat* rw3, const wmat* rw2,
                            const wmat* sw1, const wmat* sw3, const wmat* sw2,
                            const int32_t* forced_idx,
                            double* out, double* shared_part, double* routed_part,
                            int32_t* idx_out, double* gate_out, double* margin_out,
                            int32_t nthreads) {
    const int d = s->d, K = s->K;
    const int hmax = s->I > s->Is ? s->I : s->Is;
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
#pragma omp parallel num_threads(nthreads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* xt = malloc(sizeof(double) * (size_t)d);
        double* xr = malloc(sizeof(double) * (size_t)d);   /* the routed experts' input */
        uint8_t* q = malloc((size_t)(d > hmax ? d : hmax));
        uint16_t* hq = malloc(sizeof(uint16_t) * (size_t)(hmax > 0 ? hmax : 1));
        double* y = malloc(sizeof(double) * (size_t)d);
        double* h = malloc(sizeof(double) * (size_t)(hmax > 0 ? hmax : 1));
        double* lg = malloc(sizeof(double) * (size_t)s->E);
        double* pr = malloc(sizeof(double) * (size_t)s->E);
        uint8_t* tk = malloc((size_t)s->E);
#pragma omp for schedule(dynamic, 1)
        for (int32_t i = 0; i < n_tokens; ++i) {
            int32_t* idx = idx_out + (size_t)i * K;
            double* gate = gate_out + (size_t)i * K;
            double* sh = shared_part + (size_t)i * d;
            double* ro = routed_part + (size_t)i * d;
            for (int j = 0; j < d; ++j) xt[j] = widen(x_rows[(size_t)i * d + j]);
            if (s->flags & ORACLE_ACT8) {
                int32_t e;
                oracle_quantize_act8(x_rows + (size_t)i * d, 1, d, q, &e);
                for (int j = 0; j < d; ++j) xr[j] = ldexp(oracle_e4m3(q[j]), e);
            } else {
                for (int j = 0; j < d; ++j) xr[j] = xt[j];
            }

            route_token(s, xt, C, bias, lg, pr, tk, idx, gate, margin_out + i);
            if (forced_idx) {
                double z = 0.0;
                for (int k = 0; k < K; ++k) {
                    idx[k] = forced_idx[(size_t)i * K + k];
                    gate[k] = pr[idx[k]];
                    z += gate[k];
                }
                if (s->flags & ORACLE_RENORM)
                    for (int k = 0; k < K; ++k) gate[k] /= z;
            }

            for (int j = 0; j < d; ++j) sh[j] = 0.0;
            for (int si = 0; si < s->Ks; ++si) {
                expert_ffn(d, s->Is, &sw1[si], &sw3[si], &sw2[si], xt, h, y, NULL, NULL);
                for (int j = 0; j < d; ++j) sh[j] += y[j];
            }
            for (int j = 0; j < d; ++j) ro[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const int e = idx[k];
                const int a8 = (s->flags & ORACLE_ACT8) != 0;
                expert_ffn(d, s->I, &rw1[e], &rw3[e], &rw2[e], xr, h, y, a8 ? hq : NULL, q);
                for (int j = 0; j < d; ++j) ro[j] += gate[k] * y[j];
            }
            const double res = (s->flags & ORACLE_NO_RESIDUAL) ? 0.0 : 1.0;
            for (int j = 0; j < d; ++j) out[(size_t)i * d + j] = res * xt[j] + sh[j] + ro[j];
        }
        free(xt); free(xr); free(q); free(hq); free(y); free(h); free(lg); free(pr); free(tk);
    }
    return used;
}

static wmat* bf16_mats(const uint16_t* const* w, int n) {
    wmat* m = calloc((size_t)(n > 0 ? n : 1), sizeof(wmat));
    for (int i = 0; i < n; ++i) m[i].bf16 = w ? w[i] : NULL;
    return m;
}

static wmat* fp8_mats(const uint8_t* const* q, const float* const* scale, int n) {
    wmat* m = calloc((size_t)(n > 0 ? n : 1), sizeof(wmat));
    for (int i = 0; i < n; ++i) {
        m[i].q = q[i];
        m[i].scale = scale[i];
    }
    return m;
}

/* Full forward with bf16 weights.  w1[e], w3[e], w2[e]: per routed expert
 * (E of them), ws*[s]: per shared expert (Ks of them); see forward_impl. */
int32_t oracle_forward(const oracle_shape* s, const uint16_t* x_rows, int32_t n_tokens,
                       const uint16_t* C, const float* bias,
                       const uint16_t* const* w1, const uint16_t* const* w3,
                       const uint16_t* const* w2,
                       const uint16_t* const* ws1, const uint16_t* const* ws3,
                       const uint16_t* const* ws2,
                       const int32_t* forced_idx,
                       double* out, double* shared_part, double* routed_part,
                       int32_t* idx_out, double* gate_out, double* margin_out,
                       int32_t nthreads) {
    wmat *r1 = bf16_mats(w1, s->E), *r3 = bf16_mats(w3, s->E), *r2 = bf16_mats(w2, s->E);
    wmat *h1 = bf16_mats(ws1, s->Ks), *h3 = bf16_mats(ws3, s->Ks), *h2 = bf16_mats(ws2, s->Ks);
    const int32_t used = forward_impl(s, x_rows, n_tokens, C, bias, r1, r3, r2, h1, h3, h2,
                                      forced_idx, out, shared_part, routed_part, idx_out,
                                      gate_out, margin_out, nthreads);
    free(r1); free(r3); free(r2); free(h1); free(h3); free(h2);
    return used;
}

/* Full forward with 8-bit routed weights: q1[e], q3[e] [I, d] and q2[e]
 * [d, I] codes with per-row scales s1[e], s3[e] [I] and s2[e] [d]; the
 * shared experts ws*[s] stay bf16. */
int32_t oracle_forward_fp8(const oracle_shape* s, const uint16_t* x_rows, int32_t n_tokens,
                           const uint16_t* C, const float* bias,
                           const uint8_t* const* q1, const float* const* s1,
                           const uint8_t* const* q3, const float* const* s3,
                           const uint8_t* const* q2, const float* const* s2,
                           const uint16_t* const* ws1, const uint16_t* const* ws3,
                           const uint16_t* const* ws2,
                           const int32_t* forced_idx,
                           double* out, double* shared_part, double* routed_part,
                           int32_t* idx_out, double* gate_out, double* margin_out,
                           int32_t nthreads) {
    e4m3_fill();
    wmat *r1 = fp8_mats(q1, s1, s->E), *r3 = fp8_mats(q3, s3, s->E), *r2 = fp8_mats(q2, s2, s->E);
    wmat *h1 = bf16_mats(ws1, s->Ks), *h3 = bf16_mats(ws3, s->Ks), *h2 = bf16_mats(ws2, s->Ks);
    const int32_t used = forward_impl(s, x_rows, n_tokens, C, bias, r1, r3, r2, h1, h3, h2,
                                      forced_idx, out, shared_part, routed_part, idx_out,
                                      gate_out, margin_out, nthreads);
    free(r1); free(r3); free(r2); free(h1); free(h3); free(h2);
    return used;
}

/* ------------------------------------------------------------------------
 * Backward of the layer (the training side), for a given upstream gradient.
 *
 * Objective whose gradients are returned:
 *
 *   Lambda = sum_{t,j} dout[t,j] * out[t,j]  +  alpha * L_bal
 *
 * dout is the upstream gradient dLoss/dout (bf16, as the GPU receives it).
 * L_bal is the expert-level balance loss of "DeepSeekMoE 深度解读报告"
 * (sections 2.5 and 3.2): over the batch, each expert's hit rate and mean
 * gate score are taken, and their agreement with a uniform load is
 * penalised with a small factor alpha.  The pages name the two statistics
 * but print no formula; the reading here is
 *
 *   f_e = E * count_e / (K * T)         hit rate, 1 for a perfectly even load
 *   P_e = (1/T) * sum_t s_{t,e}         mean score (the full softmax or
 *                                       sigmoid score of step 2, before any
 *                                       renormalisation)
 *   L_bal = sum_e f_e * P_e
 *
 * with f_e held fixed (a count is piecewise constant in the inputs).  The
 * top-K choice is piecewise constant too, so no gradient flows through it;
 * gradients reach the affinities through the kept gates (and through every
 * score via L_bal).  The per-expert logit bias is a fixed input and gets no
 * gradient.
 *
 * Per token t (x = x[t], dO = dout[t]) and per expert with weight
 * matrices W1, W3 [inter, d], W2 [d, inter] and gate g (1 for a shared
 * expert), from step 4 of the forward:
 *
 *   a = W1 x,  b = W3 x,  h = silu(a) * b,  y = W2 h
 *   dgate   = <dO, y>                          (routed experts)
 *   dh      = g * W2^T dO
 *   silu'(a) = sig(a) * (1 + a * (1 - sig(a))),  sig(a) = 1 / (1 + e^-a)
 *   da      = dh * b * silu'(a),   db = dh * silu(a)
 *   dx     += W1^T da + W3^T db
 *   dW2    += g * dO (x) h,   dW1 += da (x) x,   dW3 += db (x) x
 *
 * and for the router, from steps 2 and 3 (s: the E scores of the token):
 *
 *   gate -> score:  ds_{e_k} = dgate_k (plain gates), or, with
 *                   ORACLE_RENORM (gate_k = s_{e_k} / Z, Z = sum_m s_{e_m}),
 *                   ds_{e_k} = (dgate_k - sum_m dgate_m * gate_m) / Z;
 *                   0 for experts not kept
 *   balance:        ds_e += alpha * f_e / T           (every expert)
 *   score -> affinity:
 *       softmax     dl_j = s_j * (ds_j - sum_e s_e * ds_e)
 *       sigmoid     dl_j = s_j * (1 - s_j) * ds_j
 *   dx += sum_j dl_j C_j,   dC_j += dl_j x            (C: the centroids)
 *
 * plus dx += dO for the residual (unless ORACLE_NO_RESIDUAL).
 * ------------------------------------------------------------------------ */

static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Per (token, expert) pieces of the expert backward: a, b and dh (= g W2^T
 * dO); dgate_out (if not NULL) = <dO, W2 h>. */
static void expert_bwd_vectors(int d, int inter, const uint16_t* w1, const uint16_t* w3,
                               const uint16_t* w2, const double* x_t, const double* dO,
                               double g, double* a, double* b, double* h, double* dh,
                               double* dgate_out) {
    for (int i = 0; i < inter; ++i) {
        double sa = 0.0, sb = 0.0;
        for (int j = 0; j < d; ++j) {
            sa += widen(w1[(size_t)i * d + j]) * x_t[j];
            sb += widen(w3[(size_t)i * d + j]) * x_t[j];
        }
        a[i] = sa;
        b[i] = sb;
        h[i] = silu(sa) * sb;
        dh[i] = 0.0;
    }
    double dg = 0.0;
    for (int o = 0; o < d; ++o) {
        double y = 0.0;
        const uint16_t* row = w2 + (size_t)o * inter;
        for (int i = 0; i < inter; ++i) {
            const double w = widen(row[i]);
            y += w * h[i];
            dh[i] += w * dO[o];
        }
        dg += dO[o] * y;
    }
    for (int i = 0; i < inter; ++i) dh[i] *= g;
    if (dgate_out) *dgate_out = dg;
}

/* da, db from a, b, dh (in place: a -> da, b -> db). */
static void swiglu_bwd(int inter, double* a, double* b, const double* dh) {
    for (int i = 0; i < inter; ++i) {
        const double sg = sigm(a[i]);
        const double dsilu = sg * (1.0 + a[i] * (1.0 - sg));
        const double da = dh[i] * b[i] * dsilu;
        const double db = dh[i] * (a[i] * sg);
        a[i] = da;
        b[i] = db;
    }
}

/* dx += W1^T da + W3^T db */
static void expert_dx(int d, int inter, const uint16_t* w1, const uint16_t* w3,
                      const double* da, const double* db, double* dx) {
    for (int i = 0; i < inter; ++i) {
        const uint16_t* r1 = w1 + (size_t)i * d;
        const uint16_t* r3 = w3 + (size_t)i * d;
        for (int j = 0; j < d; ++j) dx[j] += widen(r1[j]) * da[i] + widen(r3[j]) * db[i];
    }
}

/* Weight gradients of one expert over its tokens (in token order).  xs
 * [n, d], dOs [n, d] and gs [n] are the tokens' rows, upstream gradients
 * and gates; dw1, dw3 [inter, d], dw2 [d, inter] are written. */
static void expert_dw(int d, int inter, const uint16_t* w1, const uint16_t* w3,
                      const uint16_t* w2, int n, const double* xs, const double* dOs,
                      const double* gs, double* dw1, double* dw3, double* dw2, int nthreads) {
    double* A = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * inter);   /* -> da */
    double* B = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * inter);   /* -> db */
    double* Hh = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * inter);  /* g * h */
#pragma omp parallel num_threads(nthreads)
    {
        double* dh = malloc(sizeof(double) * (size_t)inter);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n; ++t) {
            double* a = A + (size_t)t * inter;
            double* b = B + (size_t)t * inter;
            double* h = Hh + (size_t)t * inter;
            expert_bwd_vectors(d, inter, w1, w3, w2, xs + (size_t)t * d, dOs + (size_t)t * d,
                               gs[t], a, b, h, dh, NULL);
            swiglu_bwd(inter, a, b, dh);
            for (int i = 0; i < inter; ++i) h[i] *= gs[t];
        }
        free(dh);
        /* each output row is owned by one thread; tokens summed in order */
#pragma omp for schedule(static)
        for (int i = 0; i < inter; ++i) {
            double* r1 = dw1 + (size_t)i * d;
            double* r3 = dw3 + (size_t)i * d;
            for (int j = 0; j < d; ++j) r1[j] = r3[j] = 0.0;
            for (int t = 0; t < n; ++t) {
                const double da = A[(size_t)t * inter + i], db = B[(size_t)t * inter + i];
                const double* xt = xs + (size_t)t * d;
                for (int j = 0; j < d; ++j) {
                    r1[j] += da * xt[j];
                    r3[j] += db * xt[j];
                }
            }
        }
#pragma omp for schedule(static)
        for (int o = 0; o < d; ++o) {
            double* r2 = dw2 + (size_t)o * inter;
            for (int i = 0; i < inter; ++i) r2[i] = 0.0;
            for (int t = 0; t < n; ++t) {
                const double go = dOs[(size_t)t * d + o];
                const double* h = Hh + (size_t)t * inter;
                for (int i = 0; i < inter; ++i) r2[i] += go * h[i];
            }
        }
    }
    free(A); free(B); free(Hh);
}

/* Backward of the layer on a batch of T tokens (x_all, dout_all: [T, d]
 * bf16).  Outputs, each only where asked:
 *   tok[n_tok]:  dx [n_tok, d], dgate [n_tok, K] (d Lambda / d gate_k),
 *                idx [n_tok, K] (the routing they were taken under)
 *   exps[n_exp]: dw1, dw3 [n_exp, I, d], dw2 [n_exp, d, I] of those routed
 *                experts
 *   want_shared: dws1, dws3 [Ks, Is, d], dws2 [Ks, d, Is]
 *   want_dC:     dC [E, d]
 *   always:      counts [E], mean_score [E] (P_e), bal [2] = {L_bal, alpha * L_bal}
 * forced_idx ([T, K] or NULL) replaces the selection as in the forward. */
int32_t oracle_backward(const oracle_shape* s, const uint16_t* x_all, int32_t T,
                        const uint16_t* C, const float* bias,
                        const uint16_t* const* w1, const uint16_t* const* w3,
                        const uint16_t* const* w2,
                        const uint16_t* const* ws1, const uint16_t* const* ws3,
                        const uint16_t* const* ws2,
                        const uint16_t* dout_all, double alpha, const int32_t* forced_idx,
                        const int32_t* tok, int32_t n_tok, const int32_t* exps, int32_t n_exp,
                        int32_t want_shared, int32_t want_dC,
                        double* dx, double* dgate, int32_t* idx_out,
                        double* dw1, double* dw3, double* dw2,
                        double* dws1, double* dws3, double* dws2, double* dC,
                        int64_t* counts, double* mean_score, double* bal, int32_t nthreads) {
    const int d = s->d, E = s->E, K = s->K, I = s->I, Ks = s->Ks, Is = s->Is;
    const int ren = (s->flags & ORACLE_RENORM) != 0, sig = (s->flags & ORACLE_SIGMOID) != 0;
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    /* Pass 1: routing of every token (scores, kept experts and gates). */
    int32_t* idx_all = malloc(sizeof(int32_t) * (size_t)T * (K > 0 ? K : 1));
    double* gate_all = malloc(sizeof(double) * (size_t)T * (K > 0 ? K : 1));
    double* prob_all = malloc(sizeof(double) * (size_t)T * E);
#pragma omp parallel num_threads(nthreads)
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* xt = malloc(sizeof(double) * (size_t)d);
        double* key = malloc(sizeof(double) * (size_t)E);
        uint8_t* tk = malloc((size_t)E);
        double margin;
#pragma omp for schedule(dynamic, 4)
        for (int32_t t = 0; t < T; ++t) {
            for (int j = 0; j < d; ++j) xt[j] = widen(x_all[(size_t)t * d + j]);
            int32_t* idx = idx_all + (size_t)t * K;
            double* gate = gate_all + (size_t)t * K;
            double* pr = prob_all + (size_t)t * E;
            route_token(s, xt, C, bias, key, pr, tk, idx, gate, &margin);
            if (forced_idx) {
                double z = 0.0;
                for (int k = 0; k < K; ++k) {
                    idx[k] = forced_idx[(size_t)t * K + k];
                    gate[k] = pr[idx[k]];
                    z += gate[k];
                }
                if (ren)
                    for (int k = 0; k < K; ++k) gate[k] /= z;
            }
        }
        free(xt); free(key); free(tk);
    }
    /* balance statistics, summed in token order */
    double* fe = malloc(sizeof(double) * (size_t)E);
    for (int e = 0; e < E; ++e) {
        counts[e] = 0;
        mean_score[e] = 0.0;
    }
    for (int32_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) counts[idx_all[(size_t)t * K + k]] += 1;
        for (int e = 0; e < E; ++e) mean_score[e] += prob_all[(size_t)t * E + e];
    }
    double lb = 0.0;
    for (int e = 0; e < E; ++e) {
        mean_score[e] /= (double)T;
        fe[e] = K > 0 ? (double)E * (double)counts[e] / ((double)K * (double)T) : 0.0;
        lb += fe[e] * mean_score[e];
    }
    bal[0] = lb;
    bal[1] = alpha * lb;

    /* Pass 2: per token — expert backward (dx, dgate) and router backward
     * (dl).  dl is kept for every token when dC is wanted. */
    int32_t n_rt = want_dC ? T : n_tok;                  /* tokens taken through pass 2 */
    int32_t* rt = malloc(sizeof(int32_t) * (size_t)(n_rt > 0 ? n_rt : 1));
    int32_t* slot = malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));   /* token -> tok[] position */
    for (int32_t t = 0; t < T; ++t) slot[t] = -1;
    for (int32_t i = 0; i < n_tok; ++i) slot[tok[i]] = i;
    for (int32_t i = 0; i < n_rt; ++i) rt[i] = want_dC ? i : tok[i];
    double* dl_all = want_dC ? malloc(sizeof(double) * (size_t)T * E) : NULL;
    const int hmax = I > Is ? I : Is;
#pragma omp parallel num_threads(nthreads)
    {
        double* xt = malloc(sizeof(double) * (size_t)d);
        double* dO = malloc(sizeof(double) * (size_t)d);
        double* acc = malloc(sizeof(double) * (size_t)d);
        double* a = malloc(sizeof(double) * (size_t)hmax);
        double* b = malloc(sizeof(double) * (size_t)hmax);
        double* h = malloc(sizeof(double) * (size_t)hmax);
        double* dh = malloc(sizeof(double) * (size_t)hmax);
        double* dg = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* ds = malloc(sizeof(double) * (size_t)E);
        double* dl = malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(dynamic, 1)
        for (int32_t i = 0; i < n_rt; ++i) {
            const int32_t t = rt[i];
            const int32_t out_i = slot[t];               /* -1: dl only (for dC) */
            for (int j = 0; j < d; ++j) {
                xt[j] = widen(x_all[(size_t)t * d + j]);
                dO[j] = widen(dout_all[(size_t)t * d + j]);
                acc[j] = (s->flags & ORACLE_NO_RESIDUAL) ? 0.0 : dO[j];
            }
            const int32_t* idx = idx_all + (size_t)t * K;
            const double* gate = gate_all + (size_t)t * K;
            const double* pr = prob_all + (size_t)t * E;
            for (int si = 0; si < Ks && out_i >= 0; ++si) {
                expert_bwd_vectors(d, Is, ws1[si], ws3[si], ws2[si], xt, dO, 1.0, a, b, h, dh, NULL);
                swiglu_bwd(Is, a, b, dh);
                expert_dx(d, Is, ws1[si], ws3[si], a, b, acc);
            }
            for (int k = 0; k < K; ++k) {
                const int e = idx[k];
                expert_bwd_vectors(d, I, w1[e], w3[e], w2[e], xt, dO, gate[k], a, b, h, dh, &dg[k]);
                if (out_i >= 0) {
                    swiglu_bwd(I, a, b, dh);
                    expert_dx(d, I, w1[e], w3[e], a, b, acc);
                }
            }
            /* router: gates -> scores -> affinities */
            for (int e = 0; e < E; ++e) ds[e] = K > 0 ? alpha * fe[e] / (double)T : 0.0;
            if (ren) {
                double z = 0.0, sg = 0.0;
                for (int k = 0; k < K; ++k) {
                    z += pr[idx[k]];
                    sg += dg[k] * gate[k];
                }
                for (int k = 0; k < K; ++k) ds[idx[k]] += (dg[k] - sg) / z;
            } else {
                for (int k = 0; k < K; ++k) ds[idx[k]] += dg[k];
            }
            if (sig) {
                for (int e = 0; e < E; ++e) dl[e] = pr[e] * (1.0 - pr[e]) * ds[e];
            } else {
                double m = 0.0;
                for (int e = 0; e < E; ++e) m += pr[e] * ds[e];
                for (int e = 0; e < E; ++e) dl[e] = pr[e] * (ds[e] - m);
            }
            if (K == 0)
                for (int e = 0; e < E; ++e) dl[e] = 0.0;
            if (dl_all) memcpy(dl_all + (size_t)t * E, dl, sizeof(double) * (size_t)E);
            if (out_i >= 0) {
                for (int e = 0; e < E && K > 0; ++e) {
                    const uint16_t* c = C + (size_t)e * d;
                    for (int j = 0; j < d; ++j) acc[j] += dl[e] * widen(c[j]);
                }
                memcpy(dx + (size_t)out_i * d, acc, sizeof(double) * (size_t)d);
                for (int k = 0; k < K; ++k) {
                    dgate[(size_t)out_i * K + k] = dg[k];
                    idx_out[(size_t)out_i * K + k] = idx[k];
                }
            }
        }
        free(xt); free(dO); free(acc); free(a); free(b); free(h); free(dh); free(dg); free(ds);
        free(dl);
    }

    /* Pass 3: weight gradients of the requested routed experts and of the
     * shared experts, each over its tokens in token order. */
    for (int32_t q = 0; q < n_exp + (want_shared ? Ks : 0); ++q) {
        const int shared = q >= n_exp;
        const int e = shared ? q - n_exp : exps[q];
        const int inter = shared ? Is : I;
        int n = 0;
        for (int32_t t = 0; t < T; ++t) {
            if (shared) { ++n; continue; }
            for (int k = 0; k < K; ++k) n += idx_all[(size_t)t * K + k] == e;
        }
        double* xs = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
        double* dOs = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
        double* gs = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int r = 0;
        for (int32_t t = 0; t < T; ++t) {
            double g = -1.0;
            if (shared) g = 1.0;
            else
                for (int k = 0; k < K; ++k)
                    if (idx_all[(size_t)t * K + k] == e) g = gate_all[(size_t)t * K + k];
            if (g < 0.0) continue;
            for (int j = 0; j < d; ++j) {
                xs[(size_t)r * d + j] = widen(x_all[(size_t)t * d + j]);
                dOs[(size_t)r * d + j] = widen(dout_all[(size_t)t * d + j]);
            }
            gs[r++] = g;
        }
        if (shared)
            expert_dw(d, inter, ws1[e], ws3[e], ws2[e], n, xs, dOs, gs,
                      dws1 + (size_t)e * inter * d, dws3 + (size_t)e * inter * d,
                      dws2 + (size_t)e * d * inter, nthreads);
        else
            expert_dw(d, inter, w1[e], w3[e], w2[e], n, xs, dOs, gs,
                      dw1 + (size_t)q * inter * d, dw3 + (size_t)q * inter * d,
                      dw2 + (size_t)q * d * inter, nthreads);
        free(xs); free(dOs); free(gs);
    }

    /* Pass 4: centroid gradients, tokens summed in order. */
    if (want_dC) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int e = 0; e < E; ++e) {
            double* row = dC + (size_t)e * d;
            for (int j = 0; j < d; ++j) row[j] = 0.0;
            for (int32_t t = 0; t < T; ++t) {
                const double g = dl_all[(size_t)t * E + e];
                const uint16_t* xr = x_all + (size_t)t * d;
                for (int j = 0; j < d; ++j) row[j] += g * widen(xr[j]);
            }
        }
    }
    free(idx_all); free(gate_all); free(prob_all); free(fe); free(rt); free(slot); free(dl_all);
    return used;
}
