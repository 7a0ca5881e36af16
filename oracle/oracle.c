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

/* One weight matrix of `cols` columns: bf16 bit patterns, or 8-bit codes
 * with one float scale per row. */
typedef struct {
    const uint16_t* bf16;
    const uint8_t* q;
    const float* scale;
} wmat;

static double wat(const wmat* w, int row, int cols, int col) {
    const size_t i = (size_t)row * cols + col;
    return w->bf16 ? widen(w->bf16[i]) : oracle_e4m3(w->q[i]) * (double)w->scale[row];
}

/* Step 4: y = W2 (silu(W1 x) * W3 x) for one token. h: [inter] scratch. */
static void expert_ffn(int d, int inter, const wmat* w1, const wmat* w3, const wmat* w2,
                       const double* x_t, double* h, double* y) {
    for (int i = 0; i < inter; ++i) {
        double a = 0.0, b = 0.0;
        for (int j = 0; j < d; ++j) {
            a += wat(w1, i, d, j) * x_t[j];
            b += wat(w3, i, d, j) * x_t[j];
        }
        h[i] = silu(a) * b;
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
                expert_ffn(d, s->Is, &sw1[si], &sw3[si], &sw2[si], xt, h, y);
                for (int j = 0; j < d; ++j) sh[j] += y[j];
            }
            for (int j = 0; j < d; ++j) ro[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const int e = idx[k];
                expert_ffn(d, s->I, &rw1[e], &rw3[e], &rw2[e], xt, h, y);
                for (int j = 0; j < d; ++j) ro[j] += gate[k] * y[j];
            }
            const double res = (s->flags & ORACLE_NO_RESIDUAL) ? 0.0 : 1.0;
            for (int j = 0; j < d; ++j) out[(size_t)i * d + j] = res * xt[j] + sh[j] + ro[j];
        }
        free(xt); free(y); free(h); free(lg); free(pr); free(tk);
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
    wmat *r1 = fp8_mats(q1, s1, s->E), *r3 = fp8_mats(q3, s3, s->E), *r2 = fp8_mats(q2, s2, s->E);
    wmat *h1 = bf16_mats(ws1, s->Ks), *h3 = bf16_mats(ws3, s->Ks), *h2 = bf16_mats(ws2, s->Ks);
    const int32_t used = forward_impl(s, x_rows, n_tokens, C, bias, r1, r3, r2, h1, h3, h2,
                                      forced_idx, out, shared_part, routed_part, idx_out,
                                      gate_out, margin_out, nthreads);
    free(r1); free(r3); free(r2); free(h1); free(h3); free(h2);
    return used;
}
