/*
 * oracle.c -- plain fp64 CPU oracle for the selected-token log-probability.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product library
 * (the HIP path) never links, calls or includes anything from this directory,
 * and this file includes nothing from the product either: the two share no
 * code, no headers, no constants.
 *
 * What it computes (the method's definition, written out):
 *   For hidden states h[T][H] and LM-head weight w[V][H], both given as
 *   bfloat16 bit patterns, and target ids y[T]:
 *     z[t][v]  = sum_k h[t][k] * w[v][k]                (logits)
 *     lse[t]   = log sum_v exp(z[t][v])                 (log-sum-exp over the
 *                                                        whole vocabulary)
 *     logp[t]  = z[t][y[t]] - lse[t]                    (log-softmax read at
 *                                                        the target token)
 *   Source: RL-Kernel blog (princepride.github.io, "RL-Kernel ... LogP"),
 *   section 四 ("five reduction classes"): the Linear-LogP class reduces over
 *   the vocabulary, the selected token's log-probability depends on the LSE of
 *   all vocabulary scores, and the LSE is evaluated in its stabilised form
 *   m + log sum exp(x_i - m) with m = max_i x_i.  Section 一 names the
 *   quantity: the log-probability of the selected (sampled) token.
 *
 * How (plainly, in fp64):
 *   - bf16 -> fp64 is exact (bits << 16 reinterpreted as fp32, then widened).
 *   - Each logit is one dot product accumulated in fp64 in increasing k, one
 *     multiply and one add per k.  A product of two bf16 values carries at most
 *     16 significant bits, so it is exact in fp64; only the additions round.
 *     For speed, eight independent dot products (eight vocabulary rows) are
 *     advanced together, each still in increasing k; this interleaving of
 *     independent sums changes no result bit relative to the one-at-a-time
 *     loop (the tests check that too).
 *   - m = max over the row, s = sum_v exp(z - m) sequentially in v,
 *     lse = m + log(s).
 *   - OpenMP over rows; every row is computed by one thread in a fixed order,
 *     so results do not depend on the thread count.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - Non-finite logits: a NaN or +Inf logit anywhere in a row makes that
 *     row's lse and logp NaN.  -Inf logits carry probability zero and add
 *     nothing to the sum; a row whose logits are all -Inf has lse = -Inf and
 *     logp = NaN.
 *   - A target outside [0, V) gives logp = NaN; lse is still produced.
 *   - The LSE covers exactly the V rows of w that are passed.
 *
 * Variants of the same quantity (oracle_selected_logp_ex), for the contract
 * options of the product library:
 *   - Temperature: every logit is multiplied by inv_tau = 1/tau before
 *     anything else (sampling at temperature tau draws from softmax(z / tau);
 *     training must score the same distribution).
 *   - bfloat16 logits: engines that hold their logits as a bf16 tensor round
 *     each (scaled) logit to bf16 before the softmax.  The RL-Kernel blog
 *     (sections 二 and 四) names this fp32 -> bf16 conversion point as one of
 *     the places where training and inference drift apart.  The rounding is
 *     to nearest, ties to even, taken on the logit as an fp32 value (the
 *     precision in which an engine holds it before the cast): fp64 logit ->
 *     nearest fp32 -> nearest bf16.
 *   - Backward (oracle_selected_logp_backward): for an upstream gradient
 *     g[t] = dL/dlogp[t], the gradient of L = sum_t g[t] logp[t] with respect
 *     to the logits is dz[t][v] = g[t] inv_tau (1[v == y_t] - p[t][v]),
 *     p = softmax(z'), and by the chain rule through z = h w^T:
 *       grad_hidden[t][k] = sum_v dz[t][v] w[v][k],
 *       grad_weight[v][k] = sum_t dz[t][v] h[t][k].
 *     A row whose target lies outside [0, V) has no log-probability to
 *     differentiate (its logp is NaN); it contributes no gradient (dz = 0),
 *     like an ignored index.  The training side of the vLLM blog summary
 *     differentiates the logprob it recomputes in a graph; the backward is
 *     verified on its own (its C7 check).
 *   - RMSNorm feeding the LM head (oracle_rmsnorm): the RL-Kernel blog
 *     (section 四) puts RMSNorm among the reductions whose result depends on
 *     the order of accumulation over the hidden dimension, and its H100
 *     recipe (section 六) switches to torch's RMSNorm for one normalisation
 *     semantics.  The model's convention, taken here: per row
 *     r = 1 / sqrt(mean_k x_k^2 + eps), y_k = bf16(bf16(x_k r) gamma_k);
 *     the first rounding is decided on x_k r as an fp32 value (fp64 -> fp32
 *     -> bf16, the precision the normalisation runs in), the second on the
 *     product of two bf16 values, which is exact.
 *   - Top-k log-probabilities (oracle_topk_logp): the k entries of
 *     log softmax(z') with the largest values, in decreasing order, ties
 *     broken by the smaller token id; NaN entries are never selected.  The
 *     vLLM blog summary counts them among the per-token outputs an RL step
 *     reads (its logprob outputs).
 *   - Entropy of softmax(z'): H = -sum_v p_v log p_v with
 *     p_v = exp(z'_v - lse), terms with p_v = 0 contributing 0; NaN when the
 *     row's lse is not finite.  (The vLLM blog summary lists entropy among the
 *     per-token quantities an RL step reads from these logits.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VERSION 5

int oracle_version(void) { return ORACLE_VERSION; }

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* bfloat16 bit pattern -> fp64, exactly. */
static double bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One row of logits: z[v] = sum_k h[k] * w[v][k] for v in [0, V), each sum in
 * increasing k.  h is already fp64 (exact copy of the bf16 row). */
static void row_logits(const double *h, const uint16_t *w, int64_t ldw,
                       int64_t H, int64_t V, double *z) {
    int64_t v = 0;
    for (; v + 8 <= V; v += 8) {
        const uint16_t *w0 = w + (v + 0) * ldw, *w1 = w + (v + 1) * ldw;
        const uint16_t *w2 = w + (v + 2) * ldw, *w3 = w + (v + 3) * ldw;
        const uint16_t *w4 = w + (v + 4) * ldw, *w5 = w + (v + 5) * ldw;
        const uint16_t *w6 = w + (v + 6) * ldw, *w7 = w + (v + 7) * ldw;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        double a4 = 0.0, a5 = 0.0, a6 = 0.0, a7 = 0.0;
        for (int64_t k = 0; k < H; ++k) {
            const double hk = h[k];
            a0 = a0 + hk * bf16_to_f64(w0[k]);
            a1 = a1 + hk * bf16_to_f64(w1[k]);
            a2 = a2 + hk * bf16_to_f64(w2[k]);
            a3 = a3 + hk * bf16_to_f64(w3[k]);
            a4 = a4 + hk * bf16_to_f64(w4[k]);
            a5 = a5 + hk * bf16_to_f64(w5[k]);
            a6 = a6 + hk * bf16_to_f64(w6[k]);
            a7 = a7 + hk * bf16_to_f64(w7[k]);
        }
        z[v + 0] = a0; z[v + 1] = a1; z[v + 2] = a2; z[v + 3] = a3;
        z[v + 4] = a4; z[v + 5] = a5; z[v + 6] = a6; z[v + 7] = a7;
    }
    for (; v < V; ++v) {
        const uint16_t *wv = w + v * ldw;
        double a = 0.0;
        for (int64_t k = 0; k < H; ++k) a = a + h[k] * bf16_to_f64(wv[k]);
        z[v] = a;
    }
}

/* The reference one-at-a-time dot product, kept only so the tests can check
 * that the interleaved loop above reproduces it bit for bit. */
static double dot_naive(const double *h, const uint16_t *wv, int64_t H) {
    double a = 0.0;
    for (int64_t k = 0; k < H; ++k) a = a + h[k] * bf16_to_f64(wv[k]);
    return a;
}

/* lse and logp of one row of logits (policy for non-finite values above). */
static void row_lse_logp(const double *z, int64_t V, int64_t y,
                         double *lse_out, double *logp_out) {
    double m = -INFINITY;
    int bad = 0;
    for (int64_t v = 0; v < V; ++v) {
        const double x = z[v];
        if (isnan(x) || x == INFINITY) bad = 1;
        else if (x > m) m = x;
    }
    if (bad) { *lse_out = NAN; *logp_out = NAN; return; }
    if (m == -INFINITY) { *lse_out = -INFINITY; *logp_out = NAN; return; }
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s = s + exp(z[v] - m);
    const double lse = m + log(s);
    *lse_out = lse;
    *logp_out = (y >= 0 && y < V) ? z[y] - lse : NAN;
}

/* fp64 -> bfloat16 value, round to nearest, ties to even, from the format's
 * definition: 8 significant bits, exponent range of fp32 (normal numbers down
 * to 2^-126, subnormals spaced 2^-133), largest finite (2 - 2^-7) 2^127;
 * values at or beyond the rounding boundary above it become infinities. */
static double round_bf16(double x) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    (void)frexp(x, &e);                 /* |x| = f 2^e, f in [0.5, 1) */
    int q = e - 8;                      /* spacing of 8-bit significands */
    if (q < -133) q = -133;             /* subnormal spacing */
    const double step = ldexp(1.0, q);
    const double n = x / step;          /* exact: a power-of-two division */
    double r = floor(n);
    const double frac = n - r;          /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double y = r * step;
    const double max_finite = ldexp(255.0, 120);   /* (2 - 2^-7) 2^127 */
    if (fabs(y) > max_finite) return x > 0 ? INFINITY : -INFINITY;
    return copysign(y, x);              /* a negative value rounded to 0 is -0 */
}

/* The logit as an engine holds it before a bf16 cast: nearest fp32. */
static double to_f32(double x) { return (double)(float)x; }

/* Apply the contract options to one row of fp64 logits, in place. */
static void row_transform(double *z, int64_t V, double inv_tau, int bf16) {
    for (int64_t v = 0; v < V; ++v) {
        double x = z[v] * inv_tau;
        if (bf16) x = round_bf16(to_f32(x));
        z[v] = x;
    }
}

/* Entropy of softmax(z) given its lse (finite), terms with p = 0 skipped. */
static double row_entropy(const double *z, int64_t V, double lse) {
    if (!isfinite(lse)) return NAN;
    double h = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        if (z[v] == -INFINITY) continue;
        const double lp = z[v] - lse;
        const double p = exp(lp);
        if (p == 0.0) continue;
        h = h - p * lp;
    }
    return h;
}

static void hidden_row(const uint16_t *hidden, int64_t ldh, int64_t t,
                       int64_t H, double *h) {
    const uint16_t *src = hidden + t * ldh;
    for (int64_t k = 0; k < H; ++k) h[k] = bf16_to_f64(src[k]);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Logits z[t][v] (row-major [T][V]).  Returns 0, or -1 on allocation failure. */
int oracle_logits(const uint16_t *hidden, int64_t ldh, const uint16_t *weight,
                  int64_t ldw, int64_t T, int64_t H, int64_t V, double *z,
                  int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        if (!h) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z + t * V);
            }
        }
        free(h);
    }
    return fail ? -1 : 0;
}

/* Same logits, one dot product at a time (test of the interleaving only). */
int oracle_logits_naive(const uint16_t *hidden, int64_t ldh,
                        const uint16_t *weight, int64_t ldw, int64_t T,
                        int64_t H, int64_t V, double *z) {
    double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
    if (!h) return -1;
    for (int64_t t = 0; t < T; ++t) {
        hidden_row(hidden, ldh, t, H, h);
        for (int64_t v = 0; v < V; ++v)
            z[t * V + v] = dot_naive(h, weight + v * ldw, H);
    }
    free(h);
    return 0;
}

/* lse / logp from logits given directly (row-major [T][V]). */
void oracle_lse_from_logits(const double *z, const int32_t *targets, int64_t T,
                            int64_t V, double *logp, double *lse) {
    for (int64_t t = 0; t < T; ++t)
        row_lse_logp(z + t * V, V, (int64_t)targets[t], &lse[t], &logp[t]);
}

/* The whole path: logits, vocabulary LSE, gather.  Returns 0 or -1. */
int oracle_selected_logp(const uint16_t *hidden, int64_t ldh,
                         const uint16_t *weight, int64_t ldw,
                         const int32_t *targets, int64_t T, int64_t H,
                         int64_t V, double *logp, double *lse, int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        if (!h || !z) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z);
                row_lse_logp(z, V, (int64_t)targets[t], &lse[t], &logp[t]);
            }
        }
        free(h);
        free(z);
    }
    return fail ? -1 : 0;
}

/* Full-row log-softmax out[t][v] = z[t][v] - lse[t] (test use: sum-to-one
 * checks and drawing targets from the model's distribution). */
int oracle_log_softmax(const uint16_t *hidden, int64_t ldh,
                       const uint16_t *weight, int64_t ldw, int64_t T,
                       int64_t H, int64_t V, double *out, int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        if (!h) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                double *z = out + t * V;
                double lse, logp;
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z);
                row_lse_logp(z, V, 0, &lse, &logp);
                for (int64_t v = 0; v < V; ++v) z[v] = z[v] - lse;
            }
        }
        free(h);
    }
    return fail ? -1 : 0;
}

/* Round fp32 values to bfloat16 (test of the rounding on its own). */
void oracle_round_bf16(const float *x, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_bf16((double)x[i]);
}

/* lse / logp / entropy from logits given directly, after the options. */
void oracle_ex_from_logits(const double *z_in, const int32_t *targets, int64_t T,
                           int64_t V, double inv_tau, int bf16, double *logp,
                           double *lse, double *entropy) {
    double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    if (!z) return;
    for (int64_t t = 0; t < T; ++t) {
        memcpy(z, z_in + t * V, (size_t)V * sizeof(double));
        row_transform(z, V, inv_tau, bf16);
        row_lse_logp(z, V, (int64_t)targets[t], &lse[t], &logp[t]);
        if (entropy) entropy[t] = row_entropy(z, V, lse[t]);
    }
    free(z);
}

/* The whole path with the contract options: logits, z' = z * inv_tau,
 * optionally rounded to bf16, then lse, logp and (if entropy is not NULL) the
 * entropy of softmax(z').  Returns 0 or -1. */
int oracle_selected_logp_ex(const uint16_t *hidden, int64_t ldh,
                            const uint16_t *weight, int64_t ldw,
                            const int32_t *targets, int64_t T, int64_t H,
                            int64_t V, double inv_tau, int bf16, double *logp,
                            double *lse, double *entropy, int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        if (!h || !z) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z);
                row_transform(z, V, inv_tau, bf16);
                row_lse_logp(z, V, (int64_t)targets[t], &lse[t], &logp[t]);
                if (entropy) entropy[t] = row_entropy(z, V, lse[t]);
            }
        }
        free(h);
        free(z);
    }
    return fail ? -1 : 0;
}

/* dz[t][v] of one row from its fp64 logits (already scaled by inv_tau). */
static void row_dz(const double *zs, int64_t V, int64_t y, double g, double inv_tau,
                   double *dz) {
    double lse, logp;
    row_lse_logp(zs, V, y, &lse, &logp);
    if (y < 0 || y >= V) {
        for (int64_t v = 0; v < V; ++v) dz[v] = 0.0;
        return;
    }
    for (int64_t v = 0; v < V; ++v) {
        const double p = exp(zs[v] - lse);
        dz[v] = g * inv_tau * ((v == y ? 1.0 : 0.0) - p);
    }
}

/* Gradient with respect to the logits, dz [T][V] (fp64).  Returns 0 or -1. */
int oracle_logp_grad_logits(const uint16_t *hidden, int64_t ldh,
                            const uint16_t *weight, int64_t ldw,
                            const int32_t *targets, const double *grad_logp,
                            int64_t T, int64_t H, int64_t V, double inv_tau,
                            double *dz, int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        if (!h || !z) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z);
                row_transform(z, V, inv_tau, 0);
                row_dz(z, V, (int64_t)targets[t], grad_logp[t], inv_tau, dz + t * V);
            }
        }
        free(h);
        free(z);
    }
    return fail ? -1 : 0;
}

/* grad_hidden [T][H] and / or grad_weight [V][H] (either may be NULL), fp64.
 * Each output element is one sum in increasing index order (v for
 * grad_hidden, t for grad_weight).  Returns 0 or -1. */
int oracle_selected_logp_backward(const uint16_t *hidden, int64_t ldh,
                                  const uint16_t *weight, int64_t ldw,
                                  const int32_t *targets, const double *grad_logp,
                                  int64_t T, int64_t H, int64_t V, double inv_tau,
                                  double *grad_hidden, double *grad_weight,
                                  int nthreads) {
    double *dz = (double *)malloc((size_t)(T * V > 0 ? T * V : 1) * sizeof(double));
    if (!dz) return -1;
    if (oracle_logp_grad_logits(hidden, ldh, weight, ldw, targets, grad_logp, T, H, V,
                                inv_tau, dz, nthreads)) {
        free(dz);
        return -1;
    }
    if (grad_hidden) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            double *out = grad_hidden + t * H;
            for (int64_t k = 0; k < H; ++k) out[k] = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                const double d = dz[t * V + v];
                const uint16_t *wv = weight + v * ldw;
                for (int64_t k = 0; k < H; ++k) out[k] = out[k] + d * bf16_to_f64(wv[k]);
            }
        }
    }
    if (grad_weight) {
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) {
            double *out = grad_weight + v * H;
            for (int64_t k = 0; k < H; ++k) out[k] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double d = dz[t * V + v];
                const uint16_t *ht = hidden + t * ldh;
                for (int64_t k = 0; k < H; ++k) out[k] = out[k] + d * bf16_to_f64(ht[k]);
            }
        }
    }
    free(dz);
    return 0;
}

/* bf16 value -> bit pattern (the value is a bf16 value or an infinity / NaN). */
static uint16_t f64_to_bf16_bits(double x) {
    const float f = (float)x;              /* exact: x is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(x)) u = 0x7FC00000u;
    return (uint16_t)(u >> 16);
}

/* RMSNorm of T rows of x (bf16 [T][ldx], first H columns) with weight gamma
 * (bf16 [H]): out bf16 bits [T][H]; xr (optional, fp64 [T][H]) receives the
 * unrounded x_k r.  Per row: ms = sum_k x_k^2 / H in fp64 (increasing k),
 * r = 1 / sqrt(ms + eps). */
void oracle_rmsnorm(const uint16_t *x, int64_t ldx, const uint16_t *gamma, double eps,
                    int64_t T, int64_t H, uint16_t *out, double *xr) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *row = x + t * ldx;
        double ss = 0.0;
        for (int64_t k = 0; k < H; ++k) {
            const double v = bf16_to_f64(row[k]);
            ss = ss + v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t k = 0; k < H; ++k) {
            const double a = bf16_to_f64(row[k]) * r;
            if (xr) xr[t * H + k] = a;
            const double n = round_bf16(to_f32(a));
            out[t * H + k] = f64_to_bf16_bits(round_bf16(n * bf16_to_f64(gamma[k])));
        }
    }
}

/* Top-k of one row of (transformed) logits by repeated selection of the
 * largest remaining entry under the order (value descending, id ascending).
 * Entries that are NaN are skipped; when fewer than k entries remain, the
 * tail gets id -1 and value -inf. */
static void row_topk(const double *z, int64_t V, int k, double lse, double *out_lp,
                     int32_t *out_id, unsigned char *taken) {
    memset(taken, 0, (size_t)V);
    for (int q = 0; q < k; ++q) {
        int64_t best = -1;
        for (int64_t v = 0; v < V; ++v) {
            if (taken[v] || isnan(z[v])) continue;
            if (best < 0 || z[v] > z[best]) best = v;
        }
        if (best < 0) {
            out_lp[q] = -INFINITY;
            out_id[q] = -1;
            continue;
        }
        taken[best] = 1;
        out_lp[q] = z[best] - lse;
        out_id[q] = (int32_t)best;
    }
}

/* Top-k log-probabilities [T][k] and token ids [T][k] with the contract
 * options (z' = z inv_tau, optionally rounded fp32 -> bf16).  Returns 0 or -1. */
int oracle_topk_logp(const uint16_t *hidden, int64_t ldh, const uint16_t *weight, int64_t ldw,
                     int64_t T, int64_t H, int64_t V, int k, double inv_tau, int bf16,
                     double *out_lp, int32_t *out_id, int nthreads) {
    int fail = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(H > 0 ? H : 1) * sizeof(double));
        double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        unsigned char *taken = (unsigned char *)malloc((size_t)(V > 0 ? V : 1));
        if (!h || !z || !taken) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                double lse, logp;
                hidden_row(hidden, ldh, t, H, h);
                row_logits(h, weight, ldw, H, V, z);
                row_transform(z, V, inv_tau, bf16);
                row_lse_logp(z, V, 0, &lse, &logp);
                row_topk(z, V, k, lse, out_lp + t * k, out_id + t * k, taken);
            }
        }
        free(h);
        free(z);
        free(taken);
    }
    return fail ? -1 : 0;
}

/* The same selection on logits given directly (fp64 [T][V]). */
void oracle_topk_from_logits(const double *z_in, int64_t T, int64_t V, int k, double inv_tau,
                             int bf16, double *out_lp, int32_t *out_id) {
    double *z = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    unsigned char *taken = (unsigned char *)malloc((size_t)(V > 0 ? V : 1));
    if (!z || !taken) {
        free(z);
        free(taken);
        return;
    }
    for (int64_t t = 0; t < T; ++t) {
        double lse, logp;
        memcpy(z, z_in + t * V, (size_t)V * sizeof(double));
        row_transform(z, V, inv_tau, bf16);
        row_lse_logp(z, V, 0, &lse, &logp);
        row_topk(z, V, k, lse, out_lp + t * k, out_id + t * k, taken);
    }
    free(z);
    free(taken);
}
