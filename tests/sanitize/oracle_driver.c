/* Runs every oracle entry point on small shapes with heap buffers of exactly
 * the sizes the entry points document, so that a build with
 * -fsanitize=address,undefined reports any access outside them or any
 * undefined behaviour.  Also checks a few properties of the results (logp <= 0,
 * the naive and the blocked logits agree bit for bit, log-softmax sums to one,
 * top-1 equals the row maximum).  Exit status 0 when everything holds.
 * Test infrastructure: it links the oracle, nothing of the HIP library. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_logits(const uint16_t *, int64_t, const uint16_t *, int64_t, int64_t, int64_t,
                  int64_t, double *, int);
int oracle_logits_naive(const uint16_t *, int64_t, const uint16_t *, int64_t, int64_t, int64_t,
                        int64_t, double *);
void oracle_lse_from_logits(const double *, const int32_t *, int64_t, int64_t, double *,
                            double *);
int oracle_selected_logp(const uint16_t *, int64_t, const uint16_t *, int64_t, const int32_t *,
                         int64_t, int64_t, int64_t, double *, double *, int);
int oracle_log_softmax(const uint16_t *, int64_t, const uint16_t *, int64_t, int64_t, int64_t,
                       int64_t, double *, int);
void oracle_round_bf16(const float *, int64_t, double *);
void oracle_ex_from_logits(const double *, const int32_t *, int64_t, int64_t, double, int,
                           double *, double *, double *);
int oracle_selected_logp_ex(const uint16_t *, int64_t, const uint16_t *, int64_t,
                            const int32_t *, int64_t, int64_t, int64_t, double, int, double *,
                            double *, double *, int);
int oracle_logp_grad_logits(const uint16_t *, int64_t, const uint16_t *, int64_t,
                            const int32_t *, const double *, int64_t, int64_t, int64_t, double,
                            double *, int);
int oracle_selected_logp_backward(const uint16_t *, int64_t, const uint16_t *, int64_t,
                                  const int32_t *, const double *, int64_t, int64_t, int64_t,
                                  double, double *, double *, int);
void oracle_rmsnorm(const uint16_t *, int64_t, const uint16_t *, double, int64_t, int64_t,
                    uint16_t *, double *);
int oracle_topk_logp(const uint16_t *, int64_t, const uint16_t *, int64_t, int64_t, int64_t,
                     int64_t, int, double, int, double *, int32_t *, int);
void oracle_topk_from_logits(const double *, int64_t, int64_t, int, double, int, double *,
                             int32_t *);

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32(void) {  /* xorshift64 */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 32);
}
/* a bf16 value in about [-1, 1) (bit pattern), never NaN or Inf */
static uint16_t rand_bf16(void) {
    float f = ((float)(next_u32() >> 8) / 16777216.0f) * 2.0f - 1.0f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);      \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static void run_shape(int64_t T, int64_t H, int64_t V, int k) {
    const int64_t ldh = H + 8, ldw = H + 16;   /* strides wider than H */
    uint16_t *h = xmalloc(sizeof(uint16_t) * T * ldh);
    uint16_t *w = xmalloc(sizeof(uint16_t) * V * ldw);
    uint16_t *g = xmalloc(sizeof(uint16_t) * H);
    int32_t *y = xmalloc(sizeof(int32_t) * T);
    for (int64_t i = 0; i < T * ldh; ++i) h[i] = rand_bf16();
    for (int64_t i = 0; i < V * ldw; ++i) w[i] = rand_bf16();
    for (int64_t i = 0; i < H; ++i) g[i] = rand_bf16();
    for (int64_t t = 0; t < T; ++t) y[t] = (int32_t)(next_u32() % (uint32_t)V);
    if (T > 1) y[T - 1] = (int32_t)V;   /* one out-of-range target: NaN logp */
    double *z = xmalloc(sizeof(double) * T * V), *z2 = xmalloc(sizeof(double) * T * V);
    double *lp = xmalloc(sizeof(double) * T), *lse = xmalloc(sizeof(double) * T);
    double *lp2 = xmalloc(sizeof(double) * T), *lse2 = xmalloc(sizeof(double) * T);
    double *ent = xmalloc(sizeof(double) * T), *gl = xmalloc(sizeof(double) * T);
    for (int64_t t = 0; t < T; ++t) gl[t] = (double)(int)(next_u32() % 7) - 3.0;

    CHECK(oracle_logits(h, ldh, w, ldw, T, H, V, z, 2) == 0);
    CHECK(oracle_logits_naive(h, ldh, w, ldw, T, H, V, z2) == 0);
    CHECK(memcmp(z, z2, sizeof(double) * T * V) == 0);
    oracle_lse_from_logits(z, y, T, V, lp, lse);
    CHECK(oracle_selected_logp(h, ldh, w, ldw, y, T, H, V, lp2, lse2, 3) == 0);
    for (int64_t t = 0; t < T; ++t) {
        CHECK(lse[t] == lse2[t]);
        if (y[t] < V) CHECK(lp2[t] <= 0.0 && lp[t] == lp2[t]);
        else CHECK(isnan(lp2[t]));
    }
    CHECK(oracle_log_softmax(h, ldh, w, ldw, T, H, V, z2, 1) == 0);
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v) s += exp(z2[t * V + v]);
        CHECK(fabs(s - 1.0) < 1e-12);
    }
    oracle_ex_from_logits(z, y, T, V, 0.7, 1, lp, lse, ent);
    CHECK(oracle_selected_logp_ex(h, ldh, w, ldw, y, T, H, V, 0.7, 1, lp2, lse2, ent, 2) == 0);
    for (int64_t t = 0; t < T; ++t) CHECK(lse[t] == lse2[t] && ent[t] >= 0.0);
    CHECK(oracle_logp_grad_logits(h, ldh, w, ldw, y, gl, T, H, V, 1.3, z2, 2) == 0);
    double *gh = xmalloc(sizeof(double) * T * H), *gw = xmalloc(sizeof(double) * V * H);
    CHECK(oracle_selected_logp_backward(h, ldh, w, ldw, y, gl, T, H, V, 1.3, gh, gw, 2) == 0);
    CHECK(oracle_selected_logp_backward(h, ldh, w, ldw, y, gl, T, H, V, 1.0, NULL, gw, 1) == 0);
    CHECK(oracle_selected_logp_backward(h, ldh, w, ldw, y, gl, T, H, V, 1.0, gh, NULL, 1) == 0);
    uint16_t *out = xmalloc(sizeof(uint16_t) * T * H);
    double *xr = xmalloc(sizeof(double) * T * H);
    oracle_rmsnorm(h, ldh, g, 1e-6, T, H, out, xr);
    oracle_rmsnorm(h, ldh, g, 0.0, T, H, out, NULL);
    double *tl = xmalloc(sizeof(double) * T * k);
    int32_t *ti = xmalloc(sizeof(int32_t) * T * k);
    CHECK(oracle_topk_logp(h, ldh, w, ldw, T, H, V, k, 1.0, 0, tl, ti, 2) == 0);
    oracle_topk_from_logits(z, T, V, k, 0.5, 1, tl, ti);
    oracle_topk_from_logits(z, T, V, k, 1.0, 0, tl, ti);
    for (int64_t t = 0; t < T; ++t) {
        double m = z[t * V];
        for (int64_t v = 1; v < V; ++v) m = z[t * V + v] > m ? z[t * V + v] : m;
        CHECK(z[t * V + ti[t * k]] == m);
    }
    float fx[5] = {1.0f, -2.5f, 3.0e38f, 1e-40f, 0.0f};
    double fr[5];
    oracle_round_bf16(fx, 5, fr);
    CHECK(fr[0] == 1.0 && fr[1] == -2.5);
    free(h); free(w); free(g); free(y); free(z); free(z2); free(lp); free(lse); free(lp2);
    free(lse2); free(ent); free(gl); free(gh); free(gw); free(out); free(xr); free(tl); free(ti);
}

int main(void) {
    /* ragged shapes, V = 1, k = V, a single row, H not a multiple of 64 */
    run_shape(1, 64, 1, 1);
    run_shape(3, 8, 5, 5);
    run_shape(7, 24, 37, 4);
    run_shape(16, 64, 129, 20);
    run_shape(5, 136, 300, 64);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
