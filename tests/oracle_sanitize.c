/*
 * Driver for the oracle under AddressSanitizer / UndefinedBehaviorSanitizer (CPU only).
 *
 * Every input and output lives in its own heap block of exactly the size the oracle's contract
 * gives it, so a read or write one element past any array is reported.  The driver runs every
 * oracle entry point on tiny layers of all three weight encodings and checks a few identities
 * that hold whatever the values (mask of all ones == no mask; the output is additive over a split
 * of the active set; router weights sum to one), returning non-zero on any mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_half_to_double(uint16_t h);
long oracle_predictor(long d, long ffn, long rank, int p_dtype, const void *p1, const void *p2,
                      const float *c1, const float *c2, int x_dtype, const void *x, double tau,
                      double *z, double *s, double *p, uint8_t *active);
long oracle_active_list(long ffn, const uint8_t *active, int32_t *idx);
void oracle_ffn(long d, long ffn, int act, int w_dtype,
                const void *w_up, const void *w_gate, const void *w_down_t,
                const void *s_up, const void *s_gate, const void *s_down_t,
                const float *b_up, const float *b_gate, const float *b_down,
                int x_dtype, const void *x, const uint8_t *mask, double *h, double *y);
void oracle_router(long d, long n_exp, long k, int r_dtype, const void *R, int x_dtype,
                   const void *x, double *logits, int32_t *ids, double *w);
void oracle_attn_kv(long d, long G, long e, int w_dtype, const void *w_k, const void *w_v,
                    int x_dtype, const void *x, double *k, double *v);
void oracle_attn(long d, long H, long G, long e, long S, long t, int w_dtype, const void *w_q,
                 const void *w_o_t, int kv_dtype, const void *Kc, const void *Vc, int x_dtype,
                 const void *x, const uint8_t *mask, double *o, double *y);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 32);
}
static float uniform(void) { return (float)(next_u32() >> 8) / 16777216.0f - 0.5f; }

/* a small finite fp16 value: exponent 10..17 (magnitudes 2^-5 .. 2^2), random sign and mantissa */
static uint16_t rand_half(void)
{
    uint32_t r = next_u32();
    return (uint16_t)(((r & 1u) << 15) | ((10u + (r >> 1) % 8u) << 10) | ((r >> 4) & 0x3ffu));
}

static void *block(size_t n, int fill_kind)
{
    void *p = malloc(n);
    size_t i;
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    if (fill_kind == 0) {                       /* fp32 */
        for (i = 0; i < n / 4; ++i) ((float *)p)[i] = uniform();
    } else if (fill_kind == 1) {                /* fp16 */
        for (i = 0; i < n / 2; ++i) ((uint16_t *)p)[i] = rand_half();
    } else {                                    /* raw bytes (int4 nibbles) */
        for (i = 0; i < n; ++i) ((uint8_t *)p)[i] = (uint8_t)next_u32();
    }
    return p;
}

static int close_rel(const double *a, const double *b, long n)
{
    double mx = 0.0, err = 0.0;
    long i;
    for (i = 0; i < n; ++i) {
        if (fabs(b[i]) > mx) mx = fabs(b[i]);
        if (fabs(a[i] - b[i]) > err) err = fabs(a[i] - b[i]);
    }
    return err <= 1e-12 * (mx > 1.0 ? mx : 1.0);
}

/* one layer of shape d x ffn in w_dtype (0 f32, 1 f16, 2 int4 g32) with activation act */
static int run_layer(long d, long ffn, long rank, int w_dtype, int act)
{
    const int xd = w_dtype == 0 ? 0 : 1;
    const size_t xb = (size_t)d * (xd == 0 ? 4 : 2);
    const size_t wb = w_dtype == 0 ? (size_t)ffn * d * 4 : w_dtype == 1 ? (size_t)ffn * d * 2
                                                                          : (size_t)ffn * d / 2;
    const size_t sb = w_dtype == 2 ? (size_t)ffn * (d / 32) * 2 : 0;
    const int wk = w_dtype == 2 ? 2 : w_dtype;  /* fill kind */
    void *x = block(xb, xd);
    void *w_up = block(wb, wk), *w_gate = block(wb, wk), *w_dn = block(wb, wk);
    void *s_up = sb ? block(sb, 1) : NULL, *s_gate = sb ? block(sb, 1) : NULL;
    void *s_dn = sb ? block(sb, 1) : NULL;
    float *b_up = block((size_t)ffn * 4, 0), *b_gate = block((size_t)ffn * 4, 0);
    float *b_down = block((size_t)d * 4, 0);
    const int pd = w_dtype == 0 ? 0 : 1;
    void *p1 = block((size_t)rank * d * (pd ? 2 : 4), pd);
    void *p2 = block((size_t)ffn * rank * (pd ? 2 : 4), pd);
    float *c1 = block((size_t)rank * 4, 0), *c2 = block((size_t)ffn * 4, 0);
    double *z = malloc((size_t)rank * 8), *s = malloc((size_t)ffn * 8), *p = malloc((size_t)ffn * 8);
    uint8_t *active = malloc((size_t)ffn), *ones = malloc((size_t)ffn), *m1 = malloc((size_t)ffn);
    uint8_t *m2 = malloc((size_t)ffn);
    int32_t *idx = malloc((size_t)ffn * 4);
    double *h = malloc((size_t)ffn * 8), *y = malloc((size_t)d * 8), *y1 = malloc((size_t)d * 8);
    double *y2 = malloc((size_t)d * 8), *ya = malloc((size_t)d * 8);
    long i, n, n2;
    int ok = 1;

    n = oracle_predictor(d, ffn, rank, pd, p1, p2, c1, c2, xd, x, 0.5, z, s, p, active);
    n2 = oracle_active_list(ffn, active, idx);
    ok &= n == n2;
    for (i = 1; i < n2; ++i) ok &= idx[i] > idx[i - 1];

    /* no mask == mask of all ones */
    memset(ones, 1, (size_t)ffn);
    oracle_ffn(d, ffn, act, w_dtype, w_up, w_gate, w_dn, s_up, s_gate, s_dn, b_up, b_gate, b_down,
               xd, x, NULL, h, y);
    oracle_ffn(d, ffn, act, w_dtype, w_up, w_gate, w_dn, s_up, s_gate, s_dn, b_up, b_gate, b_down,
               xd, x, ones, h, ya);
    ok &= memcmp(y, ya, (size_t)d * 8) == 0;

    /* additive over a split of the predicted set (no down bias): y(A) = y(A1) + y(A2) */
    for (i = 0; i < ffn; ++i) {
        m1[i] = active[i] && (i % 3 == 0);
        m2[i] = active[i] && (i % 3 != 0);
    }
    oracle_ffn(d, ffn, act, w_dtype, w_up, w_gate, w_dn, s_up, s_gate, s_dn, b_up, b_gate, NULL,
               xd, x, active, h, y);
    oracle_ffn(d, ffn, act, w_dtype, w_up, w_gate, w_dn, s_up, s_gate, s_dn, b_up, b_gate, NULL,
               xd, x, m1, h, y1);
    oracle_ffn(d, ffn, act, w_dtype, w_up, w_gate, w_dn, s_up, s_gate, s_dn, b_up, b_gate, NULL,
               xd, x, m2, h, y2);
    for (i = 0; i < d; ++i) ya[i] = y1[i] + y2[i];
    ok &= close_rel(y, ya, d);

    free(x); free(w_up); free(w_gate); free(w_dn); free(s_up); free(s_gate); free(s_dn);
    free(b_up); free(b_gate); free(b_down); free(p1); free(p2); free(c1); free(c2);
    free(z); free(s); free(p); free(active); free(ones); free(m1); free(m2); free(idx);
    free(h); free(y); free(y1); free(y2); free(ya);
    if (!ok) fprintf(stderr, "layer d=%ld ffn=%ld w_dtype=%d act=%d: identity failed\n", d, ffn,
                     w_dtype, act);
    return ok;
}

static int run_router(long d, long n_exp, long k)
{
    uint16_t *R = block((size_t)n_exp * d * 2, 1), *x = block((size_t)d * 2, 1);
    double *logits = malloc((size_t)n_exp * 8), *w = malloc((size_t)k * 8), sum = 0.0;
    int32_t *ids = malloc((size_t)k * 4);
    long t;
    int ok = 1;
    oracle_router(d, n_exp, k, 1, R, 1, x, logits, ids, w);
    for (t = 0; t < k; ++t) {
        ok &= ids[t] >= 0 && ids[t] < n_exp;
        sum += w[t];
        if (t) ok &= logits[ids[t]] <= logits[ids[t - 1]];
    }
    ok &= fabs(sum - 1.0) < 1e-12;
    free(R); free(x); free(logits); free(w); free(ids);
    if (!ok) fprintf(stderr, "router d=%ld E=%ld k=%ld: identity failed\n", d, n_exp, k);
    return ok;
}

/* Attention block: caches sized for exactly t + 1 positions (so a read past t is reported), the
 * output additive over a split of the heads, and every-head == no mask. */
static int run_attn(long d, long H, long G, long e, long t)
{
    long i, S = t + 1;
    uint16_t *wq = malloc(sizeof(uint16_t) * H * e * d), *wo = malloc(sizeof(uint16_t) * H * e * d);
    uint16_t *wk = malloc(sizeof(uint16_t) * G * e * d), *wv = malloc(sizeof(uint16_t) * G * e * d);
    uint16_t *K = malloc(sizeof(uint16_t) * G * S * e), *V = malloc(sizeof(uint16_t) * G * S * e);
    uint16_t *x = malloc(sizeof(uint16_t) * d);
    uint8_t *m1 = malloc(H), *m2 = malloc(H), *all = malloc(H);
    double *k = malloc(sizeof(double) * G * e), *v = malloc(sizeof(double) * G * e);
    double *o = malloc(sizeof(double) * H * e);
    double *y = malloc(sizeof(double) * d), *y1 = malloc(sizeof(double) * d);
    double *y2 = malloc(sizeof(double) * d), *ya = malloc(sizeof(double) * d);
    int ok = 1;
    for (i = 0; i < H * e * d; ++i) { wq[i] = rand_half(); wo[i] = rand_half(); }
    for (i = 0; i < G * e * d; ++i) { wk[i] = rand_half(); wv[i] = rand_half(); }
    for (i = 0; i < G * S * e; ++i) { K[i] = rand_half(); V[i] = rand_half(); }
    for (i = 0; i < d; ++i) x[i] = rand_half();
    for (i = 0; i < H; ++i) { m1[i] = (uint8_t)(next_u32() & 1); m2[i] = (uint8_t)!m1[i]; all[i] = 1; }
    oracle_attn_kv(d, G, e, 1, wk, wv, 1, x, k, v);
    oracle_attn(d, H, G, e, S, t, 1, wq, wo, 1, K, V, 1, x, NULL, o, y);
    oracle_attn(d, H, G, e, S, t, 1, wq, wo, 1, K, V, 1, x, all, o, ya);
    oracle_attn(d, H, G, e, S, t, 1, wq, wo, 1, K, V, 1, x, m1, o, y1);
    oracle_attn(d, H, G, e, S, t, 1, wq, wo, 1, K, V, 1, x, m2, o, y2);
    for (i = 0; i < d; ++i) {
        ok &= y[i] == ya[i];
        ok &= fabs(y1[i] + y2[i] - y[i]) <= 1e-9 * (1.0 + fabs(y[i]));
    }
    for (i = 0; i < G * e; ++i) ok &= isfinite(k[i]) && isfinite(v[i]);
    free(wq); free(wo); free(wk); free(wv); free(K); free(V); free(x); free(m1); free(m2);
    free(all); free(k); free(v); free(o); free(y); free(y1); free(y2); free(ya);
    if (!ok) fprintf(stderr, "attn d=%ld H=%ld G=%ld e=%ld t=%ld: identity failed\n", d, H, G, e, t);
    return ok;
}

int main(void)
{
    int ok = 1, act, wd;
    /* every fp16 bit pattern decodes (subnormals, infinities, NaNs included) */
    unsigned v;
    for (v = 0; v < 65536u; ++v) (void)oracle_half_to_double((uint16_t)v);
    for (wd = 0; wd < 3; ++wd)
        for (act = 0; act < 3; ++act) {
            ok &= run_layer(32, 8, 4, wd, act);
            ok &= run_layer(64, 96, 8, wd, act);
        }
    ok &= run_router(64, 8, 2);
    ok &= run_router(32, 4, 4);
    ok &= run_attn(32, 4, 2, 8, 0);
    ok &= run_attn(48, 6, 3, 16, 9);
    printf(ok ? "oracle sanitizer run: OK\n" : "oracle sanitizer run: FAILED\n");
    return ok ? 0 : 1;
}
