/*
 * ffn_oracle.c -- plain, slow, single-threaded CPU oracle for the activation-sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The product path (the HIP library) never links, loads or calls it,
 * and the two share no source: no headers, no helpers, no constants.
 *
 * Everything is accumulated in double precision, in plain loop order, with no blocking, fusion
 * or reordering.  Inputs are read from the very same bytes the GPU path reads: fp32, fp16 (decoded
 * bit by bit, exactly) or int4 with fp16 group scales (s*q is exact in double).
 *
 * Sources (web pages on PowerInfer / PowerInfer-2; cited by title and section):
 *  [UA]  "PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU" (unite.ai, zh)
 *        sections "Adaptive sparse predictor" (自适应稀疏预测器), "Neuron placement and management"
 *        (神经元放置和管理), "Neuron-aware operator" (神经元感知运算符), "Online stage" (在线阶段).
 *  [NA]  "Can the 4090 replace the A100? ..." (nearauto.com, ja), section "PowerInfer architecture",
 *        Fig. 8 (GPU and CPU each compute only the activated neurons they hold; results merged).
 *  [CN]  "PowerInfer-2 ... 29x" (citnews.com.cn, zh), sections "Dynamic neuron cache" (inactive
 *        neurons do not change the output) and "Low-cost high-quality sparsification" (dReLU).
 *  [NB]  "PowerInfer-2: Fast LLM Inference on a Smartphone" (nubint.ai review), TurboSparse-Mixtral.
 *
 * Readings where the pages are silent (each one is listed in the design notes of the repo):
 *  - predictor = rank-r linear factorisation s = P2 (P1 x + c1) + c2, no hidden nonlinearity;
 *  - neuron i is active iff sigmoid(s_i) > tau, strictly;
 *  - ReLU h = max(u,0); ReGLU h = max(g,0)*u; dReLU h = max(g,0)*max(u,0);
 *  - down projection stored transposed: W_down_t[i][j] is the weight from neuron i to output j;
 *  - int4: signed two's-complement nibble, element 2k in the low nibble of byte k, one fp16 scale
 *    per 32 consecutive elements of a row, w = scale * q;
 *  - MoE router: logits l = R x, top-k with ties to the lower expert index, weights = softmax over
 *    the k selected logits;
 *  - attention block: the predicted unit is a head (W_q rows, scores, values, W_o columns); keys
 *    and values are computed for every head; scores scaled by 1/sqrt(head width), plain softmax,
 *    no positional rotation and no biases (the pages name none).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_I4G32 = 2 };
enum { OR_RELU = 0, OR_REGLU = 1, OR_DRELU = 2 };

/* IEEE-754 binary16 -> double, exactly (sign, 5-bit exponent, 10-bit fraction). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);                 /* zero or subnormal: fr * 2^-24 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);    /* (1 + fr/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

/* Element (row, j) of a row-major [rows][ncols] matrix stored in `dtype`.  For OR_I4G32 the
 * packed nibbles are `base` ([rows][ncols/2] bytes) and the fp16 scales are `scales`
 * ([rows][ncols/32]). */
double oracle_elem(int dtype, const void *base, const void *scales, long row, long j, long ncols)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[row * ncols + j];
    if (dtype == OR_F16)
        return oracle_half_to_double(((const uint16_t *)base)[row * ncols + j]);
    /* OR_I4G32 */
    {
        uint8_t byte = ((const uint8_t *)base)[row * (ncols / 2) + j / 2];
        int nib = (j & 1) ? (byte >> 4) : (byte & 0x0f);
        int q = nib >= 8 ? nib - 16 : nib;
        double s = oracle_half_to_double(((const uint16_t *)scales)[row * (ncols / 32) + j / 32]);
        return s * (double)q;
    }
}

static double vec_elem(int dtype, const void *x, long j)
{
    return oracle_elem(dtype, x, NULL, 0, j, 0);
}

/*
 * Activation predictor ([UA] "Adaptive sparse predictor": a small per-layer model that says
 * which neurons will fire for this input; [UA] "Online stage": neurons predicted inactive are
 * skipped).
 *   z_k = c1_k + sum_j P1[k][j] x_j                  (k < rank)
 *   s_i = c2_i + sum_k P2[i][k] z_k                  (i < ffn)
 *   p_i = 1 / (1 + exp(-s_i));  active_i = (p_i > tau)
 * c1, c2 may be NULL (= 0).  Outputs: z[rank], s[ffn], p[ffn], active[ffn] (0/1).
 * Returns the number of active neurons.
 */
long oracle_predictor(long d, long ffn, long rank, int p_dtype, const void *p1, const void *p2,
                      const float *c1, const float *c2, int x_dtype, const void *x, double tau,
                      double *z, double *s, double *p, uint8_t *active)
{
    long k, i, j, count = 0;
    for (k = 0; k < rank; ++k) {
        double acc = c1 ? (double)c1[k] : 0.0;
        for (j = 0; j < d; ++j)
            acc += oracle_elem(p_dtype, p1, NULL, k, j, d) * vec_elem(x_dtype, x, j);
        z[k] = acc;
    }
    for (i = 0; i < ffn; ++i) {
        double acc = c2 ? (double)c2[i] : 0.0;
        for (k = 0; k < rank; ++k)
            acc += oracle_elem(p_dtype, p2, NULL, i, k, rank) * z[k];
        s[i] = acc;
        p[i] = 1.0 / (1.0 + exp(-acc));
        active[i] = p[i] > tau ? 1 : 0;
        count += active[i];
    }
    return count;
}

/* Ascending list of active neuron indices ([UA] "Neuron placement and management": each
 * computed neuron keeps its original position in the matrix).  Returns the count. */
long oracle_active_list(long ffn, const uint8_t *active, int32_t *idx)
{
    long i, n = 0;
    for (i = 0; i < ffn; ++i)
        if (active[i])
            idx[n++] = (int32_t)i;
    return n;
}

static double act_fn(int act, double u, double g)
{
    double gr = g > 0.0 ? g : 0.0;
    double ur = u > 0.0 ? u : 0.0;
    if (act == OR_RELU)
        return ur;
    if (act == OR_REGLU)
        return gr * u;
    return gr * ur; /* OR_DRELU */
}

/*
 * Neuron-aware FFN on one token ([UA] "Neuron-aware operator": only the row / column vectors of
 * the active neurons are used, never a densified matrix; [CN] "Dynamic neuron cache": neurons
 * that are not activated leave the output unchanged; [NA] Fig. 8).
 *   for i with mask_i = 1:  u_i = b_up_i + W_up[i] . x ;  g_i = b_gate_i + W_gate[i] . x
 *                           h_i = act(u_i, g_i)
 *   for i with mask_i = 0:  h_i = 0
 *   y_j = b_down_j + sum_{i: mask_i = 1} h_i * W_down_t[i][j]
 * mask == NULL means every neuron (the dense FFN).  W_gate / b_gate are read only for ReGLU and
 * dReLU.  Any bias pointer may be NULL (= 0).  Outputs h[ffn] and y[d] in double.
 */
void oracle_ffn(long d, long ffn, int act, int w_dtype,
                const void *w_up, const void *w_gate, const void *w_down_t,
                const void *s_up, const void *s_gate, const void *s_down_t,
                const float *b_up, const float *b_gate, const float *b_down,
                int x_dtype, const void *x, const uint8_t *mask, double *h, double *y)
{
    long i, j;
    for (i = 0; i < ffn; ++i) {
        double u = 0.0, g = 0.0;
        h[i] = 0.0;
        if (mask && !mask[i])
            continue;
        u = b_up ? (double)b_up[i] : 0.0;
        for (j = 0; j < d; ++j)
            u += oracle_elem(w_dtype, w_up, s_up, i, j, d) * vec_elem(x_dtype, x, j);
        if (act != OR_RELU) {
            g = b_gate ? (double)b_gate[i] : 0.0;
            for (j = 0; j < d; ++j)
                g += oracle_elem(w_dtype, w_gate, s_gate, i, j, d) * vec_elem(x_dtype, x, j);
        }
        h[i] = act_fn(act, u, g);
    }
    for (j = 0; j < d; ++j)
        y[j] = b_down ? (double)b_down[j] : 0.0;
    for (i = 0; i < ffn; ++i) {
        if (mask && !mask[i])
            continue;
        for (j = 0; j < d; ++j)
            y[j] += h[i] * oracle_elem(w_dtype, w_down_t, s_down_t, i, j, d);
    }
}

/*
 * Top-k router of a sparse mixture of experts ([NB] / [CN]: TurboSparse-Mixtral activates a
 * subset of experts per token).  logits_e = sum_j R[e][j] x_j; the k largest logits are chosen,
 * ties to the lower expert index; weights = softmax over the chosen logits.
 * Outputs logits[n_exp], ids[k] (in selection order: largest first), w[k].
 */
void oracle_router(long d, long n_exp, long k, int r_dtype, const void *R, int x_dtype,
                   const void *x, double *logits, int32_t *ids, double *w)
{
    long e, j, t;
    double mx, den;
    for (e = 0; e < n_exp; ++e) {
        double acc = 0.0;
        for (j = 0; j < d; ++j)
            acc += oracle_elem(r_dtype, R, NULL, e, j, d) * vec_elem(x_dtype, x, j);
        logits[e] = acc;
    }
    for (t = 0; t < k; ++t) {
        long best = -1;
        for (e = 0; e < n_exp; ++e) {
            long u, taken = 0;
            for (u = 0; u < t; ++u)
                if (ids[u] == e)
                    taken = 1;
            if (taken)
                continue;
            if (best < 0 || logits[e] > logits[best])
                best = e;
        }
        ids[t] = (int32_t)best;
    }
    mx = logits[ids[0]];
    den = 0.0;
    for (t = 0; t < k; ++t)
        den += exp(logits[ids[t]] - mx);
    for (t = 0; t < k; ++t)
        w[t] = exp(logits[ids[t]] - mx) / den;
}

/*
 * Self-attention block of one token with a head-level active set.  [UA] "Adaptive sparse
 * predictor" gives every transformer layer a second predictor, for its self-attention block,
 * and [UA] "Online stage" restricts computation to what is predicted active.  The pages do not
 * say what the attention block's unit is; the reading here is one head: its W_q rows, its share
 * of the scores and values, and its W_o columns (the only unit whose contribution enters the
 * block's output as one additive term, as a neuron's row does in the FFN).
 *
 * Shapes: H query heads and G key/value heads of width e (H a multiple of G; query head h reads
 * key/value head h / (H / G)).  W_q and W_o_t are [H*e][d], W_k and W_v [G*e][d], row-major in
 * w_dtype; row h*e + c of W_q is channel c of head h, and row h*e + c of W_o_t holds the weights
 * from channel c of head h to the d outputs (the output projection stored transposed, so that a
 * head contributes whole rows).
 *
 * oracle_attn_kv: key and value of the token for every key/value head, active or not: a head
 * predicted inactive now may be active for a later token, whose scores then need this token's
 * key and value, so the cache stays exactly that of the dense model.
 *   k[g*e + c] = W_k[g*e + c] . x ;   v[g*e + c] = W_v[g*e + c] . x
 */
void oracle_attn_kv(long d, long G, long e, int w_dtype, const void *w_k, const void *w_v,
                    int x_dtype, const void *x, double *k, double *v)
{
    long r, j;
    for (r = 0; r < G * e; ++r) {
        double ak = 0.0, av = 0.0;
        for (j = 0; j < d; ++j) {
            ak += oracle_elem(w_dtype, w_k, NULL, r, j, d) * vec_elem(x_dtype, x, j);
            av += oracle_elem(w_dtype, w_v, NULL, r, j, d) * vec_elem(x_dtype, x, j);
        }
        k[r] = ak;
        v[r] = av;
    }
}

/*
 * oracle_attn: the block's output for the token at position t, over a cache Kc, Vc
 * ([G][S][e] in kv_dtype, S >= t + 1) whose positions 0..t hold the keys and values of the
 * token's context and of the token itself (position t); positions past t are never read.
 *   for h with mask_h = 1 (mask == NULL: every head), g = h / (H / G):
 *     q_h = W_q[h] x                                   (e values)
 *     a_j = (q_h . Kc[g][j]) / sqrt(e),   j = 0..t
 *     p_j = exp(a_j - max a) / sum_i exp(a_i - max a)
 *     o_h = sum_j p_j Vc[g][j]
 *   for h with mask_h = 0: o_h = 0
 *   y = sum_{h: mask_h = 1} sum_c o_h[c] W_o_t[h*e + c]
 * Outputs o[H*e] and y[d] in double.
 */
void oracle_attn(long d, long H, long G, long e, long S, long t, int w_dtype, const void *w_q,
                 const void *w_o_t, int kv_dtype, const void *Kc, const void *Vc, int x_dtype,
                 const void *x, const uint8_t *mask, double *o, double *y)
{
    long h, c, j;
    double scale = 1.0 / sqrt((double)e);
    for (j = 0; j < d; ++j)
        y[j] = 0.0;
    for (h = 0; h < H; ++h) {
        long g = h / (H / G);
        double mx = -INFINITY, den = 0.0;
        double q[512];                      /* e <= 512 */
        for (c = 0; c < e; ++c)
            o[h * e + c] = 0.0;
        if (mask && !mask[h])
            continue;
        for (c = 0; c < e; ++c) {
            double acc = 0.0;
            for (j = 0; j < d; ++j)
                acc += oracle_elem(w_dtype, w_q, NULL, h * e + c, j, d) * vec_elem(x_dtype, x, j);
            q[c] = acc;
        }
        /* scores, their maximum, and the softmax denominator */
        for (j = 0; j <= t; ++j) {
            double a = 0.0;
            for (c = 0; c < e; ++c)
                a += q[c] * oracle_elem(kv_dtype, Kc, NULL, g * S + j, c, e);
            a *= scale;
            if (a > mx)
                mx = a;
        }
        for (j = 0; j <= t; ++j) {
            double a = 0.0;
            for (c = 0; c < e; ++c)
                a += q[c] * oracle_elem(kv_dtype, Kc, NULL, g * S + j, c, e);
            den += exp(a * scale - mx);
        }
        for (j = 0; j <= t; ++j) {
            double a = 0.0, p;
            for (c = 0; c < e; ++c)
                a += q[c] * oracle_elem(kv_dtype, Kc, NULL, g * S + j, c, e);
            p = exp(a * scale - mx) / den;
            for (c = 0; c < e; ++c)
                o[h * e + c] += p * oracle_elem(kv_dtype, Vc, NULL, g * S + j, c, e);
        }
        for (c = 0; c < e; ++c)
            for (j = 0; j < d; ++j)
                y[j] += o[h * e + c] * oracle_elem(w_dtype, w_o_t, NULL, h * e + c, j, d);
    }
}
