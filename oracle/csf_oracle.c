/*
 * csf_oracle.c -- plain, slow, obviously-correct CPU oracle for the contextual-sparsity FFN step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product (HIP) path never calls it, links it or
 * shares code with it.
 *
 * Conventions
 *   - Every sum is accumulated in double precision, in ascending index order.
 *   - Weights and activations arrive as raw bytes in one of three storage types
 *     (0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16) and are widened to double exactly.
 *   - Matrices are row-major and contiguous:  V[r][d], U[f][r], W1[f][d], Wup[f][d], W2T[f][d].
 *     W2T is the down projection stored neuron-major: row j holds the d output weights of neuron j.
 *   - Functions return 0 (or a count) on success and a negative number on bad arguments.
 *
 * Sources (the three web pages on contextual sparsity):
 *   [DV]  "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm"
 *         -- sections "The Prediction Problem", "The SiLU/GELU Challenge: TurboSparse",
 *            "Kernel-Level Implementation", "The Empirical Foundation".
 *   [CP]  "Contextual Sparsity and Activation Predictors"
 *         -- sections "The predictor and its budget", "Precision, recall, and which error hurts",
 *            "When it breaks".
 *   [AS]  "Activation sparsity" -- section "Implementation sketch".
 *
 * Where the pages leave a step open, the reading taken is stated at the function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_RELU = 0, ORC_REGLU = 1, ORC_SILU = 2, ORC_SWIGLU = 3 };

/* Threads for the loops over independent outputs (OpenMP; 1 = plain serial loops).  Every output
 * element is still one sum in ascending index order, formed by one thread, so the thread count
 * never changes a bit of any result: it only shares out whole rows (predictor, activations) and
 * whole column blocks (the FFN output). */
static int g_threads = 1;

int orc_set_threads(int n)
{
    if (n < 1)
        return -1;
    g_threads = n;
    return 0;
}

int orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------------------------------ */
/* Storage types, from their IEEE / bfloat16 definitions.                                      */
/* ------------------------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* zero or subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);     /* (1 + m/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* Round a double to the nearest value with `mbits` fraction bits, exponent bias `bias` and
 * `ebits` exponent bits, ties to even, and return the bit pattern.  Shared by the two 16-bit
 * formats below; it is the textbook definition of round-to-nearest-even. */
static uint16_t round_to_small_float(double v, int ebits, int mbits, int bias)
{
    uint16_t sign = (uint16_t)(signbit(v) ? 1u : 0u) << (ebits + mbits);
    int emax_field = (1 << ebits) - 1;
    if (isnan(v))
        return (uint16_t)(sign | (emax_field << mbits) | (1 << (mbits - 1)));
    double a = fabs(v);
    int emin = 1 - bias;                           /* exponent of the smallest normal */
    /* overflow threshold: halfway between the largest finite value and 2^(emax+1) */
    int emax = emax_field - 1 - bias;
    double big = ldexp(2.0 - ldexp(1.0, -(mbits + 1)), emax);
    if (a >= big)
        return (uint16_t)(sign | (emax_field << mbits));
    if (a < ldexp(1.0, emin)) {
        /* subnormal range: quantum 2^(emin - mbits) */
        double q = nearbyint(ldexp(a, mbits - emin));   /* default rounding mode: ties to even */
        return (uint16_t)(sign | (uint16_t)q);          /* q == 2^mbits lands on the smallest normal */
    }
    int ex;
    frexp(a, &ex);                                 /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;                                /* a in [2^E, 2^(E+1)) */
    double q = nearbyint(ldexp(a, mbits - E));     /* in [2^mbits, 2^(mbits+1)] */
    if (q == ldexp(1.0, mbits + 1)) {
        q = ldexp(1.0, mbits);
        E += 1;
    }
    int field = E + bias;
    if (field >= emax_field)
        return (uint16_t)(sign | (emax_field << mbits));
    return (uint16_t)(sign | (field << mbits) | ((uint16_t)q - (1 << mbits)));
}

uint16_t orc_f64_to_f16(double v) { return round_to_small_float(v, 5, 10, 15); }
uint16_t orc_f64_to_bf16(double v) { return round_to_small_float(v, 8, 7, 127); }

/* Element i of a buffer of storage type dt, widened exactly to double. */
static double wid(const void *base, size_t i, int dt)
{
    if (dt == ORC_F32)
        return (double)((const float *)base)[i];
    if (dt == ORC_F16)
        return orc_f16_to_f64(((const uint16_t *)base)[i]);
    return orc_bf16_to_f64(((const uint16_t *)base)[i]);
}

static int bad_dtype(int dt) { return dt != ORC_F32 && dt != ORC_F16 && dt != ORC_BF16; }

/* ------------------------------------------------------------------------------------------ */
/* O1/O2 -- the predictor.                                                                     */
/* [DV] "The Prediction Problem": a two-layer bias-free network per layer,                     */
/* scores = sigmoid(up(relu(down(x)))), down: d -> bottleneck r, up: r -> f.                   */
/* Reading: the hidden activation a is kept in full precision (no rounding to the weight       */
/* type); each score is the double-precision sigmoid rounded once to binary32.                  */
/* ------------------------------------------------------------------------------------------ */
int orc_predict(const void *x, int d, const void *V, int r, const void *U, int f, int dt,
                double *a_out /* [r] or NULL */, double *z_out /* [f] or NULL */,
                float *s_out /* [f] */)
{
    if (d <= 0 || r <= 0 || f <= 0 || bad_dtype(dt) || !x || !V || !U || !s_out)
        return -1;
    double *a = (double *)malloc(sizeof(double) * (size_t)r);
    if (!a)
        return -2;
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int i = 0; i < r; ++i) {                  /* a = relu(V x) */
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += wid(V, (size_t)i * d + c, dt) * wid(x, c, dt);
        a[i] = acc > 0.0 ? acc : 0.0;
        if (a_out)
            a_out[i] = a[i];
    }
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int j = 0; j < f; ++j) {                  /* z = U a ; s = sigmoid(z) */
        double acc = 0.0;
        for (int i = 0; i < r; ++i)
            acc += wid(U, (size_t)j * r + i, dt) * a[i];
        if (z_out)
            z_out[j] = acc;
        s_out[j] = (float)(1.0 / (1.0 + exp(-acc)));
    }
    free(a);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* O3 -- selection.                                                                            */
/* [DV] "The Prediction Problem": the k largest scores form the predicted active set.          */
/* Readings: scores are compared as binary32 values (so -0.0 ties +0.0); among equal scores    */
/* the lower neuron index ranks first; the set is returned in ascending index order.           */
/* ------------------------------------------------------------------------------------------ */
typedef struct { float s; int32_t j; } scored;

static int by_score_then_index(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

int orc_select_topk(const float *s, int f, int k, int32_t *idx_out /* [k] */)
{
    if (f < 0 || k < 0 || k > f || !s || (k > 0 && !idx_out))
        return -1;
    for (int j = 0; j < f; ++j)
        if (!isfinite(s[j]))
            return -3;                             /* finite scores only */
    scored *order = (scored *)malloc(sizeof(scored) * (size_t)(f > 0 ? f : 1));
    unsigned char *chosen = (unsigned char *)calloc((size_t)(f > 0 ? f : 1), 1);
    if (!order || !chosen) {
        free(order); free(chosen);
        return -2;
    }
    for (int j = 0; j < f; ++j) {
        order[j].s = s[j];
        order[j].j = j;
    }
    qsort(order, (size_t)f, sizeof(scored), by_score_then_index);
    for (int n = 0; n < k; ++n)
        chosen[order[n].j] = 1;
    int m = 0;
    for (int j = 0; j < f; ++j)
        if (chosen[j])
            idx_out[m++] = j;
    free(order);
    free(chosen);
    return m;
}

/* [AS] "Implementation sketch": active = scores >= threshold (inclusive), ascending order. */
int orc_select_threshold(const float *s, int f, float tau, int32_t *idx_out /* [f] */)
{
    if (f < 0 || !s || (f > 0 && !idx_out))
        return -1;
    int m = 0;
    for (int j = 0; j < f; ++j) {
        if (!isfinite(s[j]))
            return -3;
        if (s[j] >= tau)
            idx_out[m++] = j;
    }
    return m;
}

/* ------------------------------------------------------------------------------------------ */
/* O4/O5 -- the FFN over an active set.                                                        */
/* [DV] "The Prediction Problem" (sparse_mlp_forward): gather the active gate rows and the     */
/* matching down weights, compute only those.  [DV] "The SiLU/GELU Challenge": the ReLU-fied   */
/* gated form is down(relu(gate x) * (up x)).  [DV] "Kernel-Level Implementation": per-neuron  */
/* dot product, fp32-or-better accumulation, then max(acc, 0).                                 */
/* Readings: b1 is a per-neuron bias on the gate/up pre-activation (NULL = zero), no bias on   */
/* W_up or on the output; h and y stay in full precision; the down projection is neuron-major. */
/* SiLU forms ([DV] "The Prediction Problem": the sketch applies silu to the gathered gate      */
/* product; "The SiLU/GELU Challenge": the LLaMA-style block is down(silu(gate x) * (up x))):   */
/* silu(p) = p * sigmoid(p) = p / (1 + e^-p), never exactly zero, so a sparse step over a set   */
/* that drops neurons is an approximation of the dense layer, not a rearrangement of it.        */
/* ------------------------------------------------------------------------------------------ */

/* Gate pre-activation p_j = W1[j].x + b1_j and, for the gated form, u_j = Wup[j].x. */
static void neuron_preact(const void *x, int d, int dt, const void *W1, const float *b1,
                          const void *Wup, int act, int j, double *p, double *u)
{
    double acc = 0.0;
    for (int c = 0; c < d; ++c)
        acc += wid(W1, (size_t)j * d + c, dt) * wid(x, c, dt);
    if (b1)
        acc += (double)b1[j];
    *p = acc;
    *u = 1.0;
    if (act == ORC_REGLU || act == ORC_SWIGLU) {
        double au = 0.0;
        for (int c = 0; c < d; ++c)
            au += wid(Wup, (size_t)j * d + c, dt) * wid(x, c, dt);
        *u = au;
    }
}

static int gated_act(int act) { return act == ORC_REGLU || act == ORC_SWIGLU; }
static int bad_act(int act) { return act < ORC_RELU || act > ORC_SWIGLU; }

/* silu(p) = p / (1 + e^-p); for very negative p, e^-p overflows to +inf and the quotient is -0. */
double orc_silu(double p) { return p / (1.0 + exp(-p)); }

static double neuron_act(double p, double u, int act)
{
    double g = (act == ORC_SILU || act == ORC_SWIGLU) ? orc_silu(p) : (p > 0.0 ? p : 0.0);
    return gated_act(act) ? g * u : g;
}

/* y[c] = sum over list entries n (ascending) of h[n] W2T[rows[n]][c], each y[c] starting from 0
 * and adding the terms in list order; the columns go in blocks to the threads. */
enum { ORC_COL_BLOCK = 256 };

static void down_rows(const double *h, const int32_t *rows, int count, const void *W2T, int d,
                      int dt, double *y_out)
{
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int cb = 0; cb < d; cb += ORC_COL_BLOCK) {
        const int ce = cb + ORC_COL_BLOCK < d ? cb + ORC_COL_BLOCK : d;
        for (int c = cb; c < ce; ++c)
            y_out[c] = 0.0;
        for (int n = 0; n < count; ++n) {
            const size_t row = (size_t)(rows ? rows[n] : n) * d;
            for (int c = cb; c < ce; ++c)
                y_out[c] += h[n] * wid(W2T, row + c, dt);
        }
    }
}

int orc_sparse_ffn(const void *x, int d, int f, int act, int dt, const void *W1, const float *b1,
                   const void *Wup, const void *W2T, const int32_t *idx, int count,
                   double *h_out /* [count] or NULL */, double *y_out /* [d] */)
{
    if (d <= 0 || f < 0 || count < 0 || bad_dtype(dt) || bad_act(act))
        return -1;
    if (!x || !W1 || !W2T || !y_out || (count > 0 && !idx) || (gated_act(act) && !Wup))
        return -1;
    for (int n = 0; n < count; ++n)
        if (idx[n] < 0 || idx[n] >= f)
            return -4;
    double *h = (double *)malloc(sizeof(double) * (size_t)(count > 0 ? count : 1));
    if (!h)
        return -2;
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int n = 0; n < count; ++n) {           /* the active neurons' activations */
        double p, u;
        neuron_preact(x, d, dt, W1, b1, Wup, act, idx[n], &p, &u);
        h[n] = neuron_act(p, u, act);
    }
    if (h_out)
        for (int n = 0; n < count; ++n)
            h_out[n] = h[n];
    down_rows(h, idx, count, W2T, d, dt, y_out);   /* y = sum of h_n W2T[idx[n]] */
    free(h);
    return 0;
}

/* Dense reference: every neuron, in ascending order.  [CP] "The predictor and its budget"
 * names the dense layer as the thing the sparse step must beat. */
int orc_dense_ffn(const void *x, int d, int f, int act, int dt, const void *W1, const float *b1,
                  const void *Wup, const void *W2T, double *h_out /* [f] or NULL */,
                  double *y_out /* [d] */)
{
    if (d <= 0 || f < 0 || bad_dtype(dt) || bad_act(act))
        return -1;
    if (!x || !W1 || !W2T || !y_out || (gated_act(act) && !Wup))
        return -1;
    double *h = (double *)malloc(sizeof(double) * (size_t)(f > 0 ? f : 1));
    if (!h)
        return -2;
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int j = 0; j < f; ++j) {
        double p, u;
        neuron_preact(x, d, dt, W1, b1, Wup, act, j, &p, &u);
        h[j] = neuron_act(p, u, act);
    }
    if (h_out)
        for (int j = 0; j < f; ++j)
            h_out[j] = h[j];
    down_rows(h, NULL, f, W2T, d, dt, y_out);
    free(h);
    return 0;
}

/* O6 support: gate pre-activation of every neuron (p_j for ReLU, the gate g_j for the gated
 * form).  The true active set is {j : p_j > 0}: a ReLU output is exactly zero otherwise
 * ([DV] "The Empirical Foundation"). */
int orc_preact(const void *x, int d, int f, int dt, const void *W1, const float *b1,
               double *p_out /* [f] */)
{
    if (d <= 0 || f < 0 || bad_dtype(dt) || !x || !W1 || !p_out)
        return -1;
    for (int j = 0; j < f; ++j) {
        double p, u;
        neuron_preact(x, d, dt, W1, b1, NULL, ORC_RELU, j, &p, &u);
        p_out[j] = p;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* O8 support -- the normalised block input of a residual stack.                               */
/* [CP] "The predictor and its budget": x_{l+1} = x_l + f_l(x_l) with a block update that is  */
/* small against the stream.  Reading: f_l takes an RMS-normalised copy of the stream,         */
/* xhat = x / sqrt(mean(x^2) + eps) with no gain, rounded once to the weight storage type.     */
/* ------------------------------------------------------------------------------------------ */
int orc_rms_normalize(const float *x, int d, double eps, int dt, void *xhat_out /* [d] */)
{
    if (d <= 0 || bad_dtype(dt) || !x || !xhat_out || !(eps >= 0.0))
        return -1;
    double ss = 0.0;
    for (int c = 0; c < d; ++c)
        ss += (double)x[c] * (double)x[c];
    double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int c = 0; c < d; ++c) {
        double v = (double)x[c] * inv;
        if (dt == ORC_F32)
            ((float *)xhat_out)[c] = (float)v;
        else if (dt == ORC_F16)
            ((uint16_t *)xhat_out)[c] = orc_f64_to_f16(v);
        else
            ((uint16_t *)xhat_out)[c] = orc_f64_to_bf16(v);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* O9 -- attention-head sparsity: one decode step of multi-head attention over a set of heads. */
/* [DV] opening section: for a given input a small set of attention heads (with the MLP        */
/* neurons) approximates the dense layer; "The Empirical Foundation": only a fifth to a third  */
/* of the heads matter per token; "Implications for System Design": selecting heads per token  */
/* saves attention work and, above all, key/value cache traffic and memory.                    */
/* The page gives no formulas; the step is standard multi-head attention for one new token:    */
/*   q_h = Wq_h x + bq_h,  k_h = Wk_h x + bk_h,  v_h = Wv_h x + bv_h   (Wq_h: rows h*dh..+dh-1) */
/*   the new k_h, v_h are rounded to the cache's storage type and appended at position len_h;  */
/*   a_t = q_h . K_h[t] / sqrt(dh) for t = 0..len_h (the new token included), p = softmax(a),  */
/*   o_h = sum_t p_t V_h[t];  y = sum over the computed heads of WoT_h^T o_h.                  */
/* Readings: heads outside the set compute nothing for this token; with kv_all = 0 they also   */
/* store nothing (their cache does not grow: the saving in cache memory the page points to),   */
/* with kv_all = 1 every head appends its k, v (the cache stays complete, only q, the          */
/* attention and the output projection are sparse).  No output bias (it does not depend on the  */
/* selection).  Caches are [H][Tmax][dh] in the storage type, WoT [H*dh][d] (head-dimension   */
/* major, the analogue of the neuron-major down projection).                                   */
/* Returns 0, -1 for bad arguments, -4 for a head index outside [0, H), -5 for a full cache.   */
/* ------------------------------------------------------------------------------------------ */
static void store_elem(void *base, size_t i, int dt, double v)
{
    if (dt == ORC_F32)
        ((float *)base)[i] = (float)v;
    else if (dt == ORC_F16)
        ((uint16_t *)base)[i] = orc_f64_to_f16(v);
    else
        ((uint16_t *)base)[i] = orc_f64_to_bf16(v);
}

/* One row of a head-major projection: W[row] . x + b[row]. */
static double proj_row(const void *W, const float *b, const void *x, int d, int dt, size_t row)
{
    double acc = 0.0;
    for (int c = 0; c < d; ++c)
        acc += wid(W, row * (size_t)d + c, dt) * wid(x, c, dt);
    if (b)
        acc += (double)b[row];
    return acc;
}

int orc_attention_decode(const void *x, int d, int H, int dh, int dt, const void *Wq,
                         const void *Wk, const void *Wv, const float *bq, const float *bk,
                         const float *bv, const void *WoT, void *Kc, void *Vc, int Tmax,
                         int32_t *len, const int32_t *heads, int count, int kv_all,
                         double *o_out /* [count][dh] or NULL */, double *y_out /* [d] */)
{
    if (d <= 0 || H <= 0 || dh <= 0 || Tmax <= 0 || count < 0 || count > H || bad_dtype(dt))
        return -1;
    if (!x || !Wq || !Wk || !Wv || !WoT || !Kc || !Vc || !len || !y_out || (count > 0 && !heads))
        return -1;
    char *store = (char *)calloc((size_t)H, 1);
    double *q = (double *)malloc(sizeof(double) * (size_t)dh);
    double *o = (double *)malloc(sizeof(double) * (size_t)dh);
    double *a = (double *)malloc(sizeof(double) * (size_t)(Tmax > 0 ? Tmax : 1));
    int rc = 0;
    if (!store || !q || !o || !a) {
        rc = -1;
        goto done;
    }
    for (int n = 0; n < count; ++n) {
        if (heads[n] < 0 || heads[n] >= H) {
            rc = -4;
            goto done;
        }
        store[heads[n]] = 1;
    }
    for (int h = 0; h < H; ++h) {
        if (kv_all)
            store[h] = 1;
        if (store[h] && (len[h] < 0 || len[h] >= Tmax)) {
            rc = -5;
            goto done;
        }
    }
    /* append the new token's key and value to every storing head's cache */
    for (int h = 0; h < H; ++h) {
        if (!store[h])
            continue;
        size_t pos = ((size_t)h * Tmax + (size_t)len[h]) * dh;
        for (int i = 0; i < dh; ++i) {
            size_t row = (size_t)h * dh + i;
            store_elem(Kc, pos + i, dt, proj_row(Wk, bk, x, d, dt, row));
            store_elem(Vc, pos + i, dt, proj_row(Wv, bv, x, d, dt, row));
        }
        len[h] += 1;
    }
    for (int c = 0; c < d; ++c)
        y_out[c] = 0.0;
    const double scale = 1.0 / sqrt((double)dh);
    for (int n = 0; n < count; ++n) {
        const int h = heads[n];
        const int L = len[h];
        for (int i = 0; i < dh; ++i)
            q[i] = proj_row(Wq, bq, x, d, dt, (size_t)h * dh + i);
        double amax = -INFINITY;
        for (int t = 0; t < L; ++t) {
            double s = 0.0;
            for (int i = 0; i < dh; ++i)
                s += q[i] * wid(Kc, ((size_t)h * Tmax + t) * dh + i, dt);
            a[t] = s * scale;
            if (a[t] > amax)
                amax = a[t];
        }
        double z = 0.0;
        for (int t = 0; t < L; ++t) {
            a[t] = exp(a[t] - amax);
            z += a[t];
        }
        for (int i = 0; i < dh; ++i)
            o[i] = 0.0;
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < dh; ++i)
                o[i] += (a[t] / z) * wid(Vc, ((size_t)h * Tmax + t) * dh + i, dt);
        if (o_out)
            for (int i = 0; i < dh; ++i)
                o_out[(size_t)n * dh + i] = o[i];
        for (int i = 0; i < dh; ++i)
            for (int c = 0; c < d; ++c)
                y_out[c] += o[i] * wid(WoT, ((size_t)h * dh + i) * d + c, dt);
    }
done:
    free(store);
    free(q);
    free(o);
    free(a);
    return rc;
}
