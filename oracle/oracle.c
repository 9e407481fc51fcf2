/*
 * oracle.c -- the decode step written out as its plain definition.
 *
 * TEST INFRASTRUCTURE (see oracle.h): used by the test suite, the smoke check
 * and the benchmark's CPU baseline only.
 *
 * The step follows the forward() walkthrough of the "run.c 逐行解讀" page
 * (§4, steps 1, 2a-2h and 3), cross-checked against the transformer() function
 * of the "run.c" page and the Attention / TransformerBlock / FeedForward layers
 * of the "LLaMA implemented in R Tensorflow and Keras" page.  Readings where the
 * pages leave a point open:
 *   - RMSNorm eps is added to mean(x^2) inside the square root.
 *   - RoPE rotates adjacent pairs (2j, 2j+1) of each head by pos*theta^(-2j/hs);
 *     q is rotated in every head, k in its n_kv_heads heads.
 *   - query head h reads key/value head floor(h*n_kv/n_heads), i.e. the page's
 *     h / kv_mul with kv_mul = n_heads/n_kv_heads taken as a real ratio.
 *   - argmax returns the lowest index among equal maxima.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_PAGE_LITERAL
typedef float acc_t;
#define ACC_SQRT sqrtf
#define ACC_EXP expf
#else
typedef double acc_t;
#define ACC_SQRT sqrt
#define ACC_EXP exp
#endif

int oracle_page_literal(void) {
#ifdef ORACLE_PAGE_LITERAL
    return 1;
#else
    return 0;
#endif
}

static int config_ok(const oracle_config* c) {
    if (!c) return 0;
    if (c->dim <= 0 || c->hidden_dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
        c->vocab_size <= 0 || c->seq_len <= 0)
        return 0;
    if (c->dim % c->n_heads) return 0;
    if ((c->dim / c->n_heads) % 2) return 0;
    if (c->n_kv_heads > c->n_heads) return 0;
    if (((int64_t)c->dim * c->n_kv_heads) % c->n_heads) return 0;
    return 1;
}

static int64_t kv_dim_of(const oracle_config* c) { return (int64_t)c->dim * c->n_kv_heads / c->n_heads; }

/* Per-tensor pointers into the blob ("run.c 逐行解讀" §3, memory_map_weights:
 * the tensors follow one another, offsets kept in 64 bits). */
typedef struct {
    const float *emb, *rms_att, *wq, *wk, *wv, *wo, *rms_ffn, *w1, *w2, *w3, *rms_final, *wcls;
} weights_t;

static int64_t map_weights(const oracle_config* c, const oracle_options* o, const float* blob, weights_t* w) {
    const int64_t d = c->dim, h = c->hidden_dim, L = c->n_layers, V = c->vocab_size, kv = kv_dim_of(c);
    int64_t off = 0;
    weights_t t;
#define TAKE(field, count) t.field = blob ? blob + off : NULL; off += (count);
    TAKE(emb, V * d);
    TAKE(rms_att, L * d);
    TAKE(wq, L * d * d);
    TAKE(wk, L * kv * d);
    TAKE(wv, L * kv * d);
    TAKE(wo, L * d * d);
    TAKE(rms_ffn, L * d);
    TAKE(w1, L * h * d);
    TAKE(w2, L * d * h);
    TAKE(w3, L * h * d);
    TAKE(rms_final, d);
    if (o->shared_classifier) {
        t.wcls = t.emb;
    } else {
        TAKE(wcls, V * d);
    }
#undef TAKE
    if (w) *w = t;
    return off;
}

int64_t oracle_blob_floats(const oracle_config* c, const oracle_options* o) {
    if (!config_ok(c) || !o) return -1;
    return map_weights(c, o, NULL, NULL);
}

/* RMSNorm ("run.c 逐行解讀" §4 RMSNorm; rmsnorm() of the "run.c" page): the
 * root mean square of x, with eps added to the mean square under the root,
 * divides every element, and the gain then scales it element-wise. */
void oracle_rmsnorm(float* out, const float* x, const float* g, int n, double eps) {
    acc_t sum_sq = 0;
    for (int j = 0; j < n; ++j) sum_sq += (acc_t)x[j] * (acc_t)x[j];
    const acc_t rms = ACC_SQRT(sum_sq / (acc_t)n + (acc_t)eps);
    for (int j = 0; j < n; ++j) {
        const acc_t unit = (acc_t)x[j] / rms;
        out[j] = (float)((acc_t)g[j] * unit);
    }
}

/* Matrix-vector product: "run.c 逐行解讀" §4 Matmul, W(d,n) @ x(n) -> out(d),
 * element (i, j) of W at w[i*n + j].  Output i is the dot product of row i
 * with x, summed in index order.
 *
 * The rows are independent, so oracle_set_threads(t) lets t threads share
 * them out in contiguous ranges.  Each output is still the same sequential
 * sum, so the result is bit-identical for every thread count (default 1). */
static int g_threads = 1;

void oracle_set_threads(int t) { g_threads = t < 1 ? 1 : (t > ORACLE_MAX_THREADS ? ORACLE_MAX_THREADS : t); }

/* rows i0..i1-1 of out(d) = W(d, n) x(n) */
static void matvec_rows(float* out, const float* w, const float* x, int d, int n, int i0, int i1) {
    (void)d;
    for (int i = i0; i < i1; ++i) {
        const float* row = w + (int64_t)i * n;
        acc_t s = 0;
        for (int j = 0; j < n; ++j) s += (acc_t)row[j] * (acc_t)x[j];
        out[i] = (float)s;
    }
}

typedef struct {
    float* out;
    const float* w;
    const float* x;
    int d, n, i0, i1;
} rows_job;

static void* rows_thread(void* p) {
    const rows_job* j = (const rows_job*)p;
    matvec_rows(j->out, j->w, j->x, j->d, j->n, j->i0, j->i1);
    return NULL;
}

void oracle_matvec(float* out, const float* w, const float* x, int d, int n) {
    int t = g_threads;
    if ((int64_t)d * n < ((int64_t)1 << 20) || d < 2 * t) t = 1;
    if (t == 1) {
        matvec_rows(out, w, x, d, n, 0, d);
        return;
    }
    rows_job jobs[ORACLE_MAX_THREADS];
    pthread_t tid[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    for (int k = 0; k < t; ++k) {
        jobs[k] = (rows_job){out, w, x, d, n, (int)((int64_t)d * k / t), (int)((int64_t)d * (k + 1) / t)};
        started[k] = k > 0 && pthread_create(&tid[k], NULL, rows_thread, &jobs[k]) == 0;
        if (k > 0 && !started[k]) rows_thread(&jobs[k]);
    }
    rows_thread(&jobs[0]);
    for (int k = 1; k < t; ++k)
        if (started[k]) pthread_join(tid[k], NULL);
}

/* RoPE ("run.c 逐行解讀" §4 step 2d; the rotary embedding of the R/Keras
 * page): in every head, pair j = (v[2j], v[2j+1]) is multiplied by the 2x2
 * rotation matrix of the angle a_j = pos * theta^(-2j / head_size),
 *     [ cos a_j   -sin a_j ]
 *     [ sin a_j    cos a_j ].
 * The double build takes the angle, cos and sin in double; the page-literal
 * build takes them in fp32 (powf, cosf, sinf), as the pages do. */
void oracle_rope(float* v, int n_heads, int head_size, int pos, double theta) {
    for (int j = 0; 2 * j < head_size; ++j) {
#ifdef ORACLE_PAGE_LITERAL
        const float a = (float)pos * (1.0f / powf((float)theta, (float)(2 * j) / (float)head_size));
        const acc_t R[2][2] = {{cosf(a), -sinf(a)}, {sinf(a), cosf(a)}};
#else
        const double a = (double)pos * pow(theta, -(double)(2 * j) / (double)head_size);
        const acc_t R[2][2] = {{cos(a), -sin(a)}, {sin(a), cos(a)}};
#endif
        for (int h = 0; h < n_heads; ++h) {
            float* pair = v + (int64_t)h * head_size + 2 * j;
            const acc_t in[2] = {pair[0], pair[1]};
            for (int r = 0; r < 2; ++r) pair[r] = (float)(R[r][0] * in[0] + R[r][1] * in[1]);
        }
    }
}

int oracle_kv_head(int h, int n_heads, int n_kv_heads) { return (int)(((int64_t)h * n_kv_heads) / n_heads); }

/* Causal multi-head attention with grouped KV heads: "run.c 逐行解讀" §4
 * step 2e.  For every query head: scores q.k_t / sqrt(head_size) for t = 0..pos,
 * softmax with the maximum subtracted (§4 Softmax), then the weighted sum of
 * the value rows.  Heads are independent; like the matrix rows above they may
 * be shared out among the oracle_set_threads() threads, with results that do
 * not depend on the thread count. */
typedef struct {
    float* out;
    const float *q, *kc, *vc;
    int n_heads, n_kv_heads, head_size, pos, h0, h1;
} heads_job;

static void* attend_heads(void* p) {
    const heads_job* J = (const heads_job*)p;
    const int head_size = J->head_size, pos = J->pos;
    const int64_t kv_dim = (int64_t)head_size * J->n_kv_heads;
    acc_t* att = (acc_t*)malloc(sizeof(acc_t) * (size_t)(pos + 1));
    for (int h = J->h0; h < J->h1; ++h) {
        const int g = oracle_kv_head(h, J->n_heads, J->n_kv_heads);
        const float* qh = J->q + (int64_t)h * head_size;
        for (int t = 0; t <= pos; ++t) {
            const float* k = J->kc + (int64_t)t * kv_dim + (int64_t)g * head_size;
            acc_t s = 0;
            for (int i = 0; i < head_size; ++i) s += (acc_t)qh[i] * (acc_t)k[i];
            att[t] = s / ACC_SQRT((acc_t)head_size);
        }
        acc_t m = att[0];
        for (int t = 1; t <= pos; ++t)
            if (att[t] > m) m = att[t];
        acc_t sum = 0;
        for (int t = 0; t <= pos; ++t) {
            att[t] = ACC_EXP(att[t] - m);
            sum += att[t];
        }
        for (int t = 0; t <= pos; ++t) att[t] /= sum;
        for (int i = 0; i < head_size; ++i) {
            acc_t acc = 0;
            for (int t = 0; t <= pos; ++t)
                acc += att[t] * (acc_t)J->vc[(int64_t)t * kv_dim + (int64_t)g * head_size + i];
            J->out[(int64_t)h * head_size + i] = (float)acc;
        }
    }
    free(att);
    return NULL;
}

void oracle_attention(float* out, const float* q, const float* kc, const float* vc, int n_heads,
                      int n_kv_heads, int head_size, int pos) {
    int t = g_threads;
    if ((int64_t)n_heads * head_size * (pos + 1) < ((int64_t)1 << 18) || n_heads < 2 * t) t = 1;
    heads_job jobs[ORACLE_MAX_THREADS];
    pthread_t tid[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    for (int k = 0; k < t; ++k) {
        jobs[k] = (heads_job){out, q, kc, vc, n_heads, n_kv_heads, head_size, pos, n_heads * k / t,
                              n_heads * (k + 1) / t};
        started[k] = k > 0 && pthread_create(&tid[k], NULL, attend_heads, &jobs[k]) == 0;
        if (k > 0 && !started[k]) attend_heads(&jobs[k]);
    }
    attend_heads(&jobs[0]);
    for (int k = 1; k < t; ++k)
        if (started[k]) pthread_join(tid[k], NULL);
}

/* The logistic function sigma(u) = 1 / (1 + e^-u).  For u far below zero
 * e^-u overflows to infinity and sigma(u) is 0, never NaN. */
static acc_t logistic(acc_t u) { return (acc_t)1 / ((acc_t)1 + ACC_EXP(-u)); }

/* SwiGLU ("run.c 逐行解讀" §4 step 2h; the FeedForward layer of the R/Keras
 * page): the SiLU of the w1 branch, silu(u) = u * sigma(u), times the w3
 * branch, element by element. */
void oracle_swiglu(float* hb, const float* h1, const float* h3, int n) {
    for (int i = 0; i < n; ++i) {
        const acc_t gate = (acc_t)h1[i] * logistic((acc_t)h1[i]);
        hb[i] = (float)(gate * (acc_t)h3[i]);
    }
}

/* Greedy choice (argmax() of the "run.c" page): the largest logit, and of the
 * indices holding it the lowest one. */
int oracle_argmax(const float* v, int n) {
    float top = v[0];
    for (int i = 1; i < n; ++i)
        if (v[i] > top) top = v[i];
    for (int i = 0; i < n; ++i)
        if (v[i] == top) return i;
    return 0;
}

typedef struct {
    acc_t p;
    int i;
} prob_index;

/* descending probability, ties to the lower index */
static int by_prob_desc(const void* a, const void* b) {
    const prob_index* x = (const prob_index*)a;
    const prob_index* y = (const prob_index*)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return x->i - y->i;
}

/* Sampling: "run.c 逐行解讀" §6 (temperature 0 -> argmax; otherwise divide by the
 * temperature, softmax, then top-p or plain multinomial), with the
 * cumulative-distribution walk of sample() on the "run.c" page. */
int oracle_sample(const float* logits, int n, double temperature, double topp, double coin) {
    if (!(temperature > 0)) return oracle_argmax(logits, n);
    prob_index* pi = (prob_index*)malloc(sizeof(prob_index) * (size_t)n);
    acc_t m = (acc_t)logits[0] / (acc_t)temperature;
    for (int i = 0; i < n; ++i) {
        pi[i].p = (acc_t)logits[i] / (acc_t)temperature;
        pi[i].i = i;
        if (pi[i].p > m) m = pi[i].p;
    }
    acc_t sum = 0;
    for (int i = 0; i < n; ++i) {
        pi[i].p = ACC_EXP(pi[i].p - m);
        sum += pi[i].p;
    }
    for (int i = 0; i < n; ++i) pi[i].p /= sum;
    int chosen = n - 1;
    if (topp <= 0 || topp >= 1) {
        acc_t cdf = 0;
        for (int i = 0; i < n; ++i) {
            cdf += pi[i].p;
            if ((acc_t)coin < cdf) {
                chosen = i;
                break;
            }
        }
    } else {
        qsort(pi, (size_t)n, sizeof(prob_index), by_prob_desc);
        acc_t mass = 0;
        int k = 0;
        while (k < n && mass < (acc_t)topp) mass += pi[k++].p;
        const acc_t r = (acc_t)coin * mass;
        acc_t cdf = 0;
        chosen = pi[k - 1].i;
        for (int j = 0; j < k; ++j) {
            cdf += pi[j].p;
            if (r < cdf) {
                chosen = pi[j].i;
                break;
            }
        }
    }
    free(pi);
    return chosen;
}

static void add_into(float* x, const float* y, int n) {
    for (int i = 0; i < n; ++i) x[i] = (float)((acc_t)x[i] + (acc_t)y[i]);
}

/* One decode step: "run.c 逐行解讀" §4 forward(), steps 1 to 3. */
int oracle_forward(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                   float* vcache, int token, int pos, float* logits) {
    if (!config_ok(c) || !o || !blob || !kcache || !vcache || !logits) return -1;
    if (token < 0 || token >= c->vocab_size || pos < 0 || pos >= c->seq_len) return -1;
    weights_t w;
    map_weights(c, o, blob, &w);
    const int dim = c->dim, hidden = c->hidden_dim, H = c->n_heads, KV = c->n_kv_heads;
    const int hs = dim / H, kv_dim = (int)kv_dim_of(c), S = c->seq_len;
    float* x = (float*)malloc(sizeof(float) * (size_t)dim);
    float* xb = (float*)malloc(sizeof(float) * (size_t)dim);
    float* xb2 = (float*)malloc(sizeof(float) * (size_t)dim);
    float* q = (float*)malloc(sizeof(float) * (size_t)dim);
    float* hb = (float*)malloc(sizeof(float) * (size_t)hidden);
    float* hb2 = (float*)malloc(sizeof(float) * (size_t)hidden);

    /* step 1: embedding row of the token */
    memcpy(x, w.emb + (int64_t)token * dim, sizeof(float) * (size_t)dim);

    for (int l = 0; l < c->n_layers; ++l) {
        const int64_t lw = (int64_t)l;
        /* 2a: attention RMSNorm */
        oracle_rmsnorm(xb, x, w.rms_att + lw * dim, dim, o->norm_eps);
        /* 2b: k and v of this position live in cache row pos */
        float* kc = kcache + lw * S * kv_dim;
        float* vc = vcache + lw * S * kv_dim;
        float* krow = kc + (int64_t)pos * kv_dim;
        float* vrow = vc + (int64_t)pos * kv_dim;
        /* 2c: projections */
        oracle_matvec(q, w.wq + lw * dim * dim, xb, dim, dim);
        oracle_matvec(krow, w.wk + lw * kv_dim * dim, xb, kv_dim, dim);
        oracle_matvec(vrow, w.wv + lw * kv_dim * dim, xb, kv_dim, dim);
        /* 2d: RoPE on all query heads and on the key heads */
        oracle_rope(q, H, hs, pos, o->rope_theta);
        oracle_rope(krow, KV, hs, pos, o->rope_theta);
        /* 2e: attention over rows 0..pos */
        oracle_attention(xb, q, kc, vc, H, KV, hs, pos);
        /* 2f: output projection and residual */
        oracle_matvec(xb2, w.wo + lw * dim * dim, xb, dim, dim);
        add_into(x, xb2, dim);
        /* 2g: FFN RMSNorm */
        oracle_rmsnorm(xb, x, w.rms_ffn + lw * dim, dim, o->norm_eps);
        /* 2h: SwiGLU FFN and residual */
        oracle_matvec(hb, w.w1 + lw * hidden * dim, xb, hidden, dim);
        oracle_matvec(hb2, w.w3 + lw * hidden * dim, xb, hidden, dim);
        oracle_swiglu(hb, hb, hb2, hidden);
        oracle_matvec(xb, w.w2 + lw * dim * hidden, hb, dim, hidden);
        add_into(x, xb, dim);
    }
    /* step 3: final RMSNorm and classifier */
    oracle_rmsnorm(x, x, w.rms_final, dim, o->norm_eps);
    oracle_matvec(logits, w.wcls, x, c->vocab_size, dim);

    free(x);
    free(xb);
    free(xb2);
    free(q);
    free(hb);
    free(hb2);
    return 0;
}

/* Greedy generation: the decode loop of the "run.c" page at temperature 0
 * (the argmax of each step's logits is the next input token). */
int oracle_generate(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                    float* vcache, int token, int pos, int n, int32_t* tokens_out, float* logits_out) {
    if (!config_ok(c) || n < 0 || pos < 0 || (int64_t)pos + n > c->seq_len || !tokens_out) return -1;
    float* logits = (float*)malloc(sizeof(float) * (size_t)c->vocab_size);
    int rc = 0;
    for (int i = 0; i < n && rc == 0; ++i) {
        rc = oracle_forward(c, o, blob, kcache, vcache, token, pos + i, logits);
        if (rc) break;
        token = oracle_argmax(logits, c->vocab_size);
        tokens_out[i] = token;
        if (logits_out) memcpy(logits_out + (int64_t)i * c->vocab_size, logits, sizeof(float) * (size_t)c->vocab_size);
    }
    free(logits);
    return rc;
}

/* The generation loop of "run.c 逐行解讀" §7: prompt tokens are forced while the
 * prompt lasts, then tokens are sampled; the loop ends at the stop token. */
int oracle_generate_sampled(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                            float* vcache, const int32_t* prompt, int n_prompt, int pos, int n_steps,
                            double temperature, double topp, int stop_token, const float* coins,
                            int32_t* tokens_out, int* n_out, float* logits_out) {
    if (!config_ok(c) || !prompt || n_prompt < 1 || n_steps < 0 || pos < 0 || (int64_t)pos + n_steps > c->seq_len ||
        !tokens_out || !n_out || !coins)
        return -1;
    float* logits = (float*)malloc(sizeof(float) * (size_t)c->vocab_size);
    int rc = 0, token = prompt[0];
    *n_out = 0;
    for (int i = 0; i < n_steps; ++i) {
        rc = oracle_forward(c, o, blob, kcache, vcache, token, pos + i, logits);
        if (rc) break;
        if (logits_out) memcpy(logits_out + (int64_t)i * c->vocab_size, logits, sizeof(float) * (size_t)c->vocab_size);
        const int next = i + 1 < n_prompt ? prompt[i + 1]
                                          : oracle_sample(logits, c->vocab_size, temperature, topp, (double)coins[i]);
        tokens_out[i] = next;
        *n_out = i + 1;
        if (stop_token >= 0 && next == stop_token) break;
        token = next;
    }
    free(logits);
    return rc;
}

/* Full-prefix recompute with no cache, in the style of TransformerDecoder$call
 * of the R/Keras page: every layer runs over all T = p+1 positions at once and
 * the scores get the additive causal mask of make_mask (-inf where the key
 * index exceeds the query index) before the softmax. */
int oracle_bruteforce(const oracle_config* c, const oracle_options* o, const float* blob,
                      const int32_t* tokens, int p, float* logits) {
    if (!config_ok(c) || !o || !blob || !tokens || !logits || p < 0 || p >= c->seq_len) return -1;
    for (int t = 0; t <= p; ++t)
        if (tokens[t] < 0 || tokens[t] >= c->vocab_size) return -1;
    weights_t w;
    map_weights(c, o, blob, &w);
    const int dim = c->dim, hidden = c->hidden_dim, H = c->n_heads, KV = c->n_kv_heads;
    const int hs = dim / H, kv_dim = (int)kv_dim_of(c), T = p + 1;
    float* X = (float*)malloc(sizeof(float) * (size_t)T * dim);
    float* XB = (float*)malloc(sizeof(float) * (size_t)T * dim);
    float* Q = (float*)malloc(sizeof(float) * (size_t)T * dim);
    float* K = (float*)malloc(sizeof(float) * (size_t)T * kv_dim);
    float* Vv = (float*)malloc(sizeof(float) * (size_t)T * kv_dim);
    float* A = (float*)malloc(sizeof(float) * (size_t)T * dim);
    float* tmp = (float*)malloc(sizeof(float) * (size_t)dim);
    float* h1 = (float*)malloc(sizeof(float) * (size_t)hidden);
    float* h3 = (float*)malloc(sizeof(float) * (size_t)hidden);
    acc_t* sc = (acc_t*)malloc(sizeof(acc_t) * (size_t)T);

    for (int t = 0; t < T; ++t) memcpy(X + (int64_t)t * dim, w.emb + (int64_t)tokens[t] * dim, sizeof(float) * (size_t)dim);

    for (int l = 0; l < c->n_layers; ++l) {
        const int64_t lw = l;
        for (int t = 0; t < T; ++t) {
            float* xb = XB + (int64_t)t * dim;
            oracle_rmsnorm(xb, X + (int64_t)t * dim, w.rms_att + lw * dim, dim, o->norm_eps);
            oracle_matvec(Q + (int64_t)t * dim, w.wq + lw * dim * dim, xb, dim, dim);
            oracle_matvec(K + (int64_t)t * kv_dim, w.wk + lw * kv_dim * dim, xb, kv_dim, dim);
            oracle_matvec(Vv + (int64_t)t * kv_dim, w.wv + lw * kv_dim * dim, xb, kv_dim, dim);
            oracle_rope(Q + (int64_t)t * dim, H, hs, t, o->rope_theta);
            oracle_rope(K + (int64_t)t * kv_dim, KV, hs, t, o->rope_theta);
        }
        /* scores (query i, key j) over the whole T x T square, plus the mask */
        for (int h = 0; h < H; ++h) {
            const int g = oracle_kv_head(h, H, KV);
            for (int i = 0; i < T; ++i) {
                const float* qi = Q + (int64_t)i * dim + (int64_t)h * hs;
                for (int j = 0; j < T; ++j) {
                    const float* kj = K + (int64_t)j * kv_dim + (int64_t)g * hs;
                    acc_t s = 0;
                    for (int e = 0; e < hs; ++e) s += (acc_t)qi[e] * (acc_t)kj[e];
                    s /= ACC_SQRT((acc_t)hs);
                    sc[j] = s + (i < j ? (acc_t)-INFINITY : (acc_t)0);
                }
                acc_t m = sc[0];
                for (int j = 1; j < T; ++j)
                    if (sc[j] > m) m = sc[j];
                acc_t sum = 0;
                for (int j = 0; j < T; ++j) {
                    sc[j] = ACC_EXP(sc[j] - m);
                    sum += sc[j];
                }
                for (int e = 0; e < hs; ++e) {
                    acc_t acc = 0;
                    for (int j = 0; j < T; ++j) acc += (sc[j] / sum) * (acc_t)Vv[(int64_t)j * kv_dim + (int64_t)g * hs + e];
                    A[(int64_t)i * dim + (int64_t)h * hs + e] = (float)acc;
                }
            }
        }
        for (int t = 0; t < T; ++t) {
            float* x = X + (int64_t)t * dim;
            oracle_matvec(tmp, w.wo + lw * dim * dim, A + (int64_t)t * dim, dim, dim);
            add_into(x, tmp, dim);
            oracle_rmsnorm(tmp, x, w.rms_ffn + lw * dim, dim, o->norm_eps);
            oracle_matvec(h1, w.w1 + lw * hidden * dim, tmp, hidden, dim);
            oracle_matvec(h3, w.w3 + lw * hidden * dim, tmp, hidden, dim);
            oracle_swiglu(h1, h1, h3, hidden);
            oracle_matvec(tmp, w.w2 + lw * dim * hidden, h1, dim, hidden);
            add_into(x, tmp, dim);
        }
    }
    float* xl = X + (int64_t)p * dim;
    oracle_rmsnorm(xl, xl, w.rms_final, dim, o->norm_eps);
    oracle_matvec(logits, w.wcls, xl, c->vocab_size, dim);

    free(X);
    free(XB);
    free(Q);
    free(K);
    free(Vv);
    free(A);
    free(tmp);
    free(h1);
    free(h3);
    free(sc);
    return 0;
}
