/*
 * oracle.h -- plain, slow, single-threaded CPU definition of the single-token
 * Llama-2 decode step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The GPU library shares no code,
 * header, table or constant with it.
 *
 * Precision: values are stored as fp32 exactly where the pages store a float
 * (x, xb, q, k, v, cache rows, attention output, hb, hb2, logits).  Every
 * reduction (dot products, sum of squares, softmax max/sum, the attention
 * weighted sum) and every transcendental is evaluated in double and rounded
 * once at the store.  Built with -DORACLE_PAGE_LITERAL the same code instead
 * uses the pages' own fp32 arithmetic (sequential float sums, expf, sqrtf,
 * the fp32 RoPE angle); the two builds must agree within tolerance.
 *
 * Layouts: matrices are row-major (out, in), element (i, j) at w[i*n + j]
 * ("run.c", function matmul).  The KV cache of one layer is (seq_len, kv_dim)
 * row-major, layers stacked: (n_layers, seq_len, kv_dim) ("run.c 逐行解讀",
 * §3 malloc_run_state).  The weight blob layout is the checkpoint order of the
 * "run.c" page (checkpoint_init_weights) with the grouped-query shapes and the
 * separate classifier of "run.c 逐行解讀" §2 (TransformerWeights), RoPE tables
 * dropped:
 *   E (V,dim) rms_att (L,dim) wq (L,dim,dim) wk (L,kv_dim,dim)
 *   wv (L,kv_dim,dim) wo (L,dim,dim) rms_ffn (L,dim) w1 (L,hidden,dim)
 *   w2 (L,dim,hidden) w3 (L,hidden,dim) rms_final (dim) [wcls (V,dim)]
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

typedef struct {
    int32_t dim, hidden_dim, n_layers, n_heads, n_kv_heads, vocab_size, seq_len;
} oracle_config;

typedef struct {
    double norm_eps;           /* 1e-5 */
    double rope_theta;         /* 10000 */
    int32_t shared_classifier; /* 1: classifier is the embedding table */
} oracle_options;

/* 1 for the page-literal fp32 build, 0 for the double-accumulation build. */
int oracle_page_literal(void);

/* Number of floats in the weight blob, or -1 for an invalid config. */
int64_t oracle_blob_floats(const oracle_config* c, const oracle_options* o);

/* out = g * (x / sqrt(mean(x^2) + eps)), n elements. out may alias x. */
void oracle_rmsnorm(float* out, const float* x, const float* g, int n, double eps);

/* out(d) = W(d, n) x(n). */
void oracle_matvec(float* out, const float* w, const float* x, int d, int n);

/* Rotate adjacent pairs (2j, 2j+1) of the first n_heads heads of v (head_size
 * each) by the angle pos * theta^(-2j/head_size).  In place. */
void oracle_rope(float* v, int n_heads, int head_size, int pos, double theta);

/* Key/value head that query head h reads: floor(h * n_kv_heads / n_heads). */
int oracle_kv_head(int h, int n_heads, int n_kv_heads);

/* Causal attention of one layer at position pos.  q: n_heads*head_size.
 * kc, vc: this layer's cache, rows 0..pos of kv_dim floats.  out: n_heads*head_size. */
void oracle_attention(float* out, const float* q, const float* kc, const float* vc, int n_heads,
                      int n_kv_heads, int head_size, int pos);

/* hb[i] = silu(h1[i]) * h3[i], silu(u) = u / (1 + e^-u).  hb may alias h1 or h3. */
void oracle_swiglu(float* hb, const float* h1, const float* h3, int n);

/* Lowest index holding the maximum of v[0..n). */
int oracle_argmax(const float* v, int n);

/* One decode step: writes cache row pos of every layer, returns logits (V).
 * Returns 0, or -1 when an argument is out of range. */
int oracle_forward(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                   float* vcache, int token, int pos, float* logits);

/* n greedy steps from (token, pos): tokens_out[i] = argmax of the logits at pos+i.
 * logits_out, if not NULL, receives n*V floats. */
int oracle_generate(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                    float* vcache, int token, int pos, int n, int32_t* tokens_out, float* logits_out);

/* Logits at position p recomputed from tokens[0..p] with no cache: every layer
 * over the whole prefix, causal mask of -inf above the diagonal. */
int oracle_bruteforce(const oracle_config* c, const oracle_options* o, const float* blob,
                      const int32_t* tokens, int p, float* logits);

#endif
