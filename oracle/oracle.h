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

/* Threads over which matrix rows and attention heads are shared out (1 by
 * default, at most ORACLE_MAX_THREADS).  Every output is computed the same way
 * whatever the count, so results are bit-identical; only the wall time changes.
 * Process-wide; not to be changed while another thread is inside the oracle. */
#define ORACLE_MAX_THREADS 64
void oracle_set_threads(int t);

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

/* Next token from logits ("run.c 逐行解讀" §6, three modes): temperature 0 is the
 * argmax; otherwise logits are divided by the temperature and softmaxed, and
 * with 0 < topp < 1 the draw is restricted to the smallest set of most likely
 * tokens (descending probability, ties to the lower index) whose cumulative
 * probability reaches topp, else it is over all tokens.  The draw walks the
 * cumulative distribution ("run.c", sample): the first token whose cumulative
 * probability exceeds coin * (mass of the set); coin is in [0, 1). */
int oracle_sample(const float* logits, int n, double temperature, double topp, double coin);

/* One decode step: writes cache row pos of every layer, returns logits (V).
 * Returns 0, or -1 when an argument is out of range. */
int oracle_forward(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                   float* vcache, int token, int pos, float* logits);

/* n greedy steps from (token, pos): tokens_out[i] = argmax of the logits at pos+i.
 * logits_out, if not NULL, receives n*V floats. */
int oracle_generate(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                    float* vcache, int token, int pos, int n, int32_t* tokens_out, float* logits_out);

/* The generation loop of "run.c 逐行解讀" §7: step i runs at position pos+i on
 * token t_i (t_0 = prompt[0]); its next token is prompt[i+1] while the prompt
 * lasts, else oracle_sample(logits, temperature, topp, coins[i]).
 * tokens_out[i] = next token of step i; the loop ends after n_steps steps or
 * after the step whose next token equals stop_token (>= 0; included in the
 * output).  *n_out = steps run.  logits_out, if not NULL, gets n_steps*V floats. */
int oracle_generate_sampled(const oracle_config* c, const oracle_options* o, const float* blob, float* kcache,
                            float* vcache, const int32_t* prompt, int n_prompt, int pos, int n_steps,
                            double temperature, double topp, int stop_token, const float* coins,
                            int32_t* tokens_out, int* n_out, float* logits_out);

/* Logits at position p recomputed from tokens[0..p] with no cache: every layer
 * over the whole prefix, causal mask of -inf above the diagonal. */
int oracle_bruteforce(const oracle_config* c, const oracle_options* o, const float* blob,
                      const int32_t* tokens, int p, float* logits);

#endif
