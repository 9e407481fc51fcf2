/*
 * ld.h -- C ABI of the MI355X (gfx950) single-token Llama-2 decode library.
 *
 * The library runs one decode step of a Llama-2 decoder at batch 1 in fp32:
 * embedding lookup, per layer RMSNorm, q/k/v projections, RoPE, KV-cache
 * append, causal grouped-query attention, output projection + residual,
 * RMSNorm, SwiGLU FFN + residual; then the final RMSNorm, classifier logits
 * and the greedy argmax.  The step is the forward() walkthrough of the
 * "run.c 逐行解讀" page (§4, steps 1, 2a-2h, 3) and transformer() of the
 * "run.c" page; the interface follows those pages: Config is the create
 * argument, the Transformer aggregate becomes an opaque handle, forward(token,
 * pos) returns logits, and the greedy loop is the generate loop of "run.c"
 * at temperature 0.
 *
 * Around that step: the generation loop with temperature / top-p sampling,
 * prompt forcing and a stop token ("run.c 逐行解讀" §6-§7, ld_generate), a
 * prompt prefilled in one pass (ld_prefill), and several sequences decoded
 * per step, each on its own KV cache (ld_forward_batch,
 * ld_generate_greedy_batch).
 *
 * Conventions for every call:
 *   - Every call returns an int status: LD_OK (0) or a negative LD_E_* code.
 *     No call aborts the process or lets a C++ exception escape.
 *   - Pointers named d_* are device pointers (HIP device memory, e.g. the
 *     storage of a torch CUDA tensor); h_* are host pointers.
 *   - A model may be used by one host thread at a time.
 *   - Matrices are fp32, row-major (out, in): element (i, j) at w[i*in + j]
 *     ("run.c", matmul).
 */
#ifndef LD_H
#define LD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model shape: the Config struct of the "run.c" page (seven int32 fields in
 * this order).  kv_dim = dim * n_kv_heads / n_heads ("run.c 逐行解讀", §3).
 * Validity (else LD_E_CONFIG): every field > 0; dim % n_heads == 0; head_size
 * = dim / n_heads even; n_kv_heads <= n_heads; dim * n_kv_heads % n_heads == 0;
 * dim, hidden_dim and kv_dim multiples of 4.  Supported by the kernels (else
 * LD_E_UNSUPPORTED): head_size in {16, 32, 48, 64, 80, 96, 128, 256}; at most 8
 * query heads per kv head; dim and hidden_dim <= 32768. */
typedef struct ld_config {
    int32_t dim;
    int32_t hidden_dim;
    int32_t n_layers;
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t vocab_size;
    int32_t seq_len;
} ld_config;

/* Options.  norm_eps is added to mean(x^2) inside the RMSNorm square root
 * (1e-5 on the "run.c" page).  rope_theta is the RoPE base (10000).
 * shared_classifier = 1 makes the classifier the embedding table ("run.c"
 * transformer(); "run.c 逐行解讀" §2 wcls may share the embedding), 0 reads a
 * separate wcls from the end of the blob.  flags: LD_OPT_* bits.
 * max_batch: the number of sequences with a KV cache of their own (0 or 1:
 * one), for ld_forward_batch / ld_generate_greedy_batch; the single-sequence
 * calls use sequence 0.  With max_batch > 4, and dim, hidden_dim, kv_dim and
 * vocab_size multiples of 16, ld_create also keeps a second copy of the
 * weight matrices and the classifier in device memory (about the size of the
 * blob), laid out for the matrix-core products of 5 to 64 sequences, and a
 * 4 MB workspace with one counter per compute unit for their K split. */
typedef struct ld_options {
    float norm_eps;
    float rope_theta;
    int32_t shared_classifier;
    int32_t flags;
    int32_t max_batch;
} ld_options;

/* Replay-free mode: launch every kernel of a step directly instead of
 * replaying the captured per-token HIP graph.  Results are bit-identical. */
#define LD_OPT_NO_GRAPH 1
/* Every decode step launches the attention kernel of each layer on its own.
 * Without this flag, models with dim <= 256 (where the fused launch measured
 * faster; the fused kernel also needs head size 16, 32, 48, 64 or 128 and at
 * most two query heads per kv head) run each layer's q/k/v product and
 * attention as one launch (ld_op_qkv_attention) at short contexts, where the
 * keys and values of one kv head fill at most 64 KB.  Both compute the same
 * attention; the sums are taken in a different order, so results agree to
 * rounding. */
#define LD_OPT_NO_FUSE 2

typedef struct ld_model ld_model;

enum {
    LD_OK = 0,
    LD_E_NULL = -1,        /* a required pointer argument is NULL */
    LD_E_CONFIG = -2,      /* the config or options are invalid (see ld_config) */
    LD_E_SIZE = -3,        /* the weight blob has the wrong size */
    LD_E_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
    LD_E_RANGE = -5,       /* token, pos or a step count is out of range */
    LD_E_OOM = -6,         /* a device allocation failed */
    LD_E_HIP = -7,         /* a HIP runtime call failed */
    LD_E_UNSUPPORTED = -8  /* valid shape that the compiled kernels do not cover */
};

/* Size in bytes of the weight blob for (cfg, opt).  The blob is fp32,
 * contiguous, no padding, tensors in this order (checkpoint order of the
 * "run.c" page, checkpoint_init_weights, with the grouped-query shapes and the
 * separate classifier of "run.c 逐行解讀" §2; no RoPE tables):
 *   E (V,dim) | rms_att (L,dim) | wq (L,dim,dim) | wk (L,kv_dim,dim) |
 *   wv (L,kv_dim,dim) | wo (L,dim,dim) | rms_ffn (L,dim) | w1 (L,hidden,dim) |
 *   w2 (L,dim,hidden) | w3 (L,hidden,dim) | rms_final (dim) |
 *   [wcls (V,dim) when shared_classifier == 0]
 * Needs no GPU.  Errors: LD_E_NULL, LD_E_CONFIG. */
int ld_weights_size(const ld_config* cfg, const ld_options* opt, size_t* bytes_out);

/* Create a model over a device weight blob.
 *   d_weights: device memory holding the blob (layout above), 16-byte aligned,
 *              exactly ld_weights_size bytes.  Borrowed, never written; it must
 *              stay valid until ld_destroy.
 *   hip_stream: the caller's hipStream_t (NULL = the null stream).  Work of a
 *              call starts after the work already queued on it, and later work
 *              queued on it starts after the call's work.
 * The library allocates and owns the KV caches (zeroed), the activations, the
 * logits and the per-token graph.  Errors: LD_E_NULL, LD_E_CONFIG,
 * LD_E_UNSUPPORTED, LD_E_SIZE, LD_E_ALIGN, LD_E_OOM, LD_E_HIP. */
int ld_create(const ld_config* cfg, const ld_options* opt, const void* d_weights, size_t bytes,
              void* hip_stream, ld_model** out);

/* Zero the KV caches of every sequence (the calloc'd state of the pages).
 * Asynchronous. */
int ld_reset(ld_model* m);

/* One decode step at (token, pos): writes KV-cache row pos of every layer,
 * attends over rows 0..pos (never reads a row above pos) and leaves the logits
 * (vocab_size floats, library-owned device memory) at *d_logits_out, valid
 * until the next call on this model and ready in stream order.  Asynchronous.
 * Needs 0 <= token < vocab_size and 0 <= pos < seq_len, else LD_E_RANGE. */
int ld_forward(ld_model* m, int32_t token, int32_t pos, const float** d_logits_out);

/* Lowest index holding the maximum of the last step's logits (the strict '>'
 * scan of argmax() on the "run.c" page).  Synchronous. */
int ld_argmax_last(ld_model* m, int32_t* h_token_out);

/* Greedy generation: for i = 0..n_steps-1, logits = forward(tok_i, pos + i),
 * tok_{i+1} = argmax(logits), h_tokens_out[i] = tok_{i+1}; tok_0 = token.
 * No stop token.  Needs pos + n_steps <= seq_len (else LD_E_RANGE).
 * h_tokens_out: caller-owned host array of n_steps int32.  Synchronous. */
int ld_generate_greedy(ld_model* m, int32_t token, int32_t pos, int32_t n_steps, int32_t* h_tokens_out);

/* Prompt prefill: the decode step for h_tokens[i] at position pos + i, for
 * i = 0 .. n_tokens - 1, computed for all prompt tokens at once (the R/Keras
 * page's call_with_cache over a whole prompt with its causal mask; the same
 * result as n_tokens ld_forward calls in order).  Cache rows pos ..
 * pos + n_tokens - 1 of every layer are written; *d_logits_out receives the
 * logits of the last token (library-owned device memory, as ld_forward's),
 * and ld_argmax_last then returns their argmax.  Needs 1 <= n_tokens and
 * pos + n_tokens <= seq_len; every token id in [0, vocab_size).
 * h_tokens: caller-owned host array, read before the call returns.
 * Asynchronous on the model's stream, like ld_forward.  LD_E_UNSUPPORTED for
 * a head size the prefill attention kernel has no instance for. */
int ld_prefill(ld_model* m, const int32_t* h_tokens, int32_t n_tokens, int32_t pos, const float** d_logits_out);

/* ld_prefill into the KV cache of sequence seq (0 <= seq < max_batch, else
 * LD_E_RANGE) of a batch model, e.g. each prompt of a batch before
 * ld_generate_greedy_batch; ld_prefill is ld_prefill_seq with seq 0. */
int ld_prefill_seq(ld_model* m, int32_t seq, const int32_t* h_tokens, int32_t n_tokens, int32_t pos,
                   const float** d_logits_out);

/* How the generation loop chooses tokens after the prompt ("run.c 逐行解讀"
 * §6, sample(), three modes):
 *   temperature <= 0: the argmax (greedy, as above);
 *   temperature > 0:  a draw from softmax(logits / temperature), with coin c
 *     in [0, 1): the first token, in walk order, whose cumulative probability
 *     exceeds c times the candidates' mass.  With topp <= 0 or topp >= 1 every
 *     token is a candidate and the walk is in index order (sample() of the
 *     "run.c" page).  With 0 < topp < 1 the candidates are the smallest set of
 *     most likely tokens whose probabilities sum to at least topp, walked in
 *     descending probability, equal probabilities in index order.
 * stop_token: -1 for none, else a token id that ends the loop (§7, which ends
 * at BOS = 1; the id is the caller's choice here). */
typedef struct {
    float temperature;
    float topp;
    int32_t stop_token;
    int32_t reserved; /* 0 */
} ld_sampling;

/* The generation loop of "run.c 逐行解讀" §7.  Step i (i = 0, 1, ...) runs the
 * decode step on token t_i at position pos + i, t_0 = h_prompt[0]; its next
 * token t_{i+1} is h_prompt[i + 1] while the prompt lasts (i + 1 < n_prompt),
 * else the choice `sampling` describes, drawing with coin h_coins[i].
 * h_tokens_out[i] = t_{i+1}.  The loop ends after n_steps steps, or after the
 * step whose next token (forced or chosen) equals the stop token; that token
 * is the last one written.  *n_out receives the number of steps run.
 *
 * h_prompt: n_prompt >= 1 token ids in [0, vocab_size).  h_coins: host array
 * of n_steps floats in [0, 1); entries i < n_prompt - 1 are not read; may be
 * NULL when temperature <= 0.  Random numbers are the caller's, so a run is a
 * function of its arguments.  Needs pos + n_steps <= seq_len.  Cache rows
 * pos .. pos + *n_out - 1 are written; nothing above them.
 * Errors: LD_E_NULL, LD_E_RANGE (a token, position, count, coin, temperature
 * or stop id out of range), LD_E_UNSUPPORTED (temperature > 0 with
 * vocab_size > 32768).  Synchronous. */
int ld_generate(ld_model* m, const int32_t* h_prompt, int32_t n_prompt, int32_t pos, int32_t n_steps,
                const ld_sampling* sampling, const float* h_coins, int32_t* h_tokens_out, int32_t* n_out);

/* Batch decode: one decode step for each of n sequences at once (n <=
 * max_batch): sequence b runs forward(h_tokens[b], h_pos[b]) on its own KV
 * cache; the steps share each weight read (the R/Keras page's batch axis).
 * *d_logits_out receives n rows of vocab_size logits (library-owned device
 * memory, valid until the next call).  0 <= h_pos[b] < seq_len; ids in
 * range.  Asynchronous on the model's stream; h_tokens and h_pos are read
 * before the call returns. */
int ld_forward_batch(ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int32_t n,
                     const float** d_logits_out);

/* Greedy generation for n sequences in lockstep: sequence b starts from token
 * h_tokens[b] at position h_pos[b] and runs n_steps steps as
 * ld_generate_greedy does; h_tokens_out[b * n_steps + i] is its token after
 * step i.  Needs h_pos[b] + n_steps <= seq_len.  Synchronous. */
int ld_generate_greedy_batch(ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int32_t n,
                             int32_t n_steps, int32_t* h_tokens_out);

/* Device pointers of the key and value caches, each (max_batch, n_layers,
 * seq_len, kv_dim) fp32 row-major, and their size in floats.  The caller may
 * read or overwrite them between calls (e.g. to install a cache prefix). */
int ld_kv_cache(ld_model* m, float** d_key_out, float** d_value_out, size_t* floats_out);

/* Free everything the model owns.  NULL is accepted. */
void ld_destroy(ld_model* m);

/* Text for a status code; never NULL. */
const char* ld_strerror(int status);

/* Text naming the HIP call and error behind the calling thread's most recent
 * LD_E_HIP or LD_E_OOM ("" if none); never NULL. */
const char* ld_last_error_detail(void);

/* ---------------------------------------------------------------------------
 * Kernel timing.  Runs n_steps greedy decode steps from (token, pos) with
 * every kernel launched directly and timed with HIP events on the model's
 * stream: the GEMV kernels and attention (its split kernel, plus the merge
 * kernel where the partials of a kv group are too many for the split
 * kernel's last block to merge) with events recorded by their own dispatch
 * (their interval is the kernels' execution), the classifier (GEMV and
 * next-token kernels) between events recorded on the stream around them.  Reports per kernel kind the launch count
 * and the summed event time.  Kinds: "qkv_rope_append", "attention", "wo_residual",
 * "w1w3_swiglu", "w2_residual", "classifier_argmax", and "qkv_attention" (the
 * q/k/v product with the attention in the same launch, at short contexts
 * unless LD_OPT_NO_FUSE).  stats must hold
 * max_stats entries; *n_stats_out receives the number filled.  Synchronous.
 */
typedef struct ld_kernel_stat {
    char name[32];
    int32_t launches;
    double total_ms;
} ld_kernel_stat;

int ld_profile_steps(ld_model* m, int32_t token, int32_t pos, int32_t n_steps, ld_kernel_stat* stats,
                     int32_t max_stats, int32_t* n_stats_out);

/* ---------------------------------------------------------------------------
 * Single kernels of the step, for testing each against its definition.  Each
 * runs the same kernel the model uses, on hip_stream (NULL = null stream),
 * allocates its own temporaries and returns after the stream has synchronised.
 * Shapes follow the ld_config rules (n and rows multiples of 4, n <= 32768).
 */

/* d_out(rows) = W(rows, n) . x'(n), x' = g * x / sqrt(mean(x^2) + eps) when
 * d_g != NULL ("run.c 逐行解讀" §4 RMSNorm and Matmul), x' = x when d_g == NULL. */
int ld_op_rmsnorm_gemv(const float* d_x, const float* d_g, float eps, const float* d_w, int32_t rows,
                       int32_t n, float* d_out, void* hip_stream);

/* d_x(rows) += W(rows, n) . d_in(n)  (§4 steps 2f and 2h: projection + residual). */
int ld_op_gemv_residual(const float* d_in, const float* d_w, int32_t rows, int32_t n, float* d_x,
                        void* hip_stream);

/* d_hb(hidden) = silu(W1 . x') * (W3 . x'), x' = RMSNorm(x) with gain g
 * (§4 steps 2g-2h). */
int ld_op_swiglu(const float* d_x, const float* d_g, float eps, const float* d_w1, const float* d_w3,
                 int32_t hidden, int32_t n, float* d_hb, void* hip_stream);

/* q = Wq x', k = Wk x', v = Wv x' with x' = RMSNorm(x, g), then RoPE at pos on
 * the n_heads heads of q and the n_kv_heads heads of k (§4 steps 2a-2d).
 * q: dim floats; k, v: kv_dim floats. */
int ld_op_qkv_rope(const float* d_x, const float* d_g, float eps, const float* d_wq, const float* d_wk,
                   const float* d_wv, int32_t dim, int32_t n_heads, int32_t n_kv_heads, int32_t pos,
                   float theta, float* d_q, float* d_k, float* d_v, void* hip_stream);

/* The q/k/v product and the attention of one layer at pos in one launch
 * (§4 steps 2a-2e), the kernel of the decode step at short contexts: x' =
 * RMSNorm(x, g) (no norm when d_g == NULL), q = Wq x', k = Wk x', v = Wv x',
 * RoPE at pos on q and k, k and v written to row pos of d_kc / d_vc (rows of
 * kv_dim floats; rows 0..pos-1 are read as the earlier keys and values), then
 * d_out (dim floats) = the causal attention of every query head over rows
 * 0..pos, query head h on kv head floor(h*n_kv/n_heads).  q itself is not
 * returned.  Synchronous.  Errors: LD_E_NULL, LD_E_CONFIG, LD_E_RANGE (pos <
 * 0), LD_E_ALIGN, LD_E_UNSUPPORTED for a shape without the fused kernel (head
 * size other than 16/32/48/64/128, more than two query heads per kv head or 64
 * kv heads, dim > 4096), LD_E_HIP. */
int ld_op_qkv_attention(const float* d_x, const float* d_g, float eps, const float* d_wq, const float* d_wk,
                        const float* d_wv, int32_t dim, int32_t n_heads, int32_t n_kv_heads, int32_t pos,
                        float theta, float* d_kc, float* d_vc, float* d_out, void* hip_stream);

/* Causal GQA attention of one layer at pos (§4 step 2e): d_q (n_heads *
 * head_size), d_kc / d_vc (at least pos+1 rows of kv_dim floats), d_out
 * (n_heads * head_size).  Query head h reads kv head floor(h*n_kv/n_heads). */
int ld_op_attention(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads,
                    int32_t n_kv_heads, int32_t head_size, int32_t pos, float* d_out, void* hip_stream);

/* ld_op_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same result, bit for bit, with the split partials,
 * the arrival counts and the position kept in a device array of
 * LD_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends (looked up on the first call on a GPU; nothing is
 * allocated).  The caller passes the inputs and the output as for
 * ld_op_attention.  Every call on one GPU uses that GPU's array and leaves its
 * contents there: calls that overlap on one GPU (on different streams, or from
 * different threads) race and must not be made.  Asynchronous on hip_stream
 * (NULL = the null stream): the output is ready in stream order; no call waits
 * for the stream.  Errors: those of ld_op_attention, and LD_E_SIZE when the
 * partials of (n_heads, head_size, pos) need more than the array holds
 * (ld_last_error_detail gives the bytes); LD_E_HIP if the array's address
 * cannot be found. */
#define LD_NOALLOC_SCRATCH_BYTES (4u << 20)
int ld_op_attention_noalloc(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_size, int32_t pos, float* d_out, void* hip_stream);

/* d_out (m x n) = d_a (m x k) * d_w (n x k)^T, all fp32 row-major: the
 * matrix product of prefill, out[i][j] = sum_t a[i][t] w[j][t] ("run.c 逐行解讀"
 * §4 Matmul, for m input vectors at once).  k % 4 == 0 (else LD_E_CONFIG);
 * d_a and d_w 16-byte aligned (else LD_E_ALIGN).  Synchronous. */
int ld_op_gemm(const float* d_a, const float* d_w, int32_t m, int32_t n, int32_t k, float* d_out,
               void* hip_stream);

/* Causal attention of n_tokens queries at positions pos .. pos + n_tokens - 1
 * ("run.c 逐行解讀" §4 step 2e for each of them): d_q (n_tokens,
 * n_heads * head_size), caches with rows of n_kv_heads * head_size floats,
 * rows 0 .. pos + n_tokens - 1 read; query head h reads kv head
 * floor(h * n_kv_heads / n_heads).  d_out (n_tokens, n_heads * head_size).
 * Synchronous. */
int ld_op_attention_prefill(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_size, int32_t pos, int32_t n_tokens, float* d_out,
                            void* hip_stream);

/* Lowest index of the maximum of d_v[0..n) ("run.c", argmax). */
int ld_op_argmax(const float* d_v, int32_t n, int32_t* h_index_out, void* hip_stream);

/* One token drawn from the logits d_logits[0..n) as ld_sampling describes
 * (temperature, topp; stop_token unused), with coin in [0, 1).  n <= 32768
 * when temperature > 0 (else LD_E_UNSUPPORTED).  Synchronous. */
int ld_op_sample(const float* d_logits, int32_t n, float temperature, float topp, float coin,
                 int32_t* h_token_out, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Measurement.  A plain streaming read of d_src[0..bytes): the practical HBM
 * read ceiling that the decode step's weight streams are reported against
 * (the step reads every weight once per token, so its bound is the read
 * bandwidth).  The buffer is split into LD_STREAM_READ_BLOCKS contiguous
 * shares of bytes / 16 float4 (share b starts at float4 b * ceil(n / blocks));
 * d_sums[b] receives the fp32 sum of share b's floats in an unspecified
 * order, which keeps every load live.  bytes > 0 and a multiple of 16 (else
 * LD_E_SIZE); d_src 16-byte aligned (else LD_E_ALIGN); d_sums holds
 * LD_STREAM_READ_BLOCKS floats.  Asynchronous on hip_stream (NULL = null
 * stream), so that HIP events around it time the kernel alone.
 */
#define LD_STREAM_READ_BLOCKS 2048
int ld_op_stream_read(const void* d_src, size_t bytes, float* d_sums, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* LD_H */
