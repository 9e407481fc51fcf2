// Internal interface between the kernels (ld_kernels.hip) and the runtime
// (ld_runtime.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ld {

// Per-step scalars kept in device memory so that one captured graph serves
// every position: the next-token kernel writes `next` and advances
// (token, pos) for the following step.  Once a step has chosen the stop token
// `stopped` is set: later steps write no cache row and choose nothing, so
// graph replays queued past the stop leave the model where it stopped.
struct StepState {
    int32_t token;
    int32_t pos;
    int32_t next;
    int32_t stopped;
};

// How the next token is chosen ("run.c 逐行解讀" §6 and §7).  The step at
// position p takes forced[p + 1] while p + 1 < force_end (the prompt); else
// the argmax when temperature <= 0; else a draw with coin coins[p] from
// softmax(logits / temperature), over the smallest most likely set of
// cumulative probability >= topp when 0 < topp < 1.
struct GenControl {
    float temperature;
    float topp;
    int32_t stop_token;  // -1: none
    int32_t force_end;   // absolute position bound of the forced tokens
};

struct NextTokenParams {
    const float2* best;    // per-block (value, index bits) of the logits
    int nblocks;
    const float* logits;
    int n;                 // vocabulary size
    const GenControl* ctl;
    const int32_t* forced; // by position
    const float* coins;    // by position
    StepState* state;
    int32_t* tokens_out;   // tokens_out[pos] = the token chosen at position pos (may be NULL)
};

// Kinds of the matrix-vector kernel family.  All read one fp32 row-major
// weight matrix (or a pair / triple of them) once and differ in the prologue
// (optional RMSNorm of x) and the epilogue.
enum GemvKind : int {
    K_PLAIN = 0,   // out[r] = W x'
    K_RESID = 1,   // x_resid[r] += W in
    K_QKV = 2,     // [Wq;Wk;Wv] x', RoPE on q and k, k/v into cache row pos
    K_SWIGLU = 3,  // hb[e] = silu(W1 x')[e] * (W3 x')[e]
    K_CLS = 4,     // logits[r] = Wcls x', then the greedy argmax
    K_QKV_ATT = 5, // K_QKV, q/k/v also handed to the attention of the same
                   // launch (qkv_attention_launch); q itself is not stored
};

// Launch geometry: `nt` threads per block, each holding `nx` float4 of x;
// `rpi` weight rows per iteration; `units` row groups split evenly over `grid`
// blocks.
struct GemvPlan {
    int kind;
    int nt;
    int nx;
    int rpi;
    int units;
    int grid;
    int nb;                // 0: one vector; else the batch kernel for up to nb vectors
    int grid_nb[2];        // batch: the grids of its instances for 1 and 2 vectors (grid: nb)
};

struct GemvParams {
    const float* x;        // input vector, n floats
    const float* emb;      // K_QKV at layer 0: x := emb[token] and x_resid := emb[token]
    float* x_resid;        // residual stream (K_RESID target, K_QKV layer-0 copy)
    const float* gain;     // RMSNorm gain, nullptr = no normalisation
    float eps;
    int n;                 // input length (floats)
    int rows;              // output elements (K_SWIGLU: hidden units)
    int units;             // row groups
    const float* w0;       // weights: K_QKV wq; K_SWIGLU w1; else W
    const float* w1;       // K_QKV wk; K_SWIGLU w3
    const float* w2;       // K_QKV wv
    int seg1;              // K_QKV: first k row (dim)
    int seg2;              // K_QKV: first v row (dim + kv_dim)
    float* out;            // K_PLAIN out, K_QKV q, K_SWIGLU hb, K_CLS logits
    float* kc;             // K_QKV: key cache of the layer
    float* vc;             // K_QKV: value cache of the layer
    int kv_stride;         // K_QKV: floats between cache rows (kv_dim; 0 = single row)
    int head_size;
    const float2* rope;    // K_QKV: (position, head_size/2) -> (cos, sin)
    StepState* state;
    float2* best;          // K_CLS: per-block (value, index bits)
    // K_QKV_ATT: row r of [Wq;Wk;Wv] x' (after RoPE) also goes to
    // stage[(r / head_size) * stage_sh + r % head_size] (one slot per q head,
    // then per k head, then per v head; stage_sh a multiple of 64 floats); the
    // block that completes a kv group's rows (count in arrive[group], zero
    // before and after every launch) writes that group's attention to att_out
    float* stage;
    int stage_sh;
    unsigned* arrive;
    float* att_out;
    int n_heads;
    int n_kv_heads;
    // the batch kernel (GemvPlan.nb > 0): vectors 0..nb-1, vector b at x + b ldx
    // (out + b ldo, x_resid + b ldr); K_QKV: vector b is sequence b at
    // row_state[b].pos, its caches seq_stride floats after sequence b-1's
    int nb;
    int ldx, ldo, ldr;
    const StepState* row_state;
    size_t seq_stride;
};

struct AttnParams {
    const float* q;        // n_heads * head_size
    const float* kc;       // this layer's key cache, rows of kv_dim
    const float* vc;
    float* out;            // n_heads * head_size
    float2* part_ml;       // (n_heads, nsplit) running max and sum
    float* part_acc;       // (n_heads, nsplit, head_size) unnormalised outputs
    unsigned* arrive;      // (batch, n_kv_heads) split arrival counts: zero before and after every launch
    const StepState* state;
    int n_heads;
    int n_kv_heads;
    int kv_dim;
    int nsplit;            // grid.y: the most splits a kv head's keys are cut into at this launch
    int chunk;             // keys per tile, the unit splits are made of (set by the launcher)
    int min_tiles;         // fewest tiles a split takes (set by the launcher)
    int waves;             // waves per block: attn_waves(...) of the model (0 = 4)
    int fuse;              // 1: the last split block of a kv group merges it (set by the launcher)
    int stage_sh;          // q/k/v from a hand-off stage (the fused q/k/v kernel): its slot stride
    float* out_t;          // a decode batch of <= kTiledBatch: the outputs also in the tiled layout (or NULL)
    // a decode batch (grid.z = batch; 0 or 1: one sequence): sequence b's q,
    // out and state are b * q_stride floats / b states further, its caches
    // b * seq_stride floats, its split partials b * (n_heads * nsplit) pairs
    // and b * (n_heads * nsplit * head_size) floats, its arrival counts
    // b * n_kv_heads further
    int batch;
    int q_stride;
    size_t seq_stride;
};

// Batch decode of up to kTiledBatch sequences on the matrix cores with
// pre-tiled weights (tiled_launch).  Tiled weights: a product's rows and K
// (both multiples of 16) form 16 x 16 tiles; tile (rt, kt) is 64 float4 at
// float4 offset tiled_wtile(rt, kt, rows / 16, K / 16) * 64 (groups of 8 k
// tiles, row tile after row tile within a group), float4 l holding row
// 16 rt + l % 16 at k = 16 kt + 4 (l / 16) + 0..3, times the gain of the
// product's RMSNorm at k.
// Tiled activations (vectors of n floats, planes of 16 sequences): float4
// ((plane * n/16 + kt) * 64 + l) = x[16 plane + l % 16][16 kt + 4 (l / 16) + 0..3].
#ifndef LD_TILED_BATCH
#define LD_TILED_BATCH 64
#endif
constexpr int kTiledBatch = LD_TILED_BATCH;

struct TiledParams {
    const float* w;        // tiled weights (gain folded in)
    const float* x;        // input, tiled
    int k;                 // input length
    int rows;              // output rows (K_SWIGLU: 2 x hidden, w1 and w3 rows interleaved)
    int nb;                // sequences, 1..kTiledBatch
    int norm;              // scale row b by 1/sqrt(mean(x_b^2) + eps) (the RMSNorm's row scale)
    float eps;
    float* out;            // K_PLAIN, K_QKV (q): out[b * ldo + r]
    int ldo;
    float* x_resid;        // K_RESID: x_resid[b * ldr + r] += C
    int ldr;
    float* out_t;          // K_RESID: the new residual, K_SWIGLU: hb, tiled (K_RESID: may be NULL)
    int seg1, seg2;        // K_QKV as GemvParams
    float* kc;
    float* vc;
    int kv_stride;
    int head_size;
    const float2* rope;
    const StepState* row_state;  // K_QKV: sequence b at row_state[b].pos
    size_t seq_stride;
    float* part;           // products whose row tiles do not fill the CUs: K split over blocks,
    size_t part_floats;    //   partial tiles here (NULL: no split; tiled_part_floats() suffice)
    unsigned* arrive;      //   and arrival counts (tiled_arrive_count(), kept at zero between launches)
};

// workspace of the tiled products' K split on a device with `cus` compute units
size_t tiled_part_floats(int cus);
int tiled_arrive_count(int cus);

// Pack rows x k weights into the tiled layout: kind K_PLAIN (w0), K_QKV (w0 |
// w1 | w2 with the row segments seg1, seg2), K_SWIGLU (row 2u = w0 row u, 2u+1
// = w1 row u), each column times gain[k] (gain may be NULL).
hipError_t tile_weights_launch(int kind, const float* w0, const float* w1, const float* w2, int seg1, int seg2,
                               const float* gain, int rows, int k, float* dst, hipStream_t s);
hipError_t tiled_launch(int kind, const TiledParams& p, hipStream_t s);

// Prompt prefill (ld_prefill.hip).  C(M x N) = A(M x K) B(N x K)^T on the
// matrix cores, A the T tokens' activations, B's rows the weight rows, with
// the decode GEMVs' epilogues.
enum GemmKind : int {
    G_PLAIN = 0,   // out[m][n] = C
    G_RESID = 1,   // out[m][n] += C
    G_QKV = 2,     // rows [Wq;Wk;Wv]; RoPE at position pos0 + m; q -> out, k/v -> cache rows
    G_SWIGLU = 3,  // rows interleaved (w1 row u, w3 row u); out[m][u] = silu(C[m][2u]) * C[m][2u+1]
};

struct GemmParams {
    const float* a;        // M x K, row stride lda
    int lda;
    int m, n, k;
    const float* w0;       // B rows (as GemvParams)
    const float* w1;
    const float* w2;
    int seg1, seg2;
    float* out;
    int ldo;
    float* kc;             // G_QKV: this layer's caches
    float* vc;
    int kv_stride;
    int head_size;
    const float2* rope;
    int pos0;
    const StepState* row_state;  // G_QKV of a decode batch: row m is sequence m at row_state[m].pos
    size_t seq_stride;           //   floats between two sequences' caches
    float* part;                 // workspace for split-K partials (NULL: no split)
    size_t part_floats;          //   at least gemm_part_floats(m, n, k)
    const float* gain;           // non-NULL: C = RMSNorm(A) B^T, the norm with this gain
    float eps;                   //   (over the K columns of each row of A) and eps
    int splits;                  // set by the launcher
    int kchunk;
};

struct AttnPrefillParams {
    const float* q;        // T x ldq (query heads contiguous)
    int ldq;
    const float* kc;       // this layer's caches, rows of kv_stride floats
    const float* vc;
    int kv_stride;
    float* out;            // T x ldo
    int ldo;
    int t;                 // queries: positions pos0 .. pos0 + t - 1
    int pos0;
    int n_heads;
    int n_kv_heads;
};

hipError_t embed_launch(const float* emb, const int32_t* tokens, int t, int dim, float* x, hipStream_t s);
// out[t] = RMSNorm(x[t]) with the gain, for t rows of dim floats (dim % 4 == 0)
hipError_t rmsnorm_rows_launch(const float* x, const float* gain, float eps, int t, int dim, float* out,
                               hipStream_t s);
// a decode batch: x[b] = E[st[b].token]; the greedy token of every logits row,
// tokens_out[b * tokens_stride + pos_b], and each sequence's state advances
// xt (optional): the same rows in the tiled layout of TiledParams (batch <= kTiledBatch)
hipError_t embed_state_launch(const float* emb, const StepState* st, int batch, int dim, float* x, hipStream_t s,
                              float* xt = nullptr);
hipError_t argmax_rows_launch(const float* logits, int batch, int n, StepState* st, int32_t* tokens_out,
                              int tokens_stride, hipStream_t s);
hipError_t gemm_launch(int kind, const GemmParams& p, hipStream_t s);
int gemm_splits(int m, int n, int k);  // K splits the launcher uses for m rows
size_t gemm_part_floats(int m, int n, int k);  // split workspace: splits * m * (n + 1) floats
bool attn_prefill_supported(int head_size);
hipError_t attn_prefill_launch(int head_size, const AttnPrefillParams& p, hipStream_t s);

// Plans and launchers.  Return hipSuccess, or hipErrorInvalidValue for a
// shape outside the compiled kernels.
hipError_t gemv_plan(int kind, int rows, int n, GemvPlan* plan);
// the batch kernel for up to kGemvBatch vectors (hipErrorInvalidValue when n
// is beyond its shapes); K_PLAIN, K_RESID, K_QKV, K_SWIGLU.  gemv_launch
// takes its instance for 1, 2 or kGemvBatch vectors by GemvParams.nb.
constexpr int kGemvBatch = 4;
hipError_t gemv_plan_batch(int kind, int rows, int n, GemvPlan* plan);
// start / stop (optional): events recorded by the kernel's own dispatch, so that
// their interval is the kernel's execution alone
hipError_t gemv_launch(const GemvPlan& plan, const GemvParams& p, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);

// The q/k/v kernel with the layer's attention in the same launch (kind
// K_QKV_ATT): whether (rows n of x, head size, query heads per kv head) has a
// compiled kernel, the floats of its hand-off stage, and its launch (the plan
// from gemv_plan(K_QKV_ATT, ...)).
bool qkv_attention_supported(int n, int head_size, int n_heads, int n_kv_heads);
bool qkv_attention_pays(int n);  // whether the decode step should use it (measured)
hipError_t qkv_attention_plan(int n, int head_size, int n_heads, int n_kv_heads, GemvPlan* plan);
size_t qkv_attention_stage_floats(int head_size, int n_heads, int n_kv_heads);
int qkv_attention_stage_stride(int head_size);
hipError_t qkv_attention_launch(const GemvPlan& plan, const GemvParams& p, hipStream_t s, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);

int attn_chunk(int head_size);  // > 0 for a head size the attention kernels cover
// grid.y of the attention kernel for a context of seq_len positions (the
// splits of the longest context; shorter ones use fewer, the rest exit)
int attn_splits(int head_size, int seq_len, int n_heads, int n_kv_heads);
// grid.y for a decode batch of that many sequences (at most nsplit, the
// model's attn_splits): the batch's sequences fill the grid themselves
int attn_batch_splits(int nsplit, int n_kv_heads, int batch);
// waves per attention block for a context of seq_len positions: 4, or more
// where the whole grid would be small (few kv heads, short context)
int attn_waves(int head_size, int seq_len, int n_heads, int n_kv_heads);
// attention (+ merge); start / stop (optional) as for gemv_launch: taken by the
// attention kernel's dispatch and by the last kernel's (the merge, when it runs)
hipError_t attn_launch(int head_size, const AttnParams& p, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);

hipError_t set_state_launch(StepState* st, int token, int pos, hipStream_t s);
// st->pos = pos and arrive[0 .. n_kv_heads) = 0, for one attention launch at pos
hipError_t attn_op_init_launch(StepState* st, int pos, unsigned* arrive, int n_kv_heads, hipStream_t s);
hipError_t set_control_launch(GenControl* dst, const GenControl& c, hipStream_t s);
// per-block bests of v (the classifier kernel writes its own)
hipError_t argmax_partial_launch(const float* v, int n, float2* best, int nblocks, hipStream_t s);
// block b of kStreamReadBlocks sums its contiguous share of bytes / 16 float4 into sums[b]
constexpr int kStreamReadBlocks = 2048;
hipError_t stream_read_launch(const void* src, size_t bytes, float* sums, hipStream_t s);
int argmax_blocks(int n);
// the next token from the per-block bests and the logits: st->next,
// tokens_out[pos], advance (token, pos), set `stopped` at the stop token
hipError_t next_token_launch(const NextTokenParams& p, hipStream_t s);

constexpr int kAttnThreads = 256;
constexpr int kMaxGroup = 8;   // query heads per kv head
constexpr int kMaxN = 32768;   // longest input vector of a matrix-vector kernel
constexpr int kMaxSampleVocab = 32768;  // largest vocabulary the sampler holds in registers

}  // namespace ld
