// ld_runtime.hip -- the C ABI of include/ld.h: validation, device buffer
// plan, the launch sequence of one decode step, HIP-graph capture/replay.
//
// One decode step ("run.c 逐行解讀" §4, forward()) is 5 launches per layer plus
// one: per layer
//   qkv_rope_append  RMSNorm(x) -> [Wq;Wk;Wv] -> RoPE -> q, cache row pos
//                    (layer 0 also copies the embedding row into x)
//   attention        split-key GQA attention over rows 0..pos -> xb
//   wo_residual      x += Wo xb
//   w1w3_swiglu      RMSNorm(x) -> silu(W1 .) * (W3 .) -> hb
//   w2_residual      x += W2 hb
// then classifier_argmax: RMSNorm(x) -> Wcls -> logits -> next token (the
// greedy argmax, a forced prompt token or a temperature / top-p draw, as the
// device-side GenControl says).  Token, position and the sampling control
// live in device memory, so the same captured graph replays every step of a
// generation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <utility>
#include <new>
#include <vector>

#include "ld.h"
#include "ld_internal.h"

using namespace ld;

namespace {

thread_local char g_detail[256] = "";

// Device memory of ld_op_attention_noalloc: one array per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel or a
// copy (on the host it only stands for the symbol): it uses the device
// address hipGetSymbolAddress gives for the current GPU, looked up once per
// device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};

int fail_hip(hipError_t e, const char* what) {
    std::snprintf(g_detail, sizeof(g_detail), "%s: %s", what, hipGetErrorString(e));
    return e == hipErrorOutOfMemory ? LD_E_OOM : LD_E_HIP;
}

// A copy of `count` elements through a staging or device buffer of `capacity`
// elements (checked at every copy through pinned host memory, so that no
// argument combination can reach past one).
int check_copy(size_t count, size_t capacity, const char* what) {
    if (count <= capacity) return 0;
    std::snprintf(g_detail, sizeof(g_detail), "%s: %zu elements into a buffer of %zu", what, count, capacity);
    return LD_E_RANGE;
}

#define HIP_TRY(call)                                         \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return fail_hip(e_, #call);     \
    } while (0)

bool supported_head_size(int hs) { return attn_chunk(hs) > 0; }

}  // namespace

static __device__ __align__(256) unsigned char scratch[LD_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).
int scratch_for_current_device(unsigned char** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) {
        std::snprintf(g_detail, sizeof(g_detail), "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
        return LD_E_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) {
            std::snprintf(g_detail, sizeof(g_detail), "hipGetSymbolAddress(scratch) gave a null address");
            return LD_E_HIP;
        }
        g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return LD_OK;
}

int validate(const ld_config* c, const ld_options* o) {
    if (!c || !o) return LD_E_NULL;
    if (c->dim <= 0 || c->hidden_dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
        c->vocab_size <= 0 || c->seq_len <= 0)
        return LD_E_CONFIG;
    if (c->dim % c->n_heads) return LD_E_CONFIG;
    const int hs = c->dim / c->n_heads;
    if (hs % 2) return LD_E_CONFIG;
    if (c->n_kv_heads > c->n_heads) return LD_E_CONFIG;
    if (((long long)c->dim * c->n_kv_heads) % c->n_heads) return LD_E_CONFIG;
    const long long kv = (long long)c->dim * c->n_kv_heads / c->n_heads;
    if ((c->dim % 4) || (c->hidden_dim % 4) || (kv % 4)) return LD_E_CONFIG;
    if (!(o->norm_eps >= 0.f) || !(o->rope_theta > 0.f) || !std::isfinite(o->rope_theta)) return LD_E_CONFIG;
    if (o->shared_classifier != 0 && o->shared_classifier != 1) return LD_E_CONFIG;
    if (o->max_batch < 0) return LD_E_CONFIG;
    if (!supported_head_size(hs)) return LD_E_UNSUPPORTED;
    const int group = (c->n_heads + c->n_kv_heads - 1) / c->n_kv_heads;
    if (group > kMaxGroup) return LD_E_UNSUPPORTED;
    if (c->dim > kMaxN || c->hidden_dim > kMaxN) return LD_E_UNSUPPORTED;
    return LD_OK;
}

// Blob size in floats (tensor order of the header comment).
long long blob_floats(const ld_config* c, const ld_options* o) {
    const long long d = c->dim, h = c->hidden_dim, L = c->n_layers, V = c->vocab_size;
    const long long kv = d * c->n_kv_heads / c->n_heads;
    long long f = V * d;                 // embedding
    f += L * d;                          // rms_att
    f += L * d * d + 2 * L * kv * d;     // wq, wk, wv
    f += L * d * d;                      // wo
    f += L * d;                          // rms_ffn
    f += 3 * L * h * d;                  // w1, w2, w3
    f += d;                              // rms_final
    if (!o->shared_classifier) f += V * d;
    return f;
}

enum Kind { KQKV = 0, KATTN, KWO, KFFN, KW2, KCLS, KQKVA, KNUM };
const char* kKindName[KNUM] = {"qkv_rope_append", "attention",         "wo_residual",  "w1w3_swiglu",
                               "w2_residual",     "classifier_argmax", "qkv_attention"};

// Steps whose context holds at most this many bytes of keys and values per kv
// head run the q/k/v product and the attention as one launch (one block per kv
// group streams the keys) where that launch pays (qkv_attention_pays); longer
// contexts launch the split attention kernel.
#ifndef LD_FUSE_KEY_BYTES
#define LD_FUSE_KEY_BYTES (64 << 10)
#endif

// Events around each launch, for ld_profile_steps.
struct Timer {
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> kind;
    size_t used = 0;
};

}  // namespace

struct ld_model {
    ld_config cfg{};
    ld_options opt{};
    int device = 0;
    int hs = 0, kv_dim = 0, nsplit = 0, attn_waves = 4;
    const float *emb = nullptr, *rms_att = nullptr, *wq = nullptr, *wk = nullptr, *wv = nullptr, *wo = nullptr,
                *rms_ffn = nullptr, *w1 = nullptr, *w2 = nullptr, *w3 = nullptr, *rms_final = nullptr,
                *wcls = nullptr;
    float *x = nullptr, *xb = nullptr, *q = nullptr, *hb = nullptr, *logits = nullptr;
    float *kc = nullptr, *vc = nullptr, *part_acc = nullptr;
    float2 *part_ml = nullptr, *rope = nullptr, *best = nullptr;
    StepState* state = nullptr;
    int32_t* tokens = nullptr;     // tokens[pos] = the token chosen at step pos
    int32_t* h_tokens = nullptr;   // pinned staging
    GenControl* ctl = nullptr;     // device copy of the sampling control
    GenControl ctl_host{};         // what the queued work last set it to
    int32_t* forced = nullptr;     // forced prompt tokens by position (seq_len + 1)
    float* coins = nullptr;        // coins by position (seq_len)
    int32_t* h_forced = nullptr;   // pinned staging of ld_generate's inputs
    float* h_coins = nullptr;
    StepState* h_poll = nullptr;   // pinned: 3 state snapshots
    hipEvent_t ev_poll[2] = {nullptr, nullptr};
    // prompt prefill: tokens by position, pinned staging, and the per-chunk
    // activations (grown on demand, kept until ld_destroy)
    int32_t* ptok = nullptr;
    int32_t* h_ptok = nullptr;
    hipEvent_t ev_ptok = nullptr;
    bool ptok_pending = false;
    int pf_cap = 0;
    float *pf_x = nullptr, *pf_q = nullptr, *pf_att = nullptr, *pf_hb = nullptr;
    // decode batch: max_batch sequences, each with its own cache (caches are
    // (max_batch, L, S, kv_dim)), their activations, states and tokens, and
    // one captured graph per batch size
    int max_batch = 1;
    float *bx = nullptr, *bq = nullptr, *batt = nullptr, *bhb = nullptr, *blogits = nullptr;
    unsigned* arrive = nullptr;  // (max_batch, n_kv_heads) attention split arrival counts, kept at zero
    float2* bpart_ml = nullptr;
    float* bpart_acc = nullptr;
    float* bsplit = nullptr;         // split-K partials of the batch products
    size_t bsplit_floats = 0;
    StepState* bstate = nullptr;
    int32_t* btokens = nullptr;      // (max_batch, S): the token chosen at each position
    StepState* h_bstate = nullptr;   // pinned staging
    int32_t* h_btokens = nullptr;
    hipEvent_t ev_bstate = nullptr;
    bool bstate_pending = false;
    std::map<int, std::pair<hipGraph_t, hipGraphExec_t>> batch_graphs;
    GemvPlan pq{}, pwo{}, pffn{}, pw2{}, pcls{};
    GemvPlan bpq{}, bpwo{}, bpffn{}, bpw2{}, bpcls{};  // batches of up to kGemvBatch
    bool bgemv = false;                                  //   (when every shape but the down projection has one)
    bool bgemv_w2 = false;                               //   the down projection has one too
    // batches of kGemvBatch+1 .. kTiledBatch: the tiled matrix-core products
    // (max_batch > kGemvBatch and every dimension a multiple of 16): the
    // weights again in the tiled layout with the RMSNorm gains folded in, and
    // the batch's residual and hidden vectors in the tiled layout
    bool tiled = false;
    float *t_qkv = nullptr, *t_wo = nullptr, *t_ffn = nullptr, *t_w2 = nullptr, *t_cls = nullptr;
    float *bxt = nullptr, *bhbt = nullptr, *batt_t = nullptr;
    float* t_part = nullptr;       // K-split partials of the tiled products (tiled_part_floats)
    size_t t_part_floats = 0;
    unsigned* t_arrive = nullptr;  // their arrival counts, kept at zero between launches
    hipStream_t stream = nullptr, user = nullptr;
    hipEvent_t ev_in = nullptr, ev_out = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    bool use_graph = true;
    // short contexts: the q/k/v kernel with the attention in the same launch
    // (positions pos with pos + 1 <= fuse_keys), its own captured step
    int fuse_keys = 0;
    GemvPlan pqa{};
    float* stage = nullptr;
    unsigned* qkv_arrive = nullptr;  // (n_kv_heads) kept at zero between launches
    hipGraph_t graph_f = nullptr;
    hipGraphExec_t exec_f = nullptr;
    std::vector<void*> dev_allocs;
};

namespace {

template <class T>
int dalloc(ld_model* m, T** p, size_t count) {
    void* q = nullptr;
    hipError_t e = hipMalloc(&q, count * sizeof(T) < 256 ? 256 : count * sizeof(T));
    if (e != hipSuccess) return fail_hip(e, "hipMalloc");
    m->dev_allocs.push_back(q);
    *p = static_cast<T*>(q);
    return LD_OK;
}

void release(ld_model* m) {
    if (!m) return;
    (void)hipSetDevice(m->device);
    if (m->stream) (void)hipStreamSynchronize(m->stream);
    if (m->exec) (void)hipGraphExecDestroy(m->exec);
    if (m->graph) (void)hipGraphDestroy(m->graph);
    if (m->exec_f) (void)hipGraphExecDestroy(m->exec_f);
    if (m->graph_f) (void)hipGraphDestroy(m->graph_f);
    for (auto& g : m->batch_graphs) {
        if (g.second.second) (void)hipGraphExecDestroy(g.second.second);
        if (g.second.first) (void)hipGraphDestroy(g.second.first);
    }
    if (m->h_bstate) (void)hipHostFree(m->h_bstate);
    if (m->h_btokens) (void)hipHostFree(m->h_btokens);
    if (m->ev_bstate) (void)hipEventDestroy(m->ev_bstate);
    for (void* p : m->dev_allocs) (void)hipFree(p);
    for (float* p : {m->pf_x, m->pf_q, m->pf_att, m->pf_hb})
        if (p) (void)hipFree(p);
    if (m->h_ptok) (void)hipHostFree(m->h_ptok);
    if (m->ev_ptok) (void)hipEventDestroy(m->ev_ptok);
    if (m->h_tokens) (void)hipHostFree(m->h_tokens);
    if (m->h_forced) (void)hipHostFree(m->h_forced);
    if (m->h_coins) (void)hipHostFree(m->h_coins);
    if (m->h_poll) (void)hipHostFree(m->h_poll);
    for (hipEvent_t e : m->ev_poll)
        if (e) (void)hipEventDestroy(e);
    if (m->ev_in) (void)hipEventDestroy(m->ev_in);
    if (m->ev_out) (void)hipEventDestroy(m->ev_out);
    if (m->stream) (void)hipStreamDestroy(m->stream);
    delete m;
}

constexpr GenControl kGreedy = {0.f, 0.f, -1, 0};

// Queue a change of the device-side control when it differs from the last one.
int set_control(ld_model* m, const GenControl& c) {
    if (std::memcmp(&c, &m->ctl_host, sizeof(c)) == 0) return LD_OK;
    HIP_TRY(set_control_launch(m->ctl, c, m->stream));
    m->ctl_host = c;
    return LD_OK;
}

// Order the model's stream after the caller's queued work, and back.
int enter(ld_model* m) {
    HIP_TRY(hipSetDevice(m->device));
    HIP_TRY(hipEventRecord(m->ev_in, m->user));
    HIP_TRY(hipStreamWaitEvent(m->stream, m->ev_in, 0));
    return LD_OK;
}

int leave(ld_model* m) {
    HIP_TRY(hipEventRecord(m->ev_out, m->stream));
    HIP_TRY(hipStreamWaitEvent(m->user, m->ev_out, 0));
    return LD_OK;
}

// RoPE table: entry (p, j) = (cos, sin) of p * theta^(-2j/head_size) for the
// pair (2j, 2j+1) of every head ("run.c 逐行解讀" §4 step 2d: freq =
// 1/theta^(head_dim/head_size), angle = pos * freq), evaluated in double and
// rounded once, so the angle carries no fp32 error at large positions.
std::vector<float2> rope_table(int positions, int hs, double theta) {
    std::vector<float2> t((size_t)positions * (hs / 2));
    for (int p = 0; p < positions; ++p)
        for (int j = 0; j < hs / 2; ++j) {
            const double freq = 1.0 / std::pow(theta, (2.0 * j) / (double)hs);
            const double ang = (double)p * freq;
            t[(size_t)p * (hs / 2) + j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
    return t;
}

GemvParams base_params(const ld_model* m) {
    GemvParams p{};
    p.eps = m->opt.norm_eps;
    p.state = m->state;
    return p;
}

void mark(Timer* t, hipStream_t s, int kind, bool before) {
    if (!t) return;
    if (before) {
        t->kind[t->used / 2] = kind;
    }
    (void)hipEventRecord(t->ev[t->used++], s);
}

// the next event pair of the timer for a kernel that records them itself
// (gemv_launch), or none without a timer
std::pair<hipEvent_t, hipEvent_t> pair_for(Timer* t, int kind) {
    if (!t) return {nullptr, nullptr};
    t->kind[t->used / 2] = kind;
    const size_t i = t->used;
    t->used += 2;
    return {t->ev[i], t->ev[i + 1]};
}

// Whether the step at position pos takes the fused q/k/v + attention launch.
bool fused_at(const ld_model* m, long long pos) { return pos + 1 <= m->fuse_keys; }

// One decode step, reading (token, pos) from m->state.  fused: the q/k/v
// kernel also runs the attention (for positions with fused_at).
int launch_step(ld_model* m, Timer* timer, bool fused) {
    const ld_config& c = m->cfg;
    const size_t d = c.dim, h = c.hidden_dim, kv = m->kv_dim;
    const size_t cache_layer = (size_t)c.seq_len * kv;
    hipStream_t s = m->stream;
    for (int l = 0; l < c.n_layers; ++l) {
        if (fused) {
            GemvParams p = base_params(m);
            p.x = m->x;
            p.emb = l == 0 ? m->emb : nullptr;
            p.x_resid = m->x;
            p.gain = m->rms_att + (size_t)l * d;
            p.n = c.dim;
            p.rows = c.dim + 2 * m->kv_dim;
            p.w0 = m->wq + (size_t)l * d * d;
            p.w1 = m->wk + (size_t)l * kv * d;
            p.w2 = m->wv + (size_t)l * kv * d;
            p.seg1 = c.dim;
            p.seg2 = c.dim + m->kv_dim;
            p.kc = m->kc + (size_t)l * cache_layer;
            p.vc = m->vc + (size_t)l * cache_layer;
            p.kv_stride = m->kv_dim;
            p.head_size = m->hs;
            p.rope = m->rope;
            p.stage = m->stage;
            p.stage_sh = qkv_attention_stage_stride(m->hs);
            p.arrive = m->qkv_arrive;
            p.att_out = m->xb;
            p.n_heads = c.n_heads;
            p.n_kv_heads = c.n_kv_heads;
            const auto ev = pair_for(timer, KQKVA);
            HIP_TRY(qkv_attention_launch(m->pqa, p, s, ev.first, ev.second));
        } else {
            GemvParams p = base_params(m);
            p.x = m->x;
            p.emb = l == 0 ? m->emb : nullptr;
            p.x_resid = m->x;
            p.gain = m->rms_att + (size_t)l * d;
            p.n = c.dim;
            p.rows = c.dim + 2 * m->kv_dim;
            p.w0 = m->wq + (size_t)l * d * d;
            p.w1 = m->wk + (size_t)l * kv * d;
            p.w2 = m->wv + (size_t)l * kv * d;
            p.seg1 = c.dim;
            p.seg2 = c.dim + m->kv_dim;
            p.out = m->q;
            p.kc = m->kc + (size_t)l * cache_layer;
            p.vc = m->vc + (size_t)l * cache_layer;
            p.kv_stride = m->kv_dim;
            p.head_size = m->hs;
            p.rope = m->rope;
            const auto ev = pair_for(timer, KQKV);
            HIP_TRY(gemv_launch(m->pq, p, s, ev.first, ev.second));
        }
        if (!fused) {
            AttnParams a{};
            a.q = m->q;
            a.kc = m->kc + (size_t)l * cache_layer;
            a.vc = m->vc + (size_t)l * cache_layer;
            a.out = m->xb;
            a.part_ml = m->part_ml;
            a.part_acc = m->part_acc;
            a.arrive = m->arrive;
            a.state = m->state;
            a.n_heads = c.n_heads;
            a.n_kv_heads = c.n_kv_heads;
            a.kv_dim = m->kv_dim;
            a.nsplit = m->nsplit;
            a.waves = m->attn_waves;
            const auto ev = pair_for(timer, KATTN);
            HIP_TRY(attn_launch(m->hs, a, s, ev.first, ev.second));
        }
        {
            GemvParams p = base_params(m);
            p.x = m->xb;
            p.x_resid = m->x;
            p.n = c.dim;
            p.rows = c.dim;
            p.w0 = m->wo + (size_t)l * d * d;
            const auto ev = pair_for(timer, KWO);
            HIP_TRY(gemv_launch(m->pwo, p, s, ev.first, ev.second));
        }
        {
            GemvParams p = base_params(m);
            p.x = m->x;
            p.gain = m->rms_ffn + (size_t)l * d;
            p.n = c.dim;
            p.rows = c.hidden_dim;
            p.w0 = m->w1 + (size_t)l * h * d;
            p.w1 = m->w3 + (size_t)l * h * d;
            p.out = m->hb;
            const auto ev = pair_for(timer, KFFN);
            HIP_TRY(gemv_launch(m->pffn, p, s, ev.first, ev.second));
        }
        {
            GemvParams p = base_params(m);
            p.x = m->hb;
            p.x_resid = m->x;
            p.n = c.hidden_dim;
            p.rows = c.dim;
            p.w0 = m->w2 + (size_t)l * d * h;
            const auto ev = pair_for(timer, KW2);
            HIP_TRY(gemv_launch(m->pw2, p, s, ev.first, ev.second));
        }
    }
    GemvParams p = base_params(m);
    p.x = m->x;
    p.gain = m->rms_final;
    p.n = c.dim;
    p.rows = c.vocab_size;
    p.w0 = m->wcls;
    p.out = m->logits;
    p.best = m->best;
    mark(timer, s, KCLS, true);
    HIP_TRY(gemv_launch(m->pcls, p, s));
    NextTokenParams nt{};
    nt.best = m->best;
    nt.nblocks = m->pcls.grid;
    nt.logits = m->logits;
    nt.n = c.vocab_size;
    nt.ctl = m->ctl;
    nt.forced = m->forced;
    nt.coins = m->coins;
    nt.state = m->state;
    nt.tokens_out = m->tokens;
    HIP_TRY(next_token_launch(nt, s));
    mark(timer, s, KCLS, false);
    return LD_OK;
}

int ensure_graph(ld_model* m, bool fused) {
    hipGraph_t& graph = fused ? m->graph_f : m->graph;
    hipGraphExec_t& exec = fused ? m->exec_f : m->exec;
    if (exec) return LD_OK;
    HIP_TRY(hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
    int rc = launch_step(m, nullptr, fused);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(m->stream, &g);
    if (rc != LD_OK) {
        if (g) (void)hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess) return fail_hip(e, "hipStreamEndCapture");
    graph = g;
    HIP_TRY(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    return LD_OK;
}

// The step at position pos (the position the device state holds when the
// step runs; after a stop token the state stays put, and either launch
// sequence leaves it so).
int run_step(ld_model* m, long long pos) {
    const bool fused = fused_at(m, pos);
    if (m->use_graph) {
        int rc = ensure_graph(m, fused);
        if (rc != LD_OK) return rc;
        HIP_TRY(hipGraphLaunch(fused ? m->exec_f : m->exec, m->stream));
        return LD_OK;
    }
    return launch_step(m, nullptr, fused);
}

#ifndef LD_PREFILL_NORM_ROWS
#define LD_PREFILL_NORM_ROWS 1
#endif

// Tokens per prefill chunk: chunks run one after another, each attending to
// the cache rows the earlier ones wrote.
constexpr int kPrefillChunk = 2048;

int prefill_workspace(ld_model* m, int tokens) {
    if (tokens <= m->pf_cap) return LD_OK;
    HIP_TRY(hipStreamSynchronize(m->stream));
    for (float** p : {&m->pf_x, &m->pf_q, &m->pf_att, &m->pf_hb}) {
        if (*p) (void)hipFree(*p);
        *p = nullptr;
    }
    m->pf_cap = 0;
    const size_t d = (size_t)m->cfg.dim * tokens, h = (size_t)m->cfg.hidden_dim * tokens;
    hipError_t e = hipMalloc((void**)&m->pf_x, d * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&m->pf_q, d * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&m->pf_att, d * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&m->pf_hb, h * sizeof(float));
    if (e != hipSuccess) return fail_hip(e, "hipMalloc prefill workspace");
    m->pf_cap = tokens;
    return LD_OK;
}

// One chunk of T prompt tokens of sequence seq at positions p0 .. p0 + T - 1
// (their ids in m->ptok[p0 ..]): every layer of the step over all T tokens at
// once; leaves the final residual stream in pf_x.
int prefill_chunk(ld_model* m, int seq, int p0, int T) {
    const ld_config& c = m->cfg;
    const size_t d = c.dim, h = c.hidden_dim, kv = m->kv_dim;
    const size_t cache_layer = (size_t)c.seq_len * kv;
    float* kc = m->kc + (size_t)seq * c.n_layers * cache_layer;  // this sequence's caches
    float* vc = m->vc + (size_t)seq * c.n_layers * cache_layer;
    hipStream_t s = m->stream;
    HIP_TRY(embed_launch(m->emb, m->ptok + p0, T, c.dim, m->pf_x, s));
    for (int l = 0; l < c.n_layers; ++l) {
        {
            GemmParams g{};
#if LD_PREFILL_NORM_ROWS
            // the normalised rows go to pf_att (free until the attention writes it)
            HIP_TRY(rmsnorm_rows_launch(m->pf_x, m->rms_att + (size_t)l * d, m->opt.norm_eps, T, c.dim, m->pf_att, s));
            g.a = m->pf_att;
#else
            g.a = m->pf_x;
            g.gain = m->rms_att + (size_t)l * d;
            g.eps = m->opt.norm_eps;
#endif
            g.lda = c.dim;
            g.m = T;
            g.n = c.dim + 2 * m->kv_dim;
            g.k = c.dim;
            g.w0 = m->wq + (size_t)l * d * d;
            g.w1 = m->wk + (size_t)l * kv * d;
            g.w2 = m->wv + (size_t)l * kv * d;
            g.seg1 = c.dim;
            g.seg2 = c.dim + m->kv_dim;
            g.out = m->pf_q;
            g.ldo = c.dim;
            g.kc = kc + (size_t)l * cache_layer;
            g.vc = vc + (size_t)l * cache_layer;
            g.kv_stride = m->kv_dim;
            g.head_size = m->hs;
            g.rope = m->rope;
            g.pos0 = p0;
            HIP_TRY(gemm_launch(G_QKV, g, s));
        }
        {
            AttnPrefillParams a{};
            a.q = m->pf_q;
            a.ldq = c.dim;
            a.kc = kc + (size_t)l * cache_layer;
            a.vc = vc + (size_t)l * cache_layer;
            a.kv_stride = m->kv_dim;
            a.out = m->pf_att;
            a.ldo = c.dim;
            a.t = T;
            a.pos0 = p0;
            a.n_heads = c.n_heads;
            a.n_kv_heads = c.n_kv_heads;
            HIP_TRY(attn_prefill_launch(m->hs, a, s));
        }
        {
            GemmParams g{};
            g.a = m->pf_att;
            g.lda = c.dim;
            g.m = T;
            g.n = c.dim;
            g.k = c.dim;
            g.w0 = m->wo + (size_t)l * d * d;
            g.out = m->pf_x;
            g.ldo = c.dim;
            HIP_TRY(gemm_launch(G_RESID, g, s));
        }
        {
            GemmParams g{};
#if LD_PREFILL_NORM_ROWS
            // pf_att is free again once wo has read it
            HIP_TRY(rmsnorm_rows_launch(m->pf_x, m->rms_ffn + (size_t)l * d, m->opt.norm_eps, T, c.dim, m->pf_att, s));
            g.a = m->pf_att;
#else
            g.a = m->pf_x;
            g.gain = m->rms_ffn + (size_t)l * d;
            g.eps = m->opt.norm_eps;
#endif
            g.lda = c.dim;
            g.m = T;
            g.n = 2 * c.hidden_dim;
            g.k = c.dim;
            g.w0 = m->w1 + (size_t)l * h * d;
            g.w1 = m->w3 + (size_t)l * h * d;
            g.out = m->pf_hb;
            g.ldo = c.hidden_dim;
            HIP_TRY(gemm_launch(G_SWIGLU, g, s));
        }
        {
            GemmParams g{};
            g.a = m->pf_hb;
            g.lda = c.hidden_dim;
            g.m = T;
            g.n = c.dim;
            g.k = c.hidden_dim;
            g.w0 = m->w2 + (size_t)l * d * h;
            g.out = m->pf_x;
            g.ldo = c.dim;
            HIP_TRY(gemm_launch(G_RESID, g, s));
        }
    }
    return LD_OK;
}

// Attention of layer l for sequences 0..n-1 of the batch (q rows in bq, each
// sequence's own caches and position); out_t: the outputs also in the tiled
// layout there (the tiled products' batches).
hipError_t launch_batch_attention(ld_model* m, int n, int l, float* out_t = nullptr) {
    const ld_config& c = m->cfg;
    const size_t cache_layer = (size_t)c.seq_len * m->kv_dim;
    AttnParams a{};
    a.q = m->bq;
    a.kc = m->kc + (size_t)l * cache_layer;
    a.vc = m->vc + (size_t)l * cache_layer;
    a.out = m->batt;
    a.part_ml = m->bpart_ml;
    a.part_acc = m->bpart_acc;
    a.arrive = m->arrive;
    a.state = m->bstate;
    a.n_heads = c.n_heads;
    a.n_kv_heads = c.n_kv_heads;
    a.kv_dim = m->kv_dim;
    a.nsplit = attn_batch_splits(m->nsplit, c.n_kv_heads, n);
    a.waves = m->attn_waves;
    a.batch = n;
    a.q_stride = c.dim;
    a.seq_stride = (size_t)c.n_layers * cache_layer;
    a.out_t = out_t;
    return attn_launch(m->hs, a, m->stream);
}

// A decode step of up to kGemvBatch sequences with the batch GEMV kernels:
// the single step's launches (each weight streamed once, the RMSNorms fused)
// with the vectors of all sequences in registers.  A down projection wider
// than the batch kernel's shapes is the split-K matrix-core product instead.
int launch_batch_step_gemv(ld_model* m, int n) {
    const ld_config& c = m->cfg;
    const size_t d = c.dim, h = c.hidden_dim, kv = m->kv_dim;
    const size_t cache_layer = (size_t)c.seq_len * kv, seq_stride = (size_t)c.n_layers * cache_layer;
    hipStream_t s = m->stream;
    auto bparams = [&](const float* x, int ldx) {
        GemvParams p{};
        p.eps = m->opt.norm_eps;
        p.nb = n;
        p.x = x;
        p.ldx = ldx;
        p.ldr = c.dim;
        return p;
    };
    HIP_TRY(embed_state_launch(m->emb, m->bstate, n, c.dim, m->bx, s));
    for (int l = 0; l < c.n_layers; ++l) {
        {
            GemvParams p = bparams(m->bx, c.dim);
            p.gain = m->rms_att + (size_t)l * d;
            p.n = c.dim;
            p.rows = c.dim + 2 * m->kv_dim;
            p.w0 = m->wq + (size_t)l * d * d;
            p.w1 = m->wk + (size_t)l * kv * d;
            p.w2 = m->wv + (size_t)l * kv * d;
            p.seg1 = c.dim;
            p.seg2 = c.dim + m->kv_dim;
            p.out = m->bq;
            p.ldo = c.dim;
            p.kc = m->kc + (size_t)l * cache_layer;
            p.vc = m->vc + (size_t)l * cache_layer;
            p.kv_stride = m->kv_dim;
            p.head_size = m->hs;
            p.rope = m->rope;
            p.row_state = m->bstate;
            p.seq_stride = seq_stride;
            HIP_TRY(gemv_launch(m->bpq, p, s));
        }
        HIP_TRY(launch_batch_attention(m, n, l));
        {
            GemvParams p = bparams(m->batt, c.dim);
            p.x_resid = m->bx;
            p.n = c.dim;
            p.rows = c.dim;
            p.w0 = m->wo + (size_t)l * d * d;
            HIP_TRY(gemv_launch(m->bpwo, p, s));
        }
        {
            GemvParams p = bparams(m->bx, c.dim);
            p.gain = m->rms_ffn + (size_t)l * d;
            p.n = c.dim;
            p.rows = c.hidden_dim;
            p.w0 = m->w1 + (size_t)l * h * d;
            p.w1 = m->w3 + (size_t)l * h * d;
            p.out = m->bhb;
            p.ldo = c.hidden_dim;
            HIP_TRY(gemv_launch(m->bpffn, p, s));
        }
        if (m->bgemv_w2) {
            GemvParams p = bparams(m->bhb, c.hidden_dim);
            p.x_resid = m->bx;
            p.n = c.hidden_dim;
            p.rows = c.dim;
            p.w0 = m->w2 + (size_t)l * d * h;
            HIP_TRY(gemv_launch(m->bpw2, p, s));
        } else {
            GemmParams g{};
            g.a = m->bhb;
            g.lda = c.hidden_dim;
            g.m = n;
            g.part = m->bsplit;
            g.part_floats = m->bsplit_floats;
            g.n = c.dim;
            g.k = c.hidden_dim;
            g.w0 = m->w2 + (size_t)l * d * h;
            g.out = m->bx;
            g.ldo = c.dim;
            HIP_TRY(gemm_launch(G_RESID, g, s));
        }
    }
    {
        GemvParams p = bparams(m->bx, c.dim);
        p.gain = m->rms_final;
        p.n = c.dim;
        p.rows = c.vocab_size;
        p.w0 = m->wcls;
        p.out = m->blogits;
        p.ldo = c.vocab_size;
        HIP_TRY(gemv_launch(m->bpcls, p, s));
    }
    HIP_TRY(argmax_rows_launch(m->blogits, n, c.vocab_size, m->bstate, m->btokens, c.seq_len, s));
    return LD_OK;
}

// A decode step of kGemvBatch+1 .. kTiledBatch sequences with the tiled
// matrix-core products: the single step's launches (each weight streamed once
// for the batch, the RMSNorms fused), residual, attention and hidden vectors
// handed on in the tiled layout.
int launch_batch_step_tiled(ld_model* m, int n) {
    const ld_config& c = m->cfg;
    const size_t d = c.dim, h = c.hidden_dim, kv = m->kv_dim;
    const size_t cache_layer = (size_t)c.seq_len * kv, seq_stride = (size_t)c.n_layers * cache_layer;
    hipStream_t s = m->stream;
    auto base = [&](const float* w, const float* x, int k, int rows, int norm) {
        TiledParams p{};
        p.w = w;
        p.x = x;
        p.k = k;
        p.rows = rows;
        p.nb = n;
        p.norm = norm;
        p.eps = m->opt.norm_eps;
        p.part = m->t_part;
        p.part_floats = m->t_part_floats;
        p.arrive = m->t_arrive;
        return p;
    };
    HIP_TRY(embed_state_launch(m->emb, m->bstate, n, c.dim, m->bx, s, m->bxt));
    for (int l = 0; l < c.n_layers; ++l) {
        {
            TiledParams p = base(m->t_qkv + (size_t)l * (d + 2 * kv) * d, m->bxt, c.dim, c.dim + 2 * m->kv_dim, 1);
            p.out = m->bq;
            p.ldo = c.dim;
            p.seg1 = c.dim;
            p.seg2 = c.dim + m->kv_dim;
            p.kc = m->kc + (size_t)l * cache_layer;
            p.vc = m->vc + (size_t)l * cache_layer;
            p.kv_stride = m->kv_dim;
            p.head_size = m->hs;
            p.rope = m->rope;
            p.row_state = m->bstate;
            p.seq_stride = seq_stride;
            HIP_TRY(tiled_launch(K_QKV, p, s));
        }
        HIP_TRY(launch_batch_attention(m, n, l, m->batt_t));
        {
            TiledParams p = base(m->t_wo + (size_t)l * d * d, m->batt_t, c.dim, c.dim, 0);
            p.x_resid = m->bx;
            p.ldr = c.dim;
            p.out_t = m->bxt;
            HIP_TRY(tiled_launch(K_RESID, p, s));
        }
        {
            TiledParams p = base(m->t_ffn + (size_t)l * 2 * h * d, m->bxt, c.dim, 2 * c.hidden_dim, 1);
            p.out_t = m->bhbt;
            HIP_TRY(tiled_launch(K_SWIGLU, p, s));
        }
        {
            TiledParams p = base(m->t_w2 + (size_t)l * d * h, m->bhbt, c.hidden_dim, c.dim, 0);
            p.x_resid = m->bx;
            p.ldr = c.dim;
            p.out_t = m->bxt;
            HIP_TRY(tiled_launch(K_RESID, p, s));
        }
    }
    {
        TiledParams p = base(m->t_cls, m->bxt, c.dim, c.vocab_size, 1);
        p.out = m->blogits;
        p.ldo = c.vocab_size;
        HIP_TRY(tiled_launch(K_PLAIN, p, s));
    }
    HIP_TRY(argmax_rows_launch(m->blogits, n, c.vocab_size, m->bstate, m->btokens, c.seq_len, s));
    return LD_OK;
}

// One decode step of sequences 0..n-1 of the batch, each reading (token, pos)
// from m->bstate[b]: the single step's sequence of operations with the weight
// matrices as matrix-core products of n rows (each RMSNorm fused into the
// product it feeds), so every weight is read once for the whole batch.
int launch_batch_step(ld_model* m, int n) {
    if (n <= kGemvBatch && m->bgemv) return launch_batch_step_gemv(m, n);
    if (n <= kTiledBatch && m->tiled) return launch_batch_step_tiled(m, n);
    const ld_config& c = m->cfg;
    const size_t d = c.dim, h = c.hidden_dim, kv = m->kv_dim;
    const size_t cache_layer = (size_t)c.seq_len * kv, seq_stride = (size_t)c.n_layers * cache_layer;
    hipStream_t s = m->stream;
    HIP_TRY(embed_state_launch(m->emb, m->bstate, n, c.dim, m->bx, s));
    for (int l = 0; l < c.n_layers; ++l) {
        {
            GemmParams g{};
            g.a = m->bx;
            g.gain = m->rms_att + (size_t)l * d;
            g.eps = m->opt.norm_eps;
            g.lda = c.dim;
            g.m = n;
            g.part = m->bsplit;
            g.part_floats = m->bsplit_floats;
            g.n = c.dim + 2 * m->kv_dim;
            g.k = c.dim;
            g.w0 = m->wq + (size_t)l * d * d;
            g.w1 = m->wk + (size_t)l * kv * d;
            g.w2 = m->wv + (size_t)l * kv * d;
            g.seg1 = c.dim;
            g.seg2 = c.dim + m->kv_dim;
            g.out = m->bq;
            g.ldo = c.dim;
            g.kc = m->kc + (size_t)l * cache_layer;
            g.vc = m->vc + (size_t)l * cache_layer;
            g.kv_stride = m->kv_dim;
            g.head_size = m->hs;
            g.rope = m->rope;
            g.row_state = m->bstate;
            g.seq_stride = seq_stride;
            HIP_TRY(gemm_launch(G_QKV, g, s));
        }
        HIP_TRY(launch_batch_attention(m, n, l));
        {
            GemmParams g{};
            g.a = m->batt;
            g.lda = c.dim;
            g.m = n;
            g.part = m->bsplit;
            g.part_floats = m->bsplit_floats;
            g.n = c.dim;
            g.k = c.dim;
            g.w0 = m->wo + (size_t)l * d * d;
            g.out = m->bx;
            g.ldo = c.dim;
            HIP_TRY(gemm_launch(G_RESID, g, s));
        }
        {
            GemmParams g{};
            g.a = m->bx;
            g.gain = m->rms_ffn + (size_t)l * d;
            g.eps = m->opt.norm_eps;
            g.lda = c.dim;
            g.m = n;
            g.part = m->bsplit;
            g.part_floats = m->bsplit_floats;
            g.n = 2 * c.hidden_dim;
            g.k = c.dim;
            g.w0 = m->w1 + (size_t)l * h * d;
            g.w1 = m->w3 + (size_t)l * h * d;
            g.out = m->bhb;
            g.ldo = c.hidden_dim;
            HIP_TRY(gemm_launch(G_SWIGLU, g, s));
        }
        {
            GemmParams g{};
            g.a = m->bhb;
            g.lda = c.hidden_dim;
            g.m = n;
            g.part = m->bsplit;
            g.part_floats = m->bsplit_floats;
            g.n = c.dim;
            g.k = c.hidden_dim;
            g.w0 = m->w2 + (size_t)l * d * h;
            g.out = m->bx;
            g.ldo = c.dim;
            HIP_TRY(gemm_launch(G_RESID, g, s));
        }
    }
    {
        GemmParams g{};
        g.a = m->bx;
        g.gain = m->rms_final;
        g.eps = m->opt.norm_eps;
        g.lda = c.dim;
        g.m = n;
        g.part = m->bsplit;
        g.part_floats = m->bsplit_floats;
        g.n = c.vocab_size;
        g.k = c.dim;
        g.w0 = m->wcls;
        g.out = m->blogits;
        g.ldo = c.vocab_size;
        HIP_TRY(gemm_launch(G_PLAIN, g, s));
    }
    HIP_TRY(argmax_rows_launch(m->blogits, n, c.vocab_size, m->bstate, m->btokens, c.seq_len, s));
    return LD_OK;
}

int run_batch_step(ld_model* m, int n) {
    if (!m->use_graph) return launch_batch_step(m, n);
    auto it = m->batch_graphs.find(n);
    if (it == m->batch_graphs.end()) {
        HIP_TRY(hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
        int rc = launch_batch_step(m, n);
        hipGraph_t g = nullptr;
        hipError_t e = hipStreamEndCapture(m->stream, &g);
        if (rc != LD_OK) {
            if (g) (void)hipGraphDestroy(g);
            return rc;
        }
        if (e != hipSuccess) return fail_hip(e, "hipStreamEndCapture");
        hipGraphExec_t x = nullptr;
        e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            (void)hipGraphDestroy(g);
            return fail_hip(e, "hipGraphInstantiate");
        }
        it = m->batch_graphs.emplace(n, std::make_pair(g, x)).first;
    }
    HIP_TRY(hipGraphLaunch(it->second.second, m->stream));
    return LD_OK;
}

// Stage the batch's (token, pos) pairs into the device states.
int set_batch_states(ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int n) {
    if (int rc = check_copy((size_t)n, (size_t)m->max_batch, "batch states")) return rc;
    if (m->bstate_pending) HIP_TRY(hipEventSynchronize(m->ev_bstate));
    for (int b = 0; b < n; ++b) m->h_bstate[b] = StepState{h_tokens[b], h_pos[b], -1, 0};
    HIP_TRY(hipMemcpyAsync(m->bstate, m->h_bstate, sizeof(StepState) * (size_t)n, hipMemcpyHostToDevice,
                           m->stream));
    HIP_TRY(hipEventRecord(m->ev_bstate, m->stream));
    m->bstate_pending = true;
    return LD_OK;
}

int check_batch(const ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int n, int n_steps) {
    if (n < 1 || n > m->max_batch || n_steps < 0) return LD_E_RANGE;
    for (int b = 0; b < n; ++b) {
        if (h_tokens[b] < 0 || h_tokens[b] >= m->cfg.vocab_size) return LD_E_RANGE;
        if (h_pos[b] < 0 || (long long)h_pos[b] + (n_steps > 0 ? n_steps : 1) > m->cfg.seq_len) return LD_E_RANGE;
    }
    return LD_OK;
}

}  // namespace

extern "C" {

const char* ld_strerror(int status) {
    switch (status) {
        case LD_OK: return "ok";
        case LD_E_NULL: return "a required pointer argument is NULL";
        case LD_E_CONFIG: return "invalid model configuration or options";
        case LD_E_SIZE: return "weight blob has the wrong size";
        case LD_E_ALIGN: return "device pointer is not 16-byte aligned";
        case LD_E_RANGE: return "token, position or step count out of range";
        case LD_E_OOM: return "device allocation failed";
        case LD_E_HIP: return "HIP runtime call failed";
        case LD_E_UNSUPPORTED: return "shape not covered by the compiled kernels";
    }
    return "unknown status";
}

const char* ld_last_error_detail(void) { return g_detail; }

int ld_weights_size(const ld_config* cfg, const ld_options* opt, size_t* bytes_out) {
    if (!cfg || !opt || !bytes_out) return LD_E_NULL;
    const int v = validate(cfg, opt);
    if (v == LD_E_CONFIG || v == LD_E_NULL) return v;
    *bytes_out = (size_t)blob_floats(cfg, opt) * sizeof(float);
    return LD_OK;
}

int ld_create(const ld_config* cfg, const ld_options* opt, const void* d_weights, size_t bytes, void* hip_stream,
              ld_model** out) {
    if (!cfg || !opt || !d_weights || !out) return LD_E_NULL;
    *out = nullptr;
    const int v = validate(cfg, opt);
    if (v != LD_OK) return v;
    if ((size_t)blob_floats(cfg, opt) * sizeof(float) != bytes) return LD_E_SIZE;
    if (reinterpret_cast<uintptr_t>(d_weights) % 16) return LD_E_ALIGN;

    ld_model* m = new (std::nothrow) ld_model();
    if (!m) return LD_E_OOM;
    int rc = LD_OK;
    do {
        m->cfg = *cfg;
        m->opt = *opt;
        m->use_graph = !(opt->flags & LD_OPT_NO_GRAPH);
        m->max_batch = opt->max_batch > 1 ? opt->max_batch : 1;
        m->user = static_cast<hipStream_t>(hip_stream);
        hipError_t e = hipGetDevice(&m->device);
        if (e != hipSuccess) { rc = fail_hip(e, "hipGetDevice"); break; }
        m->hs = cfg->dim / cfg->n_heads;
        m->kv_dim = cfg->dim * cfg->n_kv_heads / cfg->n_heads;
        m->nsplit = attn_splits(m->hs, cfg->seq_len, cfg->n_heads, cfg->n_kv_heads);
        m->attn_waves = attn_waves(m->hs, cfg->seq_len, cfg->n_heads, cfg->n_kv_heads);

        // weight pointers: 64-bit offsets into the blob
        const float* w = static_cast<const float*>(d_weights);
        const size_t d = cfg->dim, h = cfg->hidden_dim, L = cfg->n_layers, V = cfg->vocab_size, kv = m->kv_dim;
        size_t off = 0;
        auto take = [&](size_t count) { const float* p = w + off; off += count; return p; };
        m->emb = take(V * d);
        m->rms_att = take(L * d);
        m->wq = take(L * d * d);
        m->wk = take(L * kv * d);
        m->wv = take(L * kv * d);
        m->wo = take(L * d * d);
        m->rms_ffn = take(L * d);
        m->w1 = take(L * h * d);
        m->w2 = take(L * d * h);
        m->w3 = take(L * h * d);
        m->rms_final = take(d);
        m->wcls = opt->shared_classifier ? m->emb : take(V * d);

        e = hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking);
        if (e != hipSuccess) { rc = fail_hip(e, "hipStreamCreate"); break; }
        e = hipEventCreateWithFlags(&m->ev_in, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_out, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_poll[0], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_poll[1], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_ptok, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_bstate, hipEventDisableTiming);
        if (e != hipSuccess) { rc = fail_hip(e, "hipEventCreate"); break; }

        const size_t cache = (size_t)m->max_batch * cfg->n_layers * cfg->seq_len * kv;
        if ((rc = dalloc(m, &m->kc, cache)) || (rc = dalloc(m, &m->vc, cache)) || (rc = dalloc(m, &m->x, d)) ||
            (rc = dalloc(m, &m->xb, d)) || (rc = dalloc(m, &m->q, d)) || (rc = dalloc(m, &m->hb, h)) ||
            (rc = dalloc(m, &m->logits, V)) ||
            (rc = dalloc(m, &m->part_acc, (size_t)cfg->n_heads * m->nsplit * m->hs)) ||
            (rc = dalloc(m, &m->part_ml, (size_t)cfg->n_heads * m->nsplit)) ||
            (rc = dalloc(m, &m->rope, (size_t)cfg->seq_len * (m->hs / 2))) ||
            (rc = dalloc(m, &m->state, 1)) ||
            (rc = dalloc(m, &m->tokens, (size_t)cfg->seq_len)) || (rc = dalloc(m, &m->ctl, 1)) ||
            (rc = dalloc(m, &m->forced, (size_t)cfg->seq_len + 1)) ||
            (rc = dalloc(m, &m->coins, (size_t)cfg->seq_len)) || (rc = dalloc(m, &m->ptok, (size_t)cfg->seq_len)))
            break;
        e = hipHostMalloc((void**)&m->h_tokens, sizeof(int32_t) * (size_t)cfg->seq_len, hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipHostMalloc((void**)&m->h_forced, sizeof(int32_t) * ((size_t)cfg->seq_len + 1), hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipHostMalloc((void**)&m->h_coins, sizeof(float) * (size_t)cfg->seq_len, hipHostMallocDefault);
        if (e == hipSuccess) e = hipHostMalloc((void**)&m->h_poll, sizeof(StepState) * 3, hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipHostMalloc((void**)&m->h_ptok, sizeof(int32_t) * (size_t)cfg->seq_len, hipHostMallocDefault);
        if (e != hipSuccess) { rc = fail_hip(e, "hipHostMalloc"); break; }

        if ((rc = (gemv_plan(K_QKV, cfg->dim + 2 * m->kv_dim, cfg->dim, &m->pq) == hipSuccess) ? LD_OK : LD_E_UNSUPPORTED) ||
            (rc = (gemv_plan(K_RESID, cfg->dim, cfg->dim, &m->pwo) == hipSuccess) ? LD_OK : LD_E_UNSUPPORTED) ||
            (rc = (gemv_plan(K_SWIGLU, cfg->hidden_dim, cfg->dim, &m->pffn) == hipSuccess) ? LD_OK : LD_E_UNSUPPORTED) ||
            (rc = (gemv_plan(K_RESID, cfg->dim, cfg->hidden_dim, &m->pw2) == hipSuccess) ? LD_OK : LD_E_UNSUPPORTED) ||
            (rc = (gemv_plan(K_CLS, cfg->vocab_size, cfg->dim, &m->pcls) == hipSuccess) ? LD_OK : LD_E_UNSUPPORTED))
            break;
        rc = dalloc(m, &m->best, (size_t)m->pcls.grid);
        if (rc) break;
        if (!(opt->flags & LD_OPT_NO_FUSE) && qkv_attention_pays(cfg->dim) &&
            qkv_attention_supported(cfg->dim, m->hs, cfg->n_heads, cfg->n_kv_heads)) {
            e = qkv_attention_plan(cfg->dim, m->hs, cfg->n_heads, cfg->n_kv_heads, &m->pqa);
            if (e != hipSuccess) { rc = fail_hip(e, "qkv_attention_plan"); break; }
            if ((rc = dalloc(m, &m->stage, qkv_attention_stage_floats(m->hs, cfg->n_heads, cfg->n_kv_heads))) ||
                (rc = dalloc(m, &m->qkv_arrive, (size_t)cfg->n_kv_heads)))
                break;
            e = hipMemset(m->qkv_arrive, 0, sizeof(unsigned) * (size_t)cfg->n_kv_heads);
            if (e != hipSuccess) { rc = fail_hip(e, "hipMemset"); break; }
            const int keys = LD_FUSE_KEY_BYTES / (8 * m->hs);
            m->fuse_keys = keys < 1 ? 1 : keys < cfg->seq_len ? keys : cfg->seq_len;
        }
        {  // batch buffers (also for max_batch 1, so a batch of one runs)
            const size_t B = m->max_batch;
            if ((rc = dalloc(m, &m->bx, B * d)) || (rc = dalloc(m, &m->bq, B * d)) ||
                (rc = dalloc(m, &m->batt, B * d)) || (rc = dalloc(m, &m->bhb, B * h)) ||
                (rc = dalloc(m, &m->blogits, B * V)) ||
                (rc = dalloc(m, &m->bpart_ml, B * cfg->n_heads * m->nsplit)) ||
                (rc = dalloc(m, &m->bpart_acc, B * cfg->n_heads * m->nsplit * m->hs)) ||
                (rc = dalloc(m, &m->arrive, B * cfg->n_kv_heads)) ||
                (rc = dalloc(m, &m->bstate, B)) || (rc = dalloc(m, &m->btokens, B * cfg->seq_len)))
                break;
            e = hipMemset(m->arrive, 0, sizeof(unsigned) * B * cfg->n_kv_heads);
            if (e != hipSuccess) { rc = fail_hip(e, "hipMemset"); break; }
            // the largest split-K workspace any batch size up to B needs
            const int shapes[5][2] = {{cfg->dim + 2 * m->kv_dim, cfg->dim}, {cfg->dim, cfg->dim},
                                      {2 * cfg->hidden_dim, cfg->dim}, {cfg->dim, cfg->hidden_dim},
                                      {cfg->vocab_size, cfg->dim}};
            size_t ws = 0;
            for (int nb = 1; nb <= m->max_batch; ++nb)
                for (const auto& sh : shapes) {
                    const size_t need = gemm_part_floats(nb, sh[0], sh[1]);
                    if (need > ws) ws = need;
                }
            m->bsplit_floats = ws;
            if ((rc = dalloc(m, &m->bsplit, ws))) break;
            m->bgemv = gemv_plan_batch(K_QKV, cfg->dim + 2 * m->kv_dim, cfg->dim, &m->bpq) == hipSuccess &&
                       gemv_plan_batch(K_RESID, cfg->dim, cfg->dim, &m->bpwo) == hipSuccess &&
                       gemv_plan_batch(K_SWIGLU, cfg->hidden_dim, cfg->dim, &m->bpffn) == hipSuccess &&
                       gemv_plan_batch(K_PLAIN, cfg->vocab_size, cfg->dim, &m->bpcls) == hipSuccess;
            // a hidden width beyond the batch kernel's shapes (the 70B layer's
            // 28672) takes the split-K product for the down projection alone
            m->bgemv_w2 = gemv_plan_batch(K_RESID, cfg->dim, cfg->hidden_dim, &m->bpw2) == hipSuccess;
            // the tiled copies of the weights, for batches of kGemvBatch+1 .. kTiledBatch
            const bool t16 = cfg->dim % 16 == 0 && cfg->hidden_dim % 16 == 0 && m->kv_dim % 16 == 0 &&
                             cfg->vocab_size % 16 == 0 && m->hs % 4 == 0;
            if (m->max_batch > kGemvBatch && t16) {
                const size_t qkv = (d + 2 * kv) * d, ffn = 2 * h * d;
                if ((rc = dalloc(m, &m->t_qkv, L * qkv)) || (rc = dalloc(m, &m->t_wo, L * d * d)) ||
                    (rc = dalloc(m, &m->t_ffn, L * ffn)) || (rc = dalloc(m, &m->t_w2, L * d * h)) ||
                    (rc = dalloc(m, &m->t_cls, V * d)) || (rc = dalloc(m, &m->bxt, (size_t)kTiledBatch * d)) ||
                    (rc = dalloc(m, &m->bhbt, (size_t)kTiledBatch * h)) ||
                    (rc = dalloc(m, &m->batt_t, (size_t)kTiledBatch * d)))
                    break;
                int dev = 0, cus = 0;
                e = hipGetDevice(&dev);
                if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
                if (e != hipSuccess) { rc = fail_hip(e, "device attributes"); break; }
                m->t_part_floats = tiled_part_floats(cus);
                if ((rc = dalloc(m, &m->t_part, m->t_part_floats)) ||
                    (rc = dalloc(m, &m->t_arrive, (size_t)tiled_arrive_count(cus))))
                    break;
                e = hipMemset(m->t_arrive, 0, sizeof(unsigned) * (size_t)tiled_arrive_count(cus));
                if (e != hipSuccess) { rc = fail_hip(e, "hipMemset"); break; }
                for (size_t l = 0; l < L && e == hipSuccess; ++l) {
                    e = tile_weights_launch(K_QKV, m->wq + l * d * d, m->wk + l * kv * d, m->wv + l * kv * d,
                                            cfg->dim, cfg->dim + m->kv_dim, m->rms_att + l * d,
                                            cfg->dim + 2 * m->kv_dim, cfg->dim, m->t_qkv + l * qkv, m->stream);
                    if (e == hipSuccess)
                        e = tile_weights_launch(K_PLAIN, m->wo + l * d * d, nullptr, nullptr, 0, 0, nullptr, cfg->dim,
                                                cfg->dim, m->t_wo + l * d * d, m->stream);
                    if (e == hipSuccess)
                        e = tile_weights_launch(K_SWIGLU, m->w1 + l * h * d, m->w3 + l * h * d, nullptr, 0, 0,
                                                m->rms_ffn + l * d, 2 * cfg->hidden_dim, cfg->dim, m->t_ffn + l * ffn,
                                                m->stream);
                    if (e == hipSuccess)
                        e = tile_weights_launch(K_PLAIN, m->w2 + l * d * h, nullptr, nullptr, 0, 0, nullptr, cfg->dim,
                                                cfg->hidden_dim, m->t_w2 + l * d * h, m->stream);
                }
                if (e == hipSuccess)
                    e = tile_weights_launch(K_PLAIN, m->wcls, nullptr, nullptr, 0, 0, m->rms_final, cfg->vocab_size,
                                            cfg->dim, m->t_cls, m->stream);
                if (e == hipSuccess) e = hipMemsetAsync(m->bxt, 0, sizeof(float) * kTiledBatch * d, m->stream);
                if (e == hipSuccess) e = hipMemsetAsync(m->bhbt, 0, sizeof(float) * kTiledBatch * h, m->stream);
                if (e == hipSuccess) e = hipMemsetAsync(m->batt_t, 0, sizeof(float) * kTiledBatch * d, m->stream);
                if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
                if (e != hipSuccess) { rc = fail_hip(e, "tiled weights"); break; }
                m->tiled = true;
            }
            e = hipHostMalloc((void**)&m->h_bstate, sizeof(StepState) * B, hipHostMallocDefault);
            if (e == hipSuccess)
                e = hipHostMalloc((void**)&m->h_btokens, sizeof(int32_t) * B * cfg->seq_len, hipHostMallocDefault);
            if (e != hipSuccess) { rc = fail_hip(e, "hipHostMalloc"); break; }
        }

        std::vector<float2> rt = rope_table(cfg->seq_len, m->hs, (double)opt->rope_theta);
        e = hipMemcpy(m->rope, rt.data(), rt.size() * sizeof(float2), hipMemcpyHostToDevice);
        if (e != hipSuccess) { rc = fail_hip(e, "hipMemcpy rope"); break; }
        e = hipMemset(m->kc, 0, cache * sizeof(float));
        if (e == hipSuccess) e = hipMemset(m->vc, 0, cache * sizeof(float));
        if (e == hipSuccess) e = hipMemset(m->state, 0, sizeof(StepState));
        if (e == hipSuccess) e = hipMemset(m->tokens, 0, sizeof(int32_t) * (size_t)cfg->seq_len);
        if (e == hipSuccess) e = hipMemset(m->forced, 0, sizeof(int32_t) * ((size_t)cfg->seq_len + 1));
        if (e == hipSuccess) e = hipMemset(m->coins, 0, sizeof(float) * (size_t)cfg->seq_len);
        if (e == hipSuccess) e = hipMemcpy(m->ctl, &kGreedy, sizeof(GenControl), hipMemcpyHostToDevice);
        m->ctl_host = kGreedy;
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) { rc = fail_hip(e, "initialise buffers"); break; }
    } while (0);
    if (rc != LD_OK) {
        release(m);
        return rc;
    }
    *out = m;
    return LD_OK;
}

int ld_reset(ld_model* m) {
    if (!m) return LD_E_NULL;
    int rc = enter(m);
    if (rc) return rc;
    const size_t cache = (size_t)m->max_batch * m->cfg.n_layers * m->cfg.seq_len * m->kv_dim * sizeof(float);
    HIP_TRY(hipMemsetAsync(m->kc, 0, cache, m->stream));
    HIP_TRY(hipMemsetAsync(m->vc, 0, cache, m->stream));
    return leave(m);
}

int ld_forward(ld_model* m, int32_t token, int32_t pos, const float** d_logits_out) {
    if (!m || !d_logits_out) return LD_E_NULL;
    if (token < 0 || token >= m->cfg.vocab_size || pos < 0 || pos >= m->cfg.seq_len) return LD_E_RANGE;
    int rc = enter(m);
    if (rc) return rc;
    if ((rc = set_control(m, kGreedy))) return rc;
    HIP_TRY(set_state_launch(m->state, token, pos, m->stream));
    rc = run_step(m, pos);
    if (rc) return rc;
    *d_logits_out = m->logits;
    return leave(m);
}

int ld_argmax_last(ld_model* m, int32_t* h_token_out) {
    if (!m || !h_token_out) return LD_E_NULL;
    int rc = enter(m);
    if (rc) return rc;
    HIP_TRY(hipMemcpyAsync(m->h_tokens, &m->state->next, sizeof(int32_t), hipMemcpyDeviceToHost, m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    *h_token_out = m->h_tokens[0];
    return leave(m);
}

int ld_generate_greedy(ld_model* m, int32_t token, int32_t pos, int32_t n_steps, int32_t* h_tokens_out) {
    if (!m || (!h_tokens_out && n_steps > 0)) return LD_E_NULL;
    if (token < 0 || token >= m->cfg.vocab_size || pos < 0 || n_steps < 0 ||
        (long long)pos + n_steps > m->cfg.seq_len)
        return LD_E_RANGE;
    if (n_steps == 0) return LD_OK;
    int rc = enter(m);
    if (rc) return rc;
    if ((rc = set_control(m, kGreedy))) return rc;
    if ((rc = check_copy((size_t)pos + n_steps, (size_t)m->cfg.seq_len, "generated tokens"))) return rc;
    HIP_TRY(set_state_launch(m->state, token, pos, m->stream));
    for (int i = 0; i < n_steps; ++i) {
        rc = run_step(m, (long long)pos + i);
        if (rc) return rc;
    }
    HIP_TRY(hipMemcpyAsync(m->h_tokens, m->tokens + pos, sizeof(int32_t) * (size_t)n_steps, hipMemcpyDeviceToHost,
                           m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    std::memcpy(h_tokens_out, m->h_tokens, sizeof(int32_t) * (size_t)n_steps);
    return leave(m);
}

int ld_generate(ld_model* m, const int32_t* h_prompt, int32_t n_prompt, int32_t pos, int32_t n_steps,
                const ld_sampling* sampling, const float* h_coins, int32_t* h_tokens_out, int32_t* n_out) {
    if (!m || !h_prompt || !sampling || !n_out || (!h_tokens_out && n_steps > 0)) return LD_E_NULL;
    *n_out = 0;
    const ld_config& c = m->cfg;
    if (n_prompt < 1 || pos < 0 || n_steps < 0 || (long long)pos + n_steps > c.seq_len) return LD_E_RANGE;
    for (int i = 0; i < n_prompt; ++i)
        if (h_prompt[i] < 0 || h_prompt[i] >= c.vocab_size) return LD_E_RANGE;
    const float T = sampling->temperature;
    if (std::isnan(T) || std::isinf(T) || std::isnan(sampling->topp)) return LD_E_RANGE;
    if (sampling->stop_token < -1 || sampling->stop_token >= c.vocab_size) return LD_E_RANGE;
    const int n_forced = n_prompt - 1 < n_steps ? n_prompt - 1 : n_steps;  // steps whose next token is forced
    const bool draws = T > 0.f && n_forced < n_steps;
    if (draws) {
        if (c.vocab_size > kMaxSampleVocab) return LD_E_UNSUPPORTED;
        if (!h_coins) return LD_E_NULL;
        for (int i = n_forced; i < n_steps; ++i)
            if (!(h_coins[i] >= 0.f && h_coins[i] < 1.f)) return LD_E_RANGE;
    }
    if (n_steps == 0) return LD_OK;
    int rc = enter(m);
    if (rc) return rc;

    // the step at position p takes forced[p + 1] while p + 1 < force_end
    const GenControl ctl = {T > 0.f ? T : 0.f, sampling->topp, sampling->stop_token, pos + 1 + n_forced};
    if ((rc = set_control(m, ctl))) return rc;
    // staging: forced tokens at positions pos+1 .. pos+n_forced (seq_len + 1 slots), coins and tokens at
    // positions pos .. pos+n_steps-1 (seq_len slots)
    if ((rc = check_copy((size_t)pos + 1 + n_forced, (size_t)c.seq_len + 1, "forced tokens")) ||
        (rc = check_copy((size_t)pos + n_steps, (size_t)c.seq_len, "coins and tokens")))
        return rc;
    if (n_forced > 0) {
        std::memcpy(m->h_forced, h_prompt + 1, sizeof(int32_t) * (size_t)n_forced);
        HIP_TRY(hipMemcpyAsync(m->forced + pos + 1, m->h_forced, sizeof(int32_t) * (size_t)n_forced,
                               hipMemcpyHostToDevice, m->stream));
    }
    if (draws) {
        const int nd = n_steps - n_forced;
        std::memcpy(m->h_coins, h_coins + n_forced, sizeof(float) * (size_t)nd);
        HIP_TRY(hipMemcpyAsync(m->coins + pos + n_forced, m->h_coins, sizeof(float) * (size_t)nd,
                               hipMemcpyHostToDevice, m->stream));
    }
    HIP_TRY(set_state_launch(m->state, h_prompt[0], pos, m->stream));

    // Steps go out in chunks.  With a stop token each chunk is followed by a
    // snapshot of the step state; the host reads the previous chunk's
    // snapshot while the current chunk runs, and stops queueing once a step
    // has chosen the stop token (steps queued past it change nothing).
    constexpr int kChunk = 16;
    const bool polls = sampling->stop_token >= 0;
    int issued = 0;
    for (int chunk = 0; issued < n_steps; ++chunk) {
        const int k = n_steps - issued < kChunk ? n_steps - issued : kChunk;
        for (int i = 0; i < k; ++i)
            if ((rc = run_step(m, (long long)pos + issued + i))) return rc;
        issued += k;
        if (!polls || issued >= n_steps) continue;
        const int slot = chunk & 1;
        HIP_TRY(hipMemcpyAsync(&m->h_poll[slot], m->state, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
        HIP_TRY(hipEventRecord(m->ev_poll[slot], m->stream));
        if (chunk > 0) {
            HIP_TRY(hipEventSynchronize(m->ev_poll[slot ^ 1]));
            if (m->h_poll[slot ^ 1].stopped) break;
        }
    }
    HIP_TRY(hipMemcpyAsync(&m->h_poll[2], m->state, sizeof(StepState), hipMemcpyDeviceToHost, m->stream));
    HIP_TRY(hipMemcpyAsync(m->h_tokens, m->tokens + pos, sizeof(int32_t) * (size_t)n_steps, hipMemcpyDeviceToHost,
                           m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    const int ran = m->h_poll[2].pos - pos;
    std::memcpy(h_tokens_out, m->h_tokens, sizeof(int32_t) * (size_t)ran);
    *n_out = ran;
    return leave(m);
}

int ld_prefill(ld_model* m, const int32_t* h_tokens, int32_t n_tokens, int32_t pos, const float** d_logits_out) {
    return ld_prefill_seq(m, 0, h_tokens, n_tokens, pos, d_logits_out);
}

int ld_prefill_seq(ld_model* m, int32_t seq, const int32_t* h_tokens, int32_t n_tokens, int32_t pos,
                   const float** d_logits_out) {
    if (!m || !h_tokens || !d_logits_out) return LD_E_NULL;
    const ld_config& c = m->cfg;
    if (seq < 0 || seq >= m->max_batch) return LD_E_RANGE;
    if (n_tokens < 1 || pos < 0 || (long long)pos + n_tokens > c.seq_len) return LD_E_RANGE;
    for (int i = 0; i < n_tokens; ++i)
        if (h_tokens[i] < 0 || h_tokens[i] >= c.vocab_size) return LD_E_RANGE;
    if (!attn_prefill_supported(m->hs)) return LD_E_UNSUPPORTED;
    int rc = enter(m);
    if (rc) return rc;
    if ((rc = set_control(m, kGreedy))) return rc;
    const int chunk = n_tokens < kPrefillChunk ? n_tokens : kPrefillChunk;
    if ((rc = prefill_workspace(m, chunk))) return rc;
    if ((rc = check_copy((size_t)pos + n_tokens, (size_t)c.seq_len, "prompt tokens"))) return rc;
    // the staging buffer is free once the previous prefill's copy has run
    if (m->ptok_pending) HIP_TRY(hipEventSynchronize(m->ev_ptok));
    std::memcpy(m->h_ptok, h_tokens, sizeof(int32_t) * (size_t)n_tokens);
    HIP_TRY(hipMemcpyAsync(m->ptok + pos, m->h_ptok, sizeof(int32_t) * (size_t)n_tokens, hipMemcpyHostToDevice,
                           m->stream));
    HIP_TRY(hipEventRecord(m->ev_ptok, m->stream));
    m->ptok_pending = true;
    int last = 0;
    for (int c0 = 0; c0 < n_tokens; c0 += chunk) {
        const int T = n_tokens - c0 < chunk ? n_tokens - c0 : chunk;
        if ((rc = prefill_chunk(m, seq, pos + c0, T))) return rc;
        last = T - 1;
    }
    // classifier and next token for the last prompt token, as a decode step ends
    HIP_TRY(set_state_launch(m->state, h_tokens[n_tokens - 1], pos + n_tokens - 1, m->stream));
    GemvParams p = base_params(m);
    p.x = m->pf_x + (size_t)last * c.dim;
    p.gain = m->rms_final;
    p.n = c.dim;
    p.rows = c.vocab_size;
    p.w0 = m->wcls;
    p.out = m->logits;
    p.best = m->best;
    HIP_TRY(gemv_launch(m->pcls, p, m->stream));
    NextTokenParams nt{};
    nt.best = m->best;
    nt.nblocks = m->pcls.grid;
    nt.logits = m->logits;
    nt.n = c.vocab_size;
    nt.ctl = m->ctl;
    nt.forced = m->forced;
    nt.coins = m->coins;
    nt.state = m->state;
    nt.tokens_out = m->tokens;
    HIP_TRY(next_token_launch(nt, m->stream));
    *d_logits_out = m->logits;
    return leave(m);
}

int ld_forward_batch(ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int32_t n,
                     const float** d_logits_out) {
    if (!m || !h_tokens || !h_pos || !d_logits_out) return LD_E_NULL;
    int rc = check_batch(m, h_tokens, h_pos, n, 0);
    if (rc) return rc;
    if ((rc = enter(m))) return rc;
    if ((rc = set_batch_states(m, h_tokens, h_pos, n))) return rc;
    if ((rc = run_batch_step(m, n))) return rc;
    *d_logits_out = m->blogits;
    return leave(m);
}

int ld_generate_greedy_batch(ld_model* m, const int32_t* h_tokens, const int32_t* h_pos, int32_t n,
                             int32_t n_steps, int32_t* h_tokens_out) {
    if (!m || !h_tokens || !h_pos || (!h_tokens_out && n_steps > 0)) return LD_E_NULL;
    int rc = check_batch(m, h_tokens, h_pos, n, n_steps);
    if (rc) return rc;
    if (n_steps == 0) return LD_OK;
    if ((rc = enter(m))) return rc;
    if ((rc = set_batch_states(m, h_tokens, h_pos, n))) return rc;
    for (int i = 0; i < n_steps; ++i)
        if ((rc = run_batch_step(m, n))) return rc;
    const int S = m->cfg.seq_len;
    if ((rc = check_copy((size_t)n * S, (size_t)m->max_batch * S, "batch tokens"))) return rc;
    HIP_TRY(hipMemcpyAsync(m->h_btokens, m->btokens, sizeof(int32_t) * (size_t)n * S, hipMemcpyDeviceToHost,
                           m->stream));
    HIP_TRY(hipStreamSynchronize(m->stream));
    for (int b = 0; b < n; ++b)
        std::memcpy(h_tokens_out + (size_t)b * n_steps, m->h_btokens + (size_t)b * S + h_pos[b],
                    sizeof(int32_t) * (size_t)n_steps);
    return leave(m);
}

int ld_kv_cache(ld_model* m, float** d_key_out, float** d_value_out, size_t* floats_out) {
    if (!m || !d_key_out || !d_value_out || !floats_out) return LD_E_NULL;
    *d_key_out = m->kc;
    *d_value_out = m->vc;
    *floats_out = (size_t)m->max_batch * m->cfg.n_layers * m->cfg.seq_len * m->kv_dim;
    return LD_OK;
}

void ld_destroy(ld_model* m) { release(m); }

int ld_profile_steps(ld_model* m, int32_t token, int32_t pos, int32_t n_steps, ld_kernel_stat* stats,
                     int32_t max_stats, int32_t* n_stats_out) {
    if (!m || !stats || !n_stats_out) return LD_E_NULL;
    if (token < 0 || token >= m->cfg.vocab_size || pos < 0 || n_steps < 0 ||
        (long long)pos + n_steps > m->cfg.seq_len)
        return LD_E_RANGE;
    int rc = enter(m);
    if (rc) return rc;
    const int launches = 5 * m->cfg.n_layers + 1;
    Timer t;
    t.ev.resize(2 * (size_t)launches, nullptr);
    t.kind.resize(launches, 0);
    for (auto& e : t.ev) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            for (auto& x : t.ev)
                if (x) (void)hipEventDestroy(x);
            return fail_hip(err, "hipEventCreate");
        }
    }
    double total[KNUM] = {0};
    int count[KNUM] = {0};
    if ((rc = set_control(m, kGreedy))) return rc;
    HIP_TRY(set_state_launch(m->state, token, pos, m->stream));
    for (int i = 0; i < n_steps && rc == LD_OK; ++i) {
        t.used = 0;
        rc = launch_step(m, &t, fused_at(m, (long long)pos + i));
        if (rc) break;
        hipError_t err = hipStreamSynchronize(m->stream);
        if (err != hipSuccess) {
            rc = fail_hip(err, "hipStreamSynchronize");
            break;
        }
        for (int k = 0; k < (int)(t.used / 2); ++k) {
            float ms = 0.f;
            err = hipEventElapsedTime(&ms, t.ev[2 * k], t.ev[2 * k + 1]);
            if (err != hipSuccess) {
                rc = fail_hip(err, "hipEventElapsedTime");
                break;
            }
            total[t.kind[k]] += ms;
            count[t.kind[k]] += 1;
        }
    }
    for (auto& e : t.ev) (void)hipEventDestroy(e);
    if (rc) return rc;
    int n = 0;
    for (int k = 0; k < KNUM && n < max_stats; ++k) {
        std::memset(stats[n].name, 0, sizeof(stats[n].name));
        std::strncpy(stats[n].name, kKindName[k], sizeof(stats[n].name) - 1);
        stats[n].launches = count[k];
        stats[n].total_ms = total[k];
        ++n;
    }
    *n_stats_out = n;
    return leave(m);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Single-kernel entry points (synchronous, own temporaries).

namespace {

struct Temps {
    std::vector<void*> p;
    ~Temps() {
        for (void* q : p) (void)hipFree(q);
    }
    template <class T>
    hipError_t get(T** out, size_t count) {
        void* q = nullptr;
        hipError_t e = hipMalloc(&q, (count ? count : 1) * sizeof(T));
        if (e == hipSuccess) {
            p.push_back(q);
            *out = static_cast<T*>(q);
        }
        return e;
    }
};

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// per-block bests of v, then the next-token kernel at position 0 with control c
int op_next_token(const float* d_v, int n, const GenControl& c, float coin, int32_t* h_out, hipStream_t s) {
    const int nb = argmax_blocks(n);
    Temps tmp;
    float2* best = nullptr;
    StepState* st = nullptr;
    GenControl* ctl = nullptr;
    float* coins = nullptr;
    HIP_TRY(tmp.get(&best, (size_t)nb));
    HIP_TRY(tmp.get(&st, 1));
    HIP_TRY(tmp.get(&ctl, 1));
    HIP_TRY(tmp.get(&coins, 1));
    const StepState st0 = {0, 0, -1, 0};
    HIP_TRY(hipMemcpy(st, &st0, sizeof(st0), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(ctl, &c, sizeof(c), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(coins, &coin, sizeof(coin), hipMemcpyHostToDevice));
    HIP_TRY(argmax_partial_launch(d_v, n, best, nb, s));
    NextTokenParams p{};
    p.best = best;
    p.nblocks = nb;
    p.logits = d_v;
    p.n = n;
    p.ctl = ctl;
    p.forced = nullptr;
    p.coins = coins;
    p.state = st;
    p.tokens_out = nullptr;
    HIP_TRY(next_token_launch(p, s));
    StepState out{};
    HIP_TRY(hipMemcpyAsync(&out, st, sizeof(out), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    *h_out = out.next;
    return LD_OK;
}

int op_attention_check(const float* d_q, const float* d_kc, const float* d_vc, int n_heads, int n_kv_heads,
                       int head_size, int pos, const float* d_out) {
    if (!d_q || !d_kc || !d_vc || !d_out) return LD_E_NULL;
    if (n_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > n_heads || head_size <= 0 || head_size % 2)
        return LD_E_CONFIG;
    if (!supported_head_size(head_size)) return LD_E_UNSUPPORTED;
    if ((n_heads + n_kv_heads - 1) / n_kv_heads > kMaxGroup) return LD_E_UNSUPPORTED;
    if (pos < 0) return LD_E_RANGE;
    if (!aligned16(d_q) || !aligned16(d_kc) || !aligned16(d_vc)) return LD_E_ALIGN;
    return LD_OK;
}

// One attention launch at pos over caches of pos + 1 rows, with the split
// partials, arrival counts and state in the given device buffers.  Queued on
// s; does not wait for it.
int op_attention_launch(const float* d_q, const float* d_kc, const float* d_vc, int n_heads, int n_kv_heads,
                        int head_size, int pos, float* d_out, int nsplit, float2* ml, float* acc, unsigned* arrive,
                        StepState* st, hipStream_t s) {
    HIP_TRY(attn_op_init_launch(st, pos, arrive, n_kv_heads, s));
    AttnParams a{};
    a.q = d_q;
    a.kc = d_kc;
    a.vc = d_vc;
    a.out = d_out;
    a.part_ml = ml;
    a.part_acc = acc;
    a.arrive = arrive;
    a.state = st;
    a.n_heads = n_heads;
    a.n_kv_heads = n_kv_heads;
    a.kv_dim = n_kv_heads * head_size;
    a.nsplit = nsplit;
    a.waves = attn_waves(head_size, pos + 1, n_heads, n_kv_heads);
    HIP_TRY(attn_launch(head_size, a, s));
    return LD_OK;
}

// Where ld_op_attention_noalloc keeps its temporaries within the scratch
// array: the state, the arrival counts, the (m, l) pairs and the value sums of
// the split partials, each 256-byte aligned.
struct ScratchPlan {
    size_t state = 0, arrive = 0, ml = 0, acc = 0, bytes = 0;
};

bool plan_attention_scratch(int n_heads, int n_kv_heads, int head_size, int nsplit, ScratchPlan* p) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t pairs = (size_t)n_heads * nsplit;
    p->state = 0;
    p->arrive = up(sizeof(StepState));
    p->ml = p->arrive + up(sizeof(unsigned) * (size_t)n_kv_heads);
    p->acc = p->ml + up(sizeof(float2) * pairs);
    p->bytes = p->acc + sizeof(float) * pairs * (size_t)head_size;
    return p->bytes <= (size_t)LD_NOALLOC_SCRATCH_BYTES;
}

int op_shape_ok(int rows, int n) {
    if (rows <= 0 || n <= 0 || (n % 4)) return LD_E_CONFIG;
    if (n > kMaxN) return LD_E_UNSUPPORTED;
    return LD_OK;
}

}  // namespace

extern "C" {

int ld_op_rmsnorm_gemv(const float* d_x, const float* d_g, float eps, const float* d_w, int32_t rows, int32_t n,
                       float* d_out, void* hip_stream) {
    if (!d_x || !d_w || !d_out) return LD_E_NULL;
    if (int rc = op_shape_ok(rows, n)) return rc;
    if (!aligned16(d_x) || !aligned16(d_w) || (d_g && !aligned16(d_g))) return LD_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    GemvPlan pl;
    HIP_TRY(gemv_plan(K_PLAIN, rows, n, &pl));
    GemvParams p{};
    p.x = d_x;
    p.gain = d_g;
    p.eps = eps;
    p.n = n;
    p.rows = rows;
    p.w0 = d_w;
    p.out = d_out;
    HIP_TRY(gemv_launch(pl, p, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_gemv_residual(const float* d_in, const float* d_w, int32_t rows, int32_t n, float* d_x, void* hip_stream) {
    if (!d_in || !d_w || !d_x) return LD_E_NULL;
    if (int rc = op_shape_ok(rows, n)) return rc;
    if (!aligned16(d_in) || !aligned16(d_w)) return LD_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    GemvPlan pl;
    HIP_TRY(gemv_plan(K_RESID, rows, n, &pl));
    GemvParams p{};
    p.x = d_in;
    p.x_resid = d_x;
    p.n = n;
    p.rows = rows;
    p.w0 = d_w;
    HIP_TRY(gemv_launch(pl, p, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_swiglu(const float* d_x, const float* d_g, float eps, const float* d_w1, const float* d_w3, int32_t hidden,
                 int32_t n, float* d_hb, void* hip_stream) {
    if (!d_x || !d_w1 || !d_w3 || !d_hb) return LD_E_NULL;
    if (int rc = op_shape_ok(hidden, n)) return rc;
    if (!aligned16(d_x) || !aligned16(d_w1) || !aligned16(d_w3) || (d_g && !aligned16(d_g))) return LD_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    GemvPlan pl;
    HIP_TRY(gemv_plan(K_SWIGLU, hidden, n, &pl));
    GemvParams p{};
    p.x = d_x;
    p.gain = d_g;
    p.eps = eps;
    p.n = n;
    p.rows = hidden;
    p.w0 = d_w1;
    p.w1 = d_w3;
    p.out = d_hb;
    HIP_TRY(gemv_launch(pl, p, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_qkv_rope(const float* d_x, const float* d_g, float eps, const float* d_wq, const float* d_wk,
                   const float* d_wv, int32_t dim, int32_t n_heads, int32_t n_kv_heads, int32_t pos, float theta,
                   float* d_q, float* d_k, float* d_v, void* hip_stream) {
    if (!d_x || !d_wq || !d_wk || !d_wv || !d_q || !d_k || !d_v) return LD_E_NULL;
    if (dim <= 0 || n_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > n_heads || dim % n_heads ||
        ((long long)dim * n_kv_heads) % n_heads || ((dim / n_heads) % 2) || !(theta > 0.f))
        return LD_E_CONFIG;
    const int hs = dim / n_heads, kv = (int)((long long)dim * n_kv_heads / n_heads);
    if ((dim % 4) || (kv % 4)) return LD_E_CONFIG;
    if (pos < 0) return LD_E_RANGE;
    if (int rc = op_shape_ok(dim, dim)) return rc;
    if (!aligned16(d_x) || !aligned16(d_wq) || !aligned16(d_wk) || !aligned16(d_wv) || (d_g && !aligned16(d_g)))
        return LD_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    Temps tmp;
    float2* rope = nullptr;
    StepState* st = nullptr;
    HIP_TRY(tmp.get(&rope, (size_t)(pos + 1) * (hs / 2)));
    HIP_TRY(tmp.get(&st, 1));
    std::vector<float2> rt = rope_table(pos + 1, hs, (double)theta);
    HIP_TRY(hipMemcpy(rope, rt.data(), rt.size() * sizeof(float2), hipMemcpyHostToDevice));
    StepState hs_state{0, pos, -1, 0};
    HIP_TRY(hipMemcpy(st, &hs_state, sizeof(hs_state), hipMemcpyHostToDevice));
    GemvPlan pl;
    HIP_TRY(gemv_plan(K_QKV, dim + 2 * kv, dim, &pl));
    GemvParams p{};
    p.x = d_x;
    p.gain = d_g;
    p.eps = eps;
    p.n = dim;
    p.rows = dim + 2 * kv;
    p.w0 = d_wq;
    p.w1 = d_wk;
    p.w2 = d_wv;
    p.seg1 = dim;
    p.seg2 = dim + kv;
    p.out = d_q;
    p.kc = d_k;
    p.vc = d_v;
    p.kv_stride = 0;
    p.head_size = hs;
    p.rope = rope;
    p.state = st;
    HIP_TRY(gemv_launch(pl, p, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_qkv_attention(const float* d_x, const float* d_g, float eps, const float* d_wq, const float* d_wk,
                        const float* d_wv, int32_t dim, int32_t n_heads, int32_t n_kv_heads, int32_t pos, float theta,
                        float* d_kc, float* d_vc, float* d_out, void* hip_stream) {
    if (!d_x || !d_wq || !d_wk || !d_wv || !d_kc || !d_vc || !d_out) return LD_E_NULL;
    if (dim <= 0 || n_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > n_heads || dim % n_heads ||
        ((long long)dim * n_kv_heads) % n_heads || ((dim / n_heads) % 2) || !(theta > 0.f))
        return LD_E_CONFIG;
    const int hs = dim / n_heads, kv = (int)((long long)dim * n_kv_heads / n_heads);
    if ((dim % 4) || (kv % 4)) return LD_E_CONFIG;
    if (pos < 0) return LD_E_RANGE;
    if (!qkv_attention_supported(dim, hs, n_heads, n_kv_heads)) return LD_E_UNSUPPORTED;
    if (!aligned16(d_x) || !aligned16(d_wq) || !aligned16(d_wk) || !aligned16(d_wv) || !aligned16(d_kc) ||
        !aligned16(d_vc) || !aligned16(d_out) || (d_g && !aligned16(d_g)))
        return LD_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    Temps tmp;
    float2* rope = nullptr;
    StepState* st = nullptr;
    float* stage = nullptr;
    unsigned* arrive = nullptr;
    HIP_TRY(tmp.get(&rope, (size_t)(pos + 1) * (hs / 2)));
    HIP_TRY(tmp.get(&st, 1));
    HIP_TRY(tmp.get(&stage, qkv_attention_stage_floats(hs, n_heads, n_kv_heads)));
    HIP_TRY(tmp.get(&arrive, (size_t)n_kv_heads));
    std::vector<float2> rt = rope_table(pos + 1, hs, (double)theta);
    HIP_TRY(hipMemcpy(rope, rt.data(), rt.size() * sizeof(float2), hipMemcpyHostToDevice));
    StepState hs_state{0, pos, -1, 0};
    HIP_TRY(hipMemcpy(st, &hs_state, sizeof(hs_state), hipMemcpyHostToDevice));
    HIP_TRY(hipMemset(arrive, 0, sizeof(unsigned) * (size_t)n_kv_heads));
    GemvPlan pl;
    HIP_TRY(qkv_attention_plan(dim, hs, n_heads, n_kv_heads, &pl));
    GemvParams p{};
    p.x = d_x;
    p.gain = d_g;
    p.eps = eps;
    p.n = dim;
    p.rows = dim + 2 * kv;
    p.w0 = d_wq;
    p.w1 = d_wk;
    p.w2 = d_wv;
    p.seg1 = dim;
    p.seg2 = dim + kv;
    p.kc = d_kc;
    p.vc = d_vc;
    p.kv_stride = kv;
    p.head_size = hs;
    p.rope = rope;
    p.state = st;
    p.stage = stage;
    p.stage_sh = qkv_attention_stage_stride(hs);
    p.arrive = arrive;
    p.att_out = d_out;
    p.n_heads = n_heads;
    p.n_kv_heads = n_kv_heads;
    HIP_TRY(qkv_attention_launch(pl, p, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_attention(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads, int32_t n_kv_heads,
                    int32_t head_size, int32_t pos, float* d_out, void* hip_stream) {
    if (int rc = op_attention_check(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out)) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int nsplit = attn_splits(head_size, pos + 1, n_heads, n_kv_heads);
    Temps tmp;
    float2* ml = nullptr;
    float* acc = nullptr;
    StepState* st = nullptr;
    unsigned* arrive = nullptr;
    HIP_TRY(tmp.get(&ml, (size_t)n_heads * nsplit));
    HIP_TRY(tmp.get(&acc, (size_t)n_heads * nsplit * head_size));
    HIP_TRY(tmp.get(&arrive, (size_t)n_kv_heads));
    HIP_TRY(tmp.get(&st, 1));
    if (int rc = op_attention_launch(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out, nsplit, ml, acc,
                                     arrive, st, s))
        return rc;
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_attention_noalloc(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_size, int32_t pos, float* d_out, void* hip_stream) {
    if (int rc = op_attention_check(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out)) return rc;
    const int nsplit = attn_splits(head_size, pos + 1, n_heads, n_kv_heads);
    ScratchPlan plan;
    if (!plan_attention_scratch(n_heads, n_kv_heads, head_size, nsplit, &plan)) {
        std::snprintf(g_detail, sizeof(g_detail),
                      "ld_op_attention_noalloc: %zu bytes of scratch needed, the limit is %zu", plan.bytes,
                      (size_t)LD_NOALLOC_SCRATCH_BYTES);
        return LD_E_SIZE;
    }
    unsigned char* base = nullptr;
    if (int rc = scratch_for_current_device(&base)) return rc;
    return op_attention_launch(d_q, d_kc, d_vc, n_heads, n_kv_heads, head_size, pos, d_out, nsplit,
                               reinterpret_cast<float2*>(base + plan.ml), reinterpret_cast<float*>(base + plan.acc),
                               reinterpret_cast<unsigned*>(base + plan.arrive),
                               reinterpret_cast<StepState*>(base + plan.state), static_cast<hipStream_t>(hip_stream));
}

int ld_op_gemm(const float* d_a, const float* d_w, int32_t m, int32_t n, int32_t k, float* d_out, void* hip_stream) {
    if (!d_a || !d_w || !d_out) return LD_E_NULL;
    if (m <= 0 || n <= 0 || k <= 0) return LD_E_RANGE;
    if (k % 4) return LD_E_CONFIG;
    if (!aligned16(d_a) || !aligned16(d_w)) return LD_E_ALIGN;
    GemmParams g{};
    g.a = d_a;
    g.lda = k;
    g.m = m;
    g.n = n;
    g.k = k;
    g.w0 = d_w;
    g.out = d_out;
    g.ldo = n;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    Temps tmp;
    g.part_floats = gemm_part_floats(m, n, k);
    if (g.part_floats) HIP_TRY(tmp.get(&g.part, g.part_floats));  // split K, as a decode batch runs it
    HIP_TRY(gemm_launch(G_PLAIN, g, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_attention_prefill(const float* d_q, const float* d_kc, const float* d_vc, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_size, int32_t pos, int32_t n_tokens, float* d_out,
                            void* hip_stream) {
    if (!d_q || !d_kc || !d_vc || !d_out) return LD_E_NULL;
    if (n_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > n_heads || head_size <= 0 || head_size % 2)
        return LD_E_CONFIG;
    if (!attn_prefill_supported(head_size)) return LD_E_UNSUPPORTED;
    if (pos < 0 || n_tokens < 1) return LD_E_RANGE;
    if (!aligned16(d_q) || !aligned16(d_kc) || !aligned16(d_vc)) return LD_E_ALIGN;
    AttnPrefillParams a{};
    a.q = d_q;
    a.ldq = n_heads * head_size;
    a.kc = d_kc;
    a.vc = d_vc;
    a.kv_stride = n_kv_heads * head_size;
    a.out = d_out;
    a.ldo = n_heads * head_size;
    a.t = n_tokens;
    a.pos0 = pos;
    a.n_heads = n_heads;
    a.n_kv_heads = n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    HIP_TRY(attn_prefill_launch(head_size, a, s));
    HIP_TRY(hipStreamSynchronize(s));
    return LD_OK;
}

int ld_op_argmax(const float* d_v, int32_t n, int32_t* h_index_out, void* hip_stream) {
    if (!d_v || !h_index_out) return LD_E_NULL;
    if (n <= 0) return LD_E_RANGE;
    return op_next_token(d_v, n, kGreedy, 0.f, h_index_out, static_cast<hipStream_t>(hip_stream));
}

int ld_op_sample(const float* d_logits, int32_t n, float temperature, float topp, float coin,
                 int32_t* h_token_out, void* hip_stream) {
    if (!d_logits || !h_token_out) return LD_E_NULL;
    if (n <= 0 || std::isnan(temperature) || std::isinf(temperature) || std::isnan(topp)) return LD_E_RANGE;
    if (temperature > 0.f) {
        if (!(coin >= 0.f && coin < 1.f)) return LD_E_RANGE;
        if (n > kMaxSampleVocab) return LD_E_UNSUPPORTED;
    }
    const GenControl c = {temperature > 0.f ? temperature : 0.f, topp, -1, 0};
    return op_next_token(d_logits, n, c, coin, h_token_out, static_cast<hipStream_t>(hip_stream));
}

int ld_op_stream_read(const void* d_src, size_t bytes, float* d_sums, void* hip_stream) {
    static_assert(LD_STREAM_READ_BLOCKS == kStreamReadBlocks, "stream-read block count");
    if (!d_src || !d_sums) return LD_E_NULL;
    if (bytes == 0 || bytes % 16) return LD_E_SIZE;
    if (!aligned16(d_src)) return LD_E_ALIGN;
    HIP_TRY(stream_read_launch(d_src, bytes, d_sums, static_cast<hipStream_t>(hip_stream)));
    return LD_OK;
}

}  // extern "C"
