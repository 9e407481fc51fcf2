// ld_kernels.hip -- gfx950 (CDNA4) kernels of the single-token Llama-2 decode
// step, fp32, batch 1.
//
// The step is the forward() walkthrough of the "run.c 逐行解讀" page (§4):
// RMSNorm, q/k/v matmuls, RoPE, KV-cache write, grouped-query attention,
// output matmul + residual, FFN RMSNorm, SwiGLU, down matmul + residual, final
// RMSNorm, classifier, and the choice of the next token: the greedy argmax of
// the "run.c" page, or the temperature / top-p draw and prompt forcing of the
// "run.c 逐行解讀" page (§6, §7).
//
// At batch 1 every weight is used once per token for one multiply-add, so the
// step is bound by HBM bandwidth (0.5 flop per byte).  The matrix-vector
// kernels therefore stream each weight row once with 128-bit loads and keep
// the input vector in registers; there is no MFMA here because nothing is a
// dense contraction.
#include "ld_internal.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

namespace ld {
namespace {

// ---------------------------------------------------------------------------
// Wave64 reductions with DPP.  Each step adds a permuted copy of the
// register: neighbours in a quad, the quads of a half row, the halves of a row
// (16 lanes), then row 0 into row 1 and row 2 into row 3 (row_bcast:15), then
// rows 0-1 into rows 2-3 (row_bcast:31).  Lane 63 ends with the total, which
// is read back as a wave-uniform value.  Called with all 64 lanes active.

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float old, float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

constexpr int kQuadSwap1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kQuadSwap1>(0.f, v);
    v += dpp<kQuadSwap2>(0.f, v);
    v += dpp<kRowHalfMirror>(0.f, v);
    v += dpp<kRowMirror>(0.f, v);
    v += dpp<kRowBcast15, 0xa>(0.f, v);
    v += dpp<kRowBcast31, 0xc>(0.f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kQuadSwap1>(-INFINITY, v));
    v = fmaxf(v, dpp<kQuadSwap2>(-INFINITY, v));
    v = fmaxf(v, dpp<kRowHalfMirror>(-INFINITY, v));
    v = fmaxf(v, dpp<kRowMirror>(-INFINITY, v));
    v = fmaxf(v, dpp<kRowBcast15, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp<kRowBcast31, 0xc>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
    return acc;
}

// Greedy order of the "run.c" argmax: larger value first, and among equal
// values the lower index (its strict '>' scan keeps the first maximum).
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(i, off);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

// Block-wide best over (v, i); the result is valid in every thread.
template <int NT>
__device__ void block_best(float& v, int& i) {
    constexpr int NW = NT / 64;
    __shared__ float sv[NW];
    __shared__ int si[NW];
    wave_best(v, i);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = v;
        si[wave] = i;
    }
    __syncthreads();
    v = sv[0];
    i = si[0];
    for (int w = 1; w < NW; ++w)
        if (better(sv[w], si[w], v, i)) {
            v = sv[w];
            i = si[w];
        }
}

// The greedy choice in two launches: every block writes its best (value,
// index) pair, then one block reduces the pairs and writes the next token.
// Cross-block hand-off at a kernel boundary costs far less on this chip than a
// device-scope fence inside a kernel (which writes back and invalidates L2).
template <int NT>
__device__ void publish_best(float bv, int bi, float2* best) {
    block_best<NT>(bv, bi);
    if (threadIdx.x == 0) best[blockIdx.x] = make_float2(bv, __int_as_float(bi));
}

constexpr int kArgmaxThreads = 256;

// ---------------------------------------------------------------------------
// The next token ("run.c 逐行解讀" §6 sample() and §7 generate()).
//
// One block of NT threads.  A forced prompt token is taken as is.  Otherwise
// the per-block bests of the logits give the greedy choice and the maximum
// logit; at a positive temperature thread t then holds the softmax numerators
// e_i = exp((l_i - max) / T) of tokens i = t + k NT (k < E) in registers, and
// the draw is the cumulative walk of the "run.c" sample(): the first token,
// in walk order, whose cumulative mass exceeds coin * (mass of the
// candidates).  A thread sums its own numerators in fp32 (at most E terms),
// the block sums those partials in double, every sum in one fixed order, so
// every thread holds the same bits and takes the same branch.
// One CU does all of this, so the cost is counted in passes over the E
// registers of every thread (one block sum each); the searches below keep
// the passes few.
//  * Without top-p the walk runs in index order.  Token i = t + k NT lies in
//    "row" k: a bisection over rows on the threads' running sums finds the
//    row whose prefix mass brackets coin * S (log2 E passes of one select and
//    one block sum), one scan over the row's threads the token.
//  * With top-p the walk runs in descending probability, ties to the lower
//    index.  Searches over fp32 bit patterns (the integer order of positive
//    floats is their numeric order) find
//    (a) v_k, the value of the last candidate: the largest v whose mass
//        G(v) = sum of e_i >= v reaches topp * S.  The candidates are every
//        e_i > v_k and the first j tokens (index order) equal to v_k, j the
//        fewest that bring the candidate mass M to topp * S;
//    (b) u, the value of the drawn token: the largest candidate value with
//        G(u) > coin * M.  Among the tokens equal to u the draw takes the
//        (q+1)-th in index order, q = floor((coin * M - G(> u)) / u).
//    Each search bisects a bracket [lo, hi) of bit patterns; once at most
//    kCap values lie inside it, they are compacted into LDS and one wave
//    finishes the bisection over that list alone, with no block barrier.

constexpr int kCap = 512;

template <int NW>
struct SampleShared {
    double red[2][NW];
    int ired[2][NW];
    int imin[2][NW];
    float cv[kCap];
    double bd[2];
    int bi[4];
};

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xf, false);
    return __hiloint2double(hi, lo);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// the wave's total, the same bits in every lane (the wave_sum pattern in double)
__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_d<kQuadSwap1>(v);
    v += dpp_d<kQuadSwap2>(v);
    v += dpp_d<kRowHalfMirror>(v);
    v += dpp_d<kRowMirror>(v);
    v += dpp_d<kRowBcast15, 0xa>(v);
    v += dpp_d<kRowBcast31, 0xc>(v);
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ int wave_sum_i(int v) {
    v += dpp_i<kQuadSwap1>(v);
    v += dpp_i<kQuadSwap2>(v);
    v += dpp_i<kRowHalfMirror>(v);
    v += dpp_i<kRowMirror>(v);
    v += dpp_i<kRowBcast15, 0xa>(v);
    v += dpp_i<kRowBcast31, 0xc>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
    return v;
}

// Block sums of a double and an int in one barrier.  Reductions alternate
// between two LDS slots: a slot is rewritten two calls later, after every
// thread has passed the barrier of the call in between and so has read it.
template <int NW>
__device__ double block_sum_dc(double a, int& c, SampleShared<NW>& sh, int& ph) {
    a = wave_sum_d(a);
    c = wave_sum_i(c);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sh.red[ph][w] = a;
        sh.ired[ph][w] = c;
    }
    __syncthreads();
    double ta = 0.0;
    int tc = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        ta += sh.red[ph][i];
        tc += sh.ired[ph][i];
    }
    ph ^= 1;
    c = tc;
    return ta;
}

// the same, with c already the wave's total (the same in every lane)
template <int NW>
__device__ double block_sum_dc_wave(double a, int& c, SampleShared<NW>& sh, int& ph) {
    a = wave_sum_d(a);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sh.red[ph][w] = a;
        sh.ired[ph][w] = c;
    }
    __syncthreads();
    double ta = 0.0;
    int tc = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        ta += sh.red[ph][i];
        tc += sh.ired[ph][i];
    }
    ph ^= 1;
    c = tc;
    return ta;
}

template <int NW>
__device__ int block_min_i(int v, SampleShared<NW>& sh, int& ph) {
    v = wave_min_i(v);
    if ((threadIdx.x & 63) == 0) sh.imin[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    int t = INT_MAX;
#pragma unroll
    for (int i = 0; i < NW; ++i) t = min(t, sh.imin[ph][i]);
    ph ^= 1;
    return t;
}

// exclusive prefix of v over the threads in thread order; *total = the block sum
template <int NW, class T>
__device__ T block_excl_scan(T v, T* total, T (*slot)[NW], int& ph) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    T ex = __shfl_up(inc, 1);
    if (lane == 0) ex = T(0);
    if (lane == 63) slot[ph][wave] = inc;
    __syncthreads();
    T before = T(0), tot = T(0);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const T x = slot[ph][w];
        if (w < wave) before += x;
        tot += x;
    }
    ph ^= 1;
    *total = tot;
    return before + ex;
}

// A bracket [lo, hi) of fp32 bit patterns for a search "largest v whose mass
// G(v) = sum of e_i >= v passes the test": the test holds at lo and fails at
// hi.  g_hi = G(hi); c_lo, c_hi = the numbers of positive e_i >= lo, >= hi.
struct Bracket {
    uint32_t lo, hi;
    double g_hi;
    int c_lo, c_hi;
};

// Bisect b down to hi = lo + 1; STRICT tests G(v) > thr, else G(v) >= thr.
template <int NT, int E, bool STRICT>
__device__ void value_search(const float (&e)[E], double thr, Bracket& b, SampleShared<NT / 64>& sh, int& ph) {
    // over the registers while more than kCap values lie in the bracket
    while (b.hi - b.lo > 1 && b.c_lo - b.c_hi > kCap) {
        const uint32_t mid = b.lo + (b.hi - b.lo) / 2;
        const float v = __uint_as_float(mid);
        float af = 0.f;
        int c = 0;  // counted per wave from the compare masks (scalar unit)
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const bool in = e[k] >= v;
            af += in ? e[k] : 0.f;
            c += __popcll(__ballot(in));
        }
        const double a = block_sum_dc_wave((double)af, c, sh, ph);
        if (STRICT ? a > thr : a >= thr) {
            b.lo = mid;
            b.c_lo = c;
        } else {
            b.hi = mid;
            b.g_hi = a;
            b.c_hi = c;
        }
    }
    if (b.hi - b.lo <= 1) return;
    // compact the positive values in [lo, hi) into LDS; wave 0 finishes alone
    const float flo = __uint_as_float(b.lo), fhi = __uint_as_float(b.hi);
    int mine = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) mine += (e[k] >= flo) & (e[k] < fhi) & (e[k] > 0.f);
    int m;
    int off = block_excl_scan<NT / 64, int>(mine, &m, sh.ired, ph);
    m = min(m, kCap);  // m = c_lo - c_hi <= kCap; the clamp only guards the LDS list
#pragma unroll
    for (int k = 0; k < E; ++k)
        if ((e[k] >= flo) & (e[k] < fhi) & (e[k] > 0.f)) {
            if (off < kCap) sh.cv[off] = e[k];
            ++off;
        }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const double g0 = b.g_hi;  // mass and count of the values >= hi at compaction
        const int c0 = b.c_hi;
        constexpr int L = kCap / 64;
        float x[L];  // the list, 0 past its end (0 is below every probe)
#pragma unroll
        for (int i = 0; i < L; ++i) x[i] = lane + 64 * i < m ? sh.cv[lane + 64 * i] : 0.f;
        while (b.hi - b.lo > 1) {
            const uint32_t mid = b.lo + (b.hi - b.lo) / 2;
            const float v = __uint_as_float(mid);
            float af = 0.f;
            int c = 0;
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const bool in = x[i] >= v;
                af += in ? x[i] : 0.f;
                c += in;
            }
            const double a = wave_sum_d((double)af) + g0;
            c = wave_sum_i(c) + c0;
            if (STRICT ? a > thr : a >= thr) {
                b.lo = mid;
                b.c_lo = c;
            } else {
                b.hi = mid;
                b.g_hi = a;
                b.c_hi = c;
            }
        }
        if (lane == 0) {
            sh.bd[0] = b.g_hi;
            sh.bi[0] = (int)b.lo;
            sh.bi[1] = b.c_lo;
            sh.bi[2] = b.c_hi;
        }
    }
    __syncthreads();
    b.g_hi = sh.bd[0];
    b.lo = (uint32_t)sh.bi[0];
    b.hi = b.lo + 1;
    b.c_lo = sh.bi[1];
    b.c_hi = sh.bi[2];
    __syncthreads();  // sh.bd / sh.bi are read before any later writer
}

template <int NT, int E>
__device__ int sample_draw(const float* __restrict__ logits, int n, float lmax, float temperature, float topp,
                           float coin, SampleShared<NT / 64>& sh) {
    const int t = threadIdx.x;
    // e = 2^((l - max) * log2(e) / T); w is finite (checked by the caller)
    const float w = (float)(1.4426950408889634 / (double)temperature);
    float e[E];  // first the logits, then in place their numerators
#pragma unroll
    for (int k = 0; k < E; ++k) e[k] = logits[(unsigned)min(t + k * NT, n - 1)];  // clamped; masked below
    __builtin_amdgcn_sched_barrier(0);
    float sf = 0.f;
    int pos = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const float x = exp2f((e[k] - lmax) * w);
        e[k] = (x == x && k * NT < n - t) ? x : 0.f;  // a NaN logit carries no mass
        sf += e[k];
        pos += e[k] > 0.f;
    }
    int ph = 0;
    const double dcoin = (double)coin;

    if (!(topp > 0.f && topp < 1.f)) {
        // index order.  Row k holds tokens k NT .. k NT + NT - 1, one per thread;
        // M(k) = mass of rows < k, from each thread's running sums pre[k].
        // M(0) = 0 <= r < M(E) = S: bisect for the last row k with M(k) <= r,
        // then scan that row over the threads.
        float pre[E + 1];
        pre[0] = 0.f;
#pragma unroll
        for (int k = 0; k < E; ++k) pre[k + 1] = pre[k] + e[k];  // pre[E] = sf
        int c = 0;
        const double S = block_sum_dc((double)sf, c, sh, ph);
        const double r = dcoin * S;
        int klo = 0, khi = E;
        double m_lo = 0.0;
        while (khi - klo > 1) {
            const int mid = (klo + khi) >> 1;
            float x = 0.f;
#pragma unroll
            for (int k = 1; k < E; ++k) x = k == mid ? pre[k] : x;  // mid is the same in every lane
            const double a = block_sum_dc((double)x, c, sh, ph);
            if (a <= r) {
                klo = mid;
                m_lo = a;
            } else {
                khi = mid;
            }
        }
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < E; ++k) x = k == klo ? e[k] : x;
        double row;
        const double ex = block_excl_scan<NT / 64, double>((double)x, &row, sh.red, ph);
        const int i = klo * NT + t;
        int cand = (x > 0.f && m_lo + (ex + (double)x) > r) ? i : INT_MAX;
        cand = block_min_i(cand, sh, ph);
        if (cand == INT_MAX) {
            // rounding left the row's end at or below r: its last token with mass
            cand = block_min_i(x > 0.f ? -i : INT_MAX, sh, ph);
            cand = cand == INT_MAX ? n - 1 : -cand;
        }
        return cand;
    }

    const double S = block_sum_dc((double)sf, pos, sh, ph);
    constexpr uint32_t kAboveOne = 0x3f800001u;  // the float just above 1 (the largest e_i is exp(0) = 1)
    const double P = (double)topp * S;
    int minbits = INT_MAX;  // the smallest positive numerator
#pragma unroll
    for (int k = 0; k < E; ++k)
        if (e[k] > 0.f) minbits = min(minbits, __float_as_int(e[k]));
    minbits = block_min_i(minbits, sh, ph);
    // (a) the test G(v) >= P holds at the smallest positive numerator (G = S > P)
    Bracket a{(uint32_t)minbits, kAboveOne, 0.0, pos, 0};
    value_search<NT, E, false>(e, P, a, sh, ph);
    const float vk = __uint_as_float(a.lo);
    const double above_vk = a.g_hi;  // mass of the e_i > v_k
    const int n_vk = a.c_lo - a.c_hi;
    int j = (int)ceil((P - above_vk) / (double)vk);
    j = max(1, min(j, n_vk));
    const double M = above_vk + (double)j * (double)vk;
    const double r = dcoin * M;

    // (b) the test G(u) > r holds at v_k, where the candidate mass is M > r
    Bracket bb{a.lo, kAboveOne, 0.0, a.c_lo, 0};
    value_search<NT, E, true>(e, r, bb, sh, ph);
    const float u = __uint_as_float(bb.lo);
    const int n_u = bb.lo == a.lo ? j : bb.c_lo - bb.c_hi;
    int q = (int)floor((r - bb.g_hi) / (double)u);
    q = max(0, min(q, n_u - 1));

    // the (q+1)-th token equal to u in index order
    if (q == 0) {
        int cand = INT_MAX;
#pragma unroll
        for (int k = 0; k < E; ++k)
            if (e[k] == u) cand = min(cand, t + k * NT);
        cand = block_min_i(cand, sh, ph);
        return cand == INT_MAX ? n - 1 : cand;
    }
    // first i with (number of tokens equal to u at indices <= i) >= q + 1
    int ilo = -1, ihi = n - 1;
    while (ihi - ilo > 1) {
        const int mid = ilo + (ihi - ilo) / 2;
        const int rel = mid - t;
        int c = 0;
#pragma unroll
        for (int k = 0; k < E; ++k) c += (e[k] == u) & (k * NT <= rel);
        (void)block_sum_dc(0.0, c, sh, ph);
        if (c >= q + 1)
            ihi = mid;
        else
            ilo = mid;
    }
    return ihi;
}

template <int NT, int E>
__global__ __launch_bounds__(NT) void next_token_kernel(NextTokenParams p) {
    __shared__ SampleShared<NT / 64> sh;
    const int pos = p.state->pos;
    if (p.state->stopped) return;
    const GenControl c = *p.ctl;
    int next;
    if (pos + 1 < c.force_end) {
        next = p.forced[pos + 1];
    } else {
        float v = -INFINITY;
        int i = INT_MAX;
        for (int b = threadIdx.x; b < p.nblocks; b += NT) {
            const float2 e = p.best[b];
            const int ei = __float_as_int(e.y);
            if (better(e.x, ei, v, i)) {
                v = e.x;
                i = ei;
            }
        }
        block_best<NT>(v, i);
        next = i == INT_MAX ? 0 : i;  // every value NaN: token 0
        // a non-finite maximum leaves no distribution to draw from: greedy
        // (1/T must be finite in fp32: a temperature below ~1e-38 is taken as 0)
        if (c.temperature > 0.f && isfinite(v) && isfinite((float)(1.4426950408889634 / (double)c.temperature)) &&
            p.n <= E * NT)
            next = sample_draw<NT, E>(p.logits, p.n, v, c.temperature, c.topp, p.coins[pos], sh);
    }
    __syncthreads();  // every thread has read the state
    if (threadIdx.x == 0) {
        p.state->next = next;
        if (p.tokens_out) p.tokens_out[pos] = next;
        p.state->token = next;
        p.state->pos = pos + 1;
        if (c.stop_token >= 0 && next == c.stop_token) p.state->stopped = 1;
    }
}

// ---------------------------------------------------------------------------
// Matrix-vector family.
//
// A block of NT threads owns a contiguous range of row groups.  Thread t holds
// float4 number t + k*NT of the input vector (k < NX) in registers for the
// whole block, so x (and its RMSNorm) is read and computed once per block.
// Per iteration the block streams RPI weight rows: every thread issues RPI*NX
// independent 16-byte loads (coalesced: consecutive threads read consecutive
// 16 bytes of a row), multiplies with its x slice, and the row sums are
// reduced with DPP inside each wave and through LDS across waves.  The LDS
// slots are double-buffered so one barrier per iteration suffices.
//
// The weights do not depend on x, so their loads are issued early: the first
// row group's before the x prologue (load, RMSNorm), and each next group's as
// soon as the current group's products are formed, so that they are in flight
// during the reduction, the barrier and the epilogue.

#ifndef LD_NT_LOADS
#define LD_NT_LOADS 1  // weight loads carry the non-temporal hint (each is used once)
#endif

// Data handed between blocks of one launch (attention split partials, the
// fused q/k/v kernel's stage), which may run on different XCDs with separate
// L2 caches.  They are stored and loaded with agent-scope relaxed atomics (32
// or 64 bits at a time), which the compiler issues with the coherence bit set:
// stores write through the L2 and loads read past stale lines, so no
// cache-wide write-back or invalidate is needed.
__device__ __forceinline__ unsigned long long pack2(float a, float b) {
    return ((unsigned long long)__float_as_uint(b) << 32) | __float_as_uint(a);
}
__device__ __forceinline__ float2 unpack2(unsigned long long v) {
    return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), pack2(v.x, v.y), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float4* p, float4 v) {
    unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
    __hip_atomic_store(q, pack2(v.x, v.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, pack2(v.z, v.w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent(const float2* p) {
    return unpack2(
        __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float4 load_coherent(const float4* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const float2 a = unpack2(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const float2 b = unpack2(__hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return make_float4(a.x, a.y, b.x, b.y);
}

// Wait until this thread's vector memory operations have completed
// (s_waitcnt vmcnt(0)).  The memory clobber also keeps the compiler from
// moving any load or store across it.
__device__ __forceinline__ void wait_vector_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef float native_float4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_w(const float4* p) {
#if LD_NT_LOADS
    const native_float4 v = __builtin_nontemporal_load(reinterpret_cast<const native_float4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
#else
    return *p;
#endif
}

// Row groups of a GEMV go to the blocks round robin (block b: groups b, b +
// grid, ...), so at any time the blocks read one contiguous stretch of the
// matrix.  With a contiguous range of groups per block (LD_GEMV_STRIDE 0) the
// 7B-shaped decode runs at 232.0 tok/s, with round robin 235.5-235.9; the
// plain streaming read is the other way round (contiguous shares 7.07 TB/s,
// 64 KB chunks round robin 6.59).
#ifndef LD_GEMV_STRIDE
#define LD_GEMV_STRIDE 1
#endif

constexpr bool is_qkv_kind(int kind) { return kind == K_QKV || kind == K_QKV_ATT; }

// Rows of row group u.  K_SWIGLU interleaves w1 and w3 rows of the same
// hidden unit; K_QKV walks the three matrices wq | wk | wv as one.
template <int RPI, int KIND>
__device__ __forceinline__ void group_rows(const GemvParams& p, int u, const float* (&wr)[RPI]) {
    const size_t n = (size_t)p.n;
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
        if constexpr (KIND == K_SWIGLU) {
            const int e = min(u * (RPI / 2) + r / 2, p.rows - 1);
            wr[r] = ((r & 1) ? p.w1 : p.w0) + (size_t)e * n;
        } else if constexpr (is_qkv_kind(KIND)) {
            const int row = min(u * RPI + r, p.rows - 1);
            wr[r] = row < p.seg1   ? p.w0 + (size_t)row * n
                    : row < p.seg2 ? p.w1 + (size_t)(row - p.seg1) * n
                                   : p.w2 + (size_t)(row - p.seg2) * n;
        } else {
            const int row = min(u * RPI + r, p.rows - 1);
            wr[r] = p.w0 + (size_t)row * n;
        }
    }
}

__device__ __forceinline__ float4 zero_unless(bool keep, float4 v) {
    return make_float4(keep ? v.x : 0.f, keep ? v.y : 0.f, keep ? v.z : 0.f, keep ? v.w : 0.f);
}

// Lanes past the end of a row load the row's last float4 again (always in
// bounds) and multiply it by their x slice, which is zero there: the weight
// loads stay unconditional and need no select, so none of them is waited for
// before its use.  (With finite weights the extra products are exactly 0; a
// non-finite weight in the last float4 of a row makes the row non-finite
// either way.)
template <int NT, int NX, int RPI, int KIND>
__device__ __forceinline__ void load_group(const GemvParams& p, int u, int n4, float4 (&w)[RPI][NX]) {
    const float* wr[RPI];
    group_rows<RPI, KIND>(p, u, wr);
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        const int at = min((int)threadIdx.x + k * NT, n4 - 1);
#pragma unroll
        for (int r = 0; r < RPI; ++r) w[r][k] = load_w(reinterpret_cast<const float4*>(wr[r]) + at);
    }
}

template <int NT, int NX, int RPI, int KIND>
__device__ void gemv_body(const GemvParams& p) {
    constexpr int NW = NT / 64;
    __shared__ float red[2][NW][RPI];
    __shared__ float ss_part[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n4 = p.n >> 2;

    // row groups of this block: round robin over the grid, or (the q/k/v
    // kernel with fused attention, whose blocks report the rows they wrote)
    // an even split of p.units into contiguous ranges
    constexpr bool kStride = LD_GEMV_STRIDE && KIND != K_QKV_ATT;
    const int u0 = kStride ? (int)blockIdx.x : (int)(((long long)blockIdx.x * p.units) / gridDim.x);
    const int u1 = kStride ? p.units : (int)(((long long)(blockIdx.x + 1) * p.units) / gridDim.x);
    const int ustep = kStride ? (int)gridDim.x : 1;
    float4 w[RPI][NX];
    if (u0 < u1) load_group<NT, NX, RPI, KIND>(p, u0, n4, w);

    int pos = 0, token = 0, stopped = 0;
    if constexpr (is_qkv_kind(KIND) || KIND == K_CLS) {
        pos = p.state->pos;
        token = p.state->token;
        stopped = p.state->stopped;
    }

    // ---- prologue: x (layer 0 of the q/k/v kernel reads the embedding row) ----
    const float* xsrc = p.x;
    if constexpr (is_qkv_kind(KIND)) {
        if (p.emb) xsrc = p.emb + (size_t)token * (size_t)p.n;
    }
    const float4* x4 = reinterpret_cast<const float4*>(xsrc);
    float4 xr[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        const int idx = tid + k * NT;
        xr[k] = zero_unless(idx < n4, x4[min(idx, n4 - 1)]);
    }
    if constexpr (is_qkv_kind(KIND)) {
        if (p.emb && blockIdx.x == 0) {
            float4* xo = reinterpret_cast<float4*>(p.x_resid);
#pragma unroll
            for (int k = 0; k < NX; ++k) {
                const int idx = tid + k * NT;
                if (idx < n4) xo[idx] = xr[k];
            }
        }
    }
    // RMSNorm: x' = g * (x * 1/sqrt(mean(x^2) + eps))
    if (p.gain) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NX; ++k) ss = dot4(xr[k], xr[k], ss);
        ss = wave_sum(ss);
        if (lane == 0) ss_part[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) tot += ss_part[w2];
        const float r = 1.0f / sqrtf(tot / (float)p.n + p.eps);
        const float4* g4 = reinterpret_cast<const float4*>(p.gain);
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int idx = tid + k * NT;
            const float4 g = zero_unless(idx < n4, g4[min(idx, n4 - 1)]);
            xr[k] = make_float4(g.x * (r * xr[k].x), g.y * (r * xr[k].y), g.z * (r * xr[k].z), g.w * (r * xr[k].w));
        }
    }

    // The residual rows a group adds to are loaded a group ahead, with the
    // group's weights, so the residual epilogue never waits on a load (wo
    // 11.7 -> 11.3 us, w2 29.1 -> 28.8 us on the 7B shape; the same for the
    // q/k/v rotation was slower).  The load is unconditional (row clamped,
    // every thread): a load behind a branch would make the compiler's later
    // waits ones for every load in flight.
    auto res_load = [&](int uu) { return p.x_resid[min(uu * RPI + (tid % RPI), p.rows - 1)]; };
    float res_cur = 0.f, res_nxt = 0.f;
    if constexpr (KIND == K_RESID) {
        if (u0 < u1) res_cur = res_load(u0);
    }

    float bv = -INFINITY;
    int bi = INT_MAX;
    int buf = 0;
    for (int u = u0; u < u1; u += ustep) {
        float acc[RPI];
#pragma unroll
        for (int r = 0; r < RPI; ++r) {
            acc[r] = 0.f;
#pragma unroll
            for (int k = 0; k < NX; ++k) acc[r] = dot4(w[r][k], xr[k], acc[r]);
        }
        // keep the next group's loads after these products: hoisting them
        // would hold two groups of weights in registers at once
        __builtin_amdgcn_sched_barrier(0);
        if (u + ustep < u1) {
            load_group<NT, NX, RPI, KIND>(p, u + ustep, n4, w);
            if constexpr (KIND == K_RESID) res_nxt = res_load(u + ustep);
        }
#pragma unroll
        for (int r = 0; r < RPI; ++r) acc[r] = wave_sum(acc[r]);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < RPI; ++r) red[buf][wave][r] = acc[r];
        }
        __syncthreads();
        float total = 0.f;
        if (tid < RPI) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) total += red[buf][w2][tid];
        }
        buf ^= 1;

        // ---- epilogues (row u*RPI + tid lives in thread tid < RPI) ----
        if constexpr (KIND == K_PLAIN) {
            const int row = u * RPI + tid;
            if (tid < RPI && row < p.rows) p.out[row] = total;
        } else if constexpr (KIND == K_RESID) {
            const int row = u * RPI + tid;
            if (tid < RPI && row < p.rows) p.x_resid[row] = res_cur + total;
        } else if constexpr (is_qkv_kind(KIND)) {
            // RoPE ("run.c 逐行解讀" §4 step 2d): rows 2j, 2j+1 of a head form
            // one pair, turned by the angle pos * theta^(-2j/head_size); the
            // (cos, sin) of that angle come from the table.  q rows are
            // rotated, k rows are rotated and written to cache row pos, v rows
            // go to the value cache unrotated (step 2b).  K_QKV_ATT hands
            // every row to the attention through the stage as well, and keeps
            // q there only.
            const float other = __shfl_xor(total, 1);
            const int row = u * RPI + tid;
            if (tid < RPI && row < p.rows) {
                const bool odd = tid & 1;
                const int hs = p.head_size;
                float v = total;
                if (row < p.seg2) {
                    const bool is_q = row < p.seg1;
                    const int local = is_q ? row : row - p.seg1;
                    const int j = (local % hs) >> 1;
                    const float2 cs = p.rope[(size_t)pos * (size_t)(hs >> 1) + j];
                    const float a = odd ? other : total;  // element 2j
                    const float b = odd ? total : other;  // element 2j+1
                    v = odd ? (a * cs.y + b * cs.x) : (a * cs.x - b * cs.y);
                    if (is_q) {
                        if constexpr (KIND == K_QKV) p.out[row] = v;
                    } else if (!stopped) {
                        p.kc[(size_t)pos * p.kv_stride + local] = v;
                    }
                } else if (!stopped) {
                    p.vc[(size_t)pos * p.kv_stride + (row - p.seg2)] = total;
                }
                if constexpr (KIND == K_QKV_ATT) store_coherent(p.stage + (size_t)(row / hs) * p.stage_sh + row % hs, v);
            }
        } else if constexpr (KIND == K_SWIGLU) {
            // hb = silu(w1 x) * (w3 x), silu(u) = u * 1/(1 + e^-u) ("run.c
            // 逐行解讀" §4 step 2h).  Even threads hold the w1 row, odd the w3 row.
            const float other = __shfl_xor(total, 1);
            const int e = u * (RPI / 2) + (tid >> 1);
            if (tid < RPI && !(tid & 1) && e < p.rows) {
                float a = total;
                a *= 1.0f / (1.0f + expf(-a));
                a *= other;
                p.out[e] = a;
            }
        } else if constexpr (KIND == K_CLS) {
            const int row = u * RPI + tid;
            if (tid < RPI && row < p.rows) {
                p.out[row] = total;
                if (better(total, row, bv, bi)) {
                    bv = total;
                    bi = row;
                }
            }
        }
        res_cur = res_nxt;
    }

    if constexpr (KIND == K_CLS) publish_best<NT>(bv, bi, p.best);
}

template <int NT, int NX, int RPI, int KIND>
__global__ __launch_bounds__(NT) void gemv_kernel(GemvParams p) {
    gemv_body<NT, NX, RPI, KIND>(p);
}

// The same product for a few vectors at once (a decode batch of up to NB
// sequences): every weight row is streamed once and multiplied into the NB
// vectors held in registers, so for small batches the step keeps the GEMV's
// weight stream, its fused RMSNorm and epilogues, and no split of K.  Vectors
// past p.nb repeat the last one; their results are not stored.
template <int NT, int NX, int RPI, int KIND, int NB>
__global__ __launch_bounds__(NT) void gemv_batch_kernel(GemvParams p) {
    constexpr int NW = NT / 64, V = NB * RPI;
    static_assert(V <= 64, "the epilogue lanes sit in wave 0");
    __shared__ float red[2][NW][V];
    __shared__ float ss_part[NW][NB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n4 = p.n >> 2;

    constexpr bool kStride = LD_GEMV_STRIDE;
    const int u0 = kStride ? (int)blockIdx.x : (int)(((long long)blockIdx.x * p.units) / gridDim.x);
    const int u1 = kStride ? p.units : (int)(((long long)(blockIdx.x + 1) * p.units) / gridDim.x);
    const int ustep = kStride ? (int)gridDim.x : 1;
    float4 w[RPI][NX];
    if (u0 < u1) load_group<NT, NX, RPI, KIND>(p, u0, n4, w);

    float4 xr[NB][NX];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float4* x4 = reinterpret_cast<const float4*>(p.x + (size_t)min(b, p.nb - 1) * p.ldx);
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int idx = tid + k * NT;
            xr[b][k] = zero_unless(idx < n4, x4[min(idx, n4 - 1)]);
        }
    }
    // RMSNorm of every vector: x' = g * (x * 1/sqrt(mean(x^2) + eps))
    if (p.gain) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < NX; ++k) ss = dot4(xr[b][k], xr[b][k], ss);
            ss = wave_sum(ss);
            if (lane == 0) ss_part[wave][b] = ss;
        }
        __syncthreads();
        const float4* g4 = reinterpret_cast<const float4*>(p.gain);
        float4 g[NX];
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int idx = tid + k * NT;
            g[k] = zero_unless(idx < n4, g4[min(idx, n4 - 1)]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float tot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) tot += ss_part[w2][b];
            const float r = 1.0f / sqrtf(tot / (float)p.n + p.eps);
#pragma unroll
            for (int k = 0; k < NX; ++k)
                xr[b][k] = make_float4(g[k].x * (r * xr[b][k].x), g[k].y * (r * xr[b][k].y),
                                       g[k].z * (r * xr[b][k].z), g[k].w * (r * xr[b][k].w));
        }
    }

    // lane tid < V of wave 0 finishes (vector tid / RPI, row tid % RPI) of a group
    const int vb = tid / RPI, vr = tid % RPI;
    const bool mine = tid < V && vb < p.nb;
    int buf = 0;
    for (int u = u0; u < u1; u += ustep) {
        float acc[NB][RPI];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < RPI; ++r) {
                acc[b][r] = 0.f;
#pragma unroll
                for (int k = 0; k < NX; ++k) acc[b][r] = dot4(w[r][k], xr[b][k], acc[b][r]);
            }
        __builtin_amdgcn_sched_barrier(0);
        if (u + ustep < u1) load_group<NT, NX, RPI, KIND>(p, u + ustep, n4, w);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < RPI; ++r) {
                const float t = wave_sum(acc[b][r]);
                if (lane == 0) red[buf][wave][b * RPI + r] = t;
            }
        __syncthreads();
        float total = 0.f;
        if (tid < V) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) total += red[buf][w2][tid];
        }
        buf ^= 1;

        if constexpr (KIND == K_PLAIN) {
            const int row = u * RPI + vr;
            if (mine && row < p.rows) p.out[(size_t)vb * p.ldo + row] = total;
        } else if constexpr (KIND == K_RESID) {
            const int row = u * RPI + vr;
            if (mine && row < p.rows) p.x_resid[(size_t)vb * p.ldr + row] += total;
        } else if constexpr (KIND == K_QKV) {
            // RoPE and the cache append as in gemv_kernel, at sequence vb's
            // own position and in its own caches
            const float other = __shfl_xor(total, 1);
            const int row = u * RPI + vr;
            if (mine && row < p.rows) {
                const bool odd = vr & 1;
                const int pos = p.row_state[vb].pos;
                const size_t seq = (size_t)vb * p.seq_stride;
                if (row < p.seg2) {
                    const bool is_q = row < p.seg1;
                    const int local = is_q ? row : row - p.seg1;
                    const int hs = p.head_size;
                    const float2 cs = p.rope[(size_t)pos * (size_t)(hs >> 1) + ((local % hs) >> 1)];
                    const float a = odd ? other : total;  // element 2j
                    const float b = odd ? total : other;  // element 2j+1
                    const float v = odd ? (a * cs.y + b * cs.x) : (a * cs.x - b * cs.y);
                    if (is_q)
                        p.out[(size_t)vb * p.ldo + row] = v;
                    else
                        p.kc[seq + (size_t)pos * p.kv_stride + local] = v;
                } else {
                    p.vc[seq + (size_t)pos * p.kv_stride + (row - p.seg2)] = total;
                }
            }
        } else if constexpr (KIND == K_SWIGLU) {
            const float other = __shfl_xor(total, 1);
            const int e = u * (RPI / 2) + (vr >> 1);
            if (mine && !(vr & 1) && e < p.rows) {
                float a = total;
                a *= 1.0f / (1.0f + expf(-a));
                a *= other;
                p.out[(size_t)vb * p.ldo + e] = a;
            }
        }
    }
}

// A plain streaming read: the practical HBM read ceiling the weight streams
// are measured against.  Block b sums its contiguous range of the buffer
// (non-temporal 16-byte loads, 16 per thread in flight, like the weight
// loads of the GEMVs) into sums[b]; the sums keep the loads live.
// ---------------------------------------------------------------------------
// Batch decode of up to 64 sequences on the matrix cores, weights pre-tiled
// (TiledParams): the q/k/v, wo, w1/w3, w2 and classifier products of a decode
// step over the batch's vectors, C(rows x nb) = W x_b, in planes of 16
// sequences (NP planes: each weight float4 feeds the MFMAs of every plane).  Each wave loads whole
// 1 KB tiles (64 lanes x 16 contiguous bytes) and feeds each lane's float4 to
// four v_mfma_f32_16x16x4f32 steps as the A operand (rows 16 rt + l % 16, k
// 16 kt + 4 (l / 16) + t at step t), with the tiled activations as the B
// operand (sequence l % 16 at the same k).  Weights stream once for the whole
// batch without an LDS stage.  A block takes RT row tiles over all of K (or,
// with the K split, over one of KS parts of K): its NW waves take the k tiles
// round robin (wave w: tiles w, w + NW, ..., so the block reads NW
// consecutive tiles per step), then add their partial tiles through LDS in
// wave order.  The output lane l holds rows 16 rt + 4 (l / 16)
// + 0..3 of sequence l % 16: RoPE pairs and SwiGLU (w1, w3) pairs sit in one
// lane.  RMSNorm: the gain is folded into the tiled weights, and each
// sequence's sum of squares is accumulated from the same activations, so the
// row scale multiplies the result.

// float4 slot of x[b][k] (k a multiple of 4) in the tiled activations of
// vectors of n floats (planes of 16 sequences)
__host__ __device__ __forceinline__ size_t tiled_slot(int b, int k, int n) {
    return ((size_t)(b >> 4) * (size_t)(n >> 4) + (size_t)(k >> 4)) * 64 + ((k & 15) >> 2) * 16 + (b & 15);
}

// The 1 KB weight tiles of a product sit in groups of LD_TILED_KG k tiles:
// group g holds k tiles 8g .. 8g + 7 of row tile 0, then of row tile 1, and so
// on, so the blocks, which all walk K at about the same pace, read one
// contiguous stretch of the copy at a time.  With each row tile's K contiguous
// instead (LD_TILED_KG 0), the blocks' streams sit one row tile (256-688 KB)
// apart and the batch step is 3-4% slower (7B shape, 8 / 16 / 32 sequences
// 5.03 / 5.08 / 6.58 -> 4.81 / 4.87 / 6.38 ms per step; groups of 4 or 16
// within 0.5% of 8).
#ifndef LD_TILED_KG
#define LD_TILED_KG 8
#endif
// 1 KB weight tile (row tile rt of rtn, k tile kt of KT) in the tiled weights
__host__ __device__ __forceinline__ size_t tiled_wtile(int rt, int kt, int rtn, int KT) {
    if constexpr (LD_TILED_KG == 0) {
        return (size_t)rt * KT + kt;
    } else {
        const int g = kt / LD_TILED_KG, g0 = g * LD_TILED_KG;
        const int width = KT - g0 < LD_TILED_KG ? KT - g0 : LD_TILED_KG;
        return (size_t)g0 * rtn + (size_t)rt * width + (kt - g0);
    }
}

__device__ __forceinline__ float f4c(const float4& v, int t) { return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w; }

__global__ __launch_bounds__(256) void tile_weights_kernel(int kind, const float* __restrict__ w0,
                                                           const float* __restrict__ w1,
                                                           const float* __restrict__ w2, int seg1, int seg2,
                                                           const float* __restrict__ gain, int rows, int k,
                                                           float4* __restrict__ dst) {
    const size_t n4 = (size_t)rows * (size_t)k / 4;
    const int kt_n = k / 16;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        const size_t tile = i / 64;
        const int l = (int)(i % 64);
        const int rt = (int)(tile / kt_n), kt = (int)(tile % kt_n);
        const int row = 16 * rt + (l & 15), col = 16 * kt + 4 * (l >> 4);
        const float* src;
        const size_t di = tiled_wtile(rt, kt, rows / 16, kt_n) * 64 + l;
        if (kind == K_QKV)
            src = row < seg1 ? w0 + (size_t)row * k : row < seg2 ? w1 + (size_t)(row - seg1) * k : w2 + (size_t)(row - seg2) * k;
        else if (kind == K_SWIGLU)
            src = ((row & 1) ? w1 : w0) + (size_t)(row >> 1) * k;
        else
            src = w0 + (size_t)row * k;
        float4 v = *reinterpret_cast<const float4*>(src + col);
        if (gain) {
            const float4 g = *reinterpret_cast<const float4*>(gain + col);
            v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
        }
        dst[di] = v;
    }
}

// Shapes of tiled_shape (the products that take neither the one-block shapes
// nor the K split: row tiles no more than CUs, with the RMSNorm; the figures
// below were measured when every product took tiled_shape).  Waves per block
// and steps of tiles in flight: one plane (up to 16 sequences), two planes
// (17-32).  7B shape, 8 / 16 / 32 sequences: 8 waves
// and 4 steps 5.05 / 5.07 / 6.47 ms per step; 3 steps 5.05 / 5.08 / 6.44-6.47;
// 6 steps 5.16 / 5.20 / 6.72; 8 steps (one plane) 5.18 / 5.23; 4 waves
// 5.44 / 5.49 / 6.70.
#ifndef LD_TILED_NW1
#define LD_TILED_NW1 8
#endif
#ifndef LD_TILED_D1
#define LD_TILED_D1 4
#endif
#ifndef LD_TILED_NW2
#define LD_TILED_NW2 8
#endif
#ifndef LD_TILED_D2
#define LD_TILED_D2 4
#endif
// three or four planes (33-48, 49-64 sequences): 4 waves, 2 steps in
// flight, up to 4 row tiles.  7B shape, 40 / 64 sequences: 8.03 / 9.76 ms
// per step, against 10.12 / 10.68 with the split-K products; four planes for
// 40 as well 9.62; 8 waves 9.76-10.16 / 9.93-10.31 (3 steps 10.09, 1 step
// 12.08); 2 waves 14.7.
#ifndef LD_TILED_NW4
#define LD_TILED_NW4 4
#endif
#ifndef LD_TILED_D4
#define LD_TILED_D4 2
#endif
#ifndef LD_TILED_RT4
#define LD_TILED_RT4 4
#endif

// KS > 1: K in KS parts, blocks KS g .. KS g + KS - 1 take row tiles RT g ..
// RT g + RT - 1 over one part each (so each activation load serves RT row
// tiles even where the row tiles do not fill the CUs).  Each stores its
// partial tiles (coherent stores) to p.part and counts its arrival in
// p.arrive[g]; the block that completes the count resets it, adds the KS
// partials in part order and runs the epilogue.  No block waits for another.
// Not with p.norm.
template <int NW, int RT, int D, int KIND, int NP, int KS = 1>
__global__ __launch_bounds__(NW * 64) void tiled_kernel(TiledParams p) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    constexpr int NE = RT * NP;                 // output tiles of the block
    constexpr int EPT = (NE + NW - 1) / NW;     // epilogue entries per thread
    __shared__ v4 red[NW][NE][64];
    __shared__ float ss_s[NW][NP][16];
    const int KT = p.k >> 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = KS > 1 ? (int)blockIdx.x / KS : (int)blockIdx.x;
    const int part = KS > 1 ? (int)blockIdx.x % KS : 0;
    // row tiles rt0 .. rt0 + cnt - 1; the last block's surplus tiles (j >=
    // cnt) re-read its first tile, which stays in the cache, and store nothing
    const int rtn = p.rows >> 4;
    const int rt0 = grp * RT, cnt = min(RT, rtn - rt0);
    const int kb0 = KS > 1 ? part * KT / KS : 0, kb1 = KS > 1 ? (part + 1) * KT / KS : KT;  // k tiles of this block
    const float4* wt = reinterpret_cast<const float4*>(p.w) + lane;
    const float4* xt = reinterpret_cast<const float4*>(p.x) + lane;  // plane jb at + jb * KT * 64
    const int nsteps = (kb1 - kb0 + NW - 1) / NW;  // this wave: tiles kb0 + wave, kb0 + wave + NW, ... below kb1
    // the residual rows this thread adds to in the epilogue are loaded now, so
    // the epilogue does not wait on them
    float4 res[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        res[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (KIND == K_RESID) {
            const int e = threadIdx.x + i * NW * 64, t = e >> 6, l = e & 63;
            const int b = 16 * (t % NP) + (l & 15), r0 = 16 * (rt0 + t / NP) + 4 * (l >> 4);
            if (t < NE && t / NP < cnt && b < p.nb && r0 < p.rows) res[i] = *reinterpret_cast<const float4*>(p.x_resid + (size_t)b * p.ldr + r0);
        }
    }

    v4 acc[RT][NP];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int jb = 0; jb < NP; ++jb) acc[j][jb] = v4{0.f, 0.f, 0.f, 0.f};
    float ss[NP];
#pragma unroll
    for (int jb = 0; jb < NP; ++jb) ss[jb] = 0.f;
    float4 w[D][RT], xv[D][NP];
    // step kk's tiles into slot d (past the end: re-read the last tile, not used)
    auto load_one = [&](int kk, int d) {
        const int kt = min(kb0 + kk * NW + wave, kb1 - 1);
#pragma unroll
        for (int j = 0; j < RT; ++j) w[d][j] = wt[tiled_wtile(rt0 + (j < cnt ? j : 0), j < cnt ? kt : kb0, rtn, KT) * 64];
#pragma unroll
        for (int jb = 0; jb < NP; ++jb) xv[d][jb] = xt[((size_t)jb * KT + kt) * 64];
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_one(d, d);
    for (int kk = 0; kk < nsteps; kk += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (kb0 + (kk + d) * NW + wave < kb1) {  // wave-uniform
                if (p.norm) {
#pragma unroll
                    for (int jb = 0; jb < NP; ++jb) ss[jb] = dot4(xv[d][jb], xv[d][jb], ss[jb]);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int j = 0; j < RT; ++j)
#pragma unroll
                        for (int jb = 0; jb < NP; ++jb)
                            acc[j][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(f4c(w[d][j], t), f4c(xv[d][jb], t),
                                                                              acc[j][jb], 0, 0, 0);
            }
            // slot d refills with step kk + D + d as soon as its products are
            // issued, so D steps of tiles stay in flight all the time in the
            // same registers (7B shape: 16 sequences 5.18 -> 5.07 ms per step,
            // 32 sequences 6.89 -> 6.49, against refilling all D slots after
            // the D steps' products).  Unconditional: past the end it re-reads
            // the last tile; a load that may not have been issued would make
            // every later wait one for all loads in flight.
            __builtin_amdgcn_sched_barrier(0);
            load_one(kk + D + d, d);
        }
    }
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int jb = 0; jb < NP; ++jb) red[wave][j * NP + jb][lane] = acc[j][jb];
    if (p.norm) {  // lanes c, c + 16, c + 32, c + 48 hold sequence c's k in parts
#pragma unroll
        for (int jb = 0; jb < NP; ++jb) {
            float v = ss[jb];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (lane < 16) ss_s[wave][jb][lane] = v;
        }
    }
    __syncthreads();
    v4 sums[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NW * 64, t = e >> 6, l = e & 63;
        sums[i] = v4{0.f, 0.f, 0.f, 0.f};
        if (t >= NE) break;
        v4 sum = red[0][t][l];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) sum += red[w2][t][l];
        if (p.norm) {
            float q2 = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) q2 += ss_s[w2][t % NP][l & 15];
            sum *= 1.0f / sqrtf(q2 / (float)p.k + p.eps);
        }
        sums[i] = sum;
    }
    if constexpr (KS > 1) {
        __shared__ int last_s;
        float4* pt = reinterpret_cast<float4*>(p.part) + (size_t)grp * KS * NE * 64;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * NW * 64;
            if (e >= NE * 64) break;
            store_coherent(pt + (size_t)part * NE * 64 + e, make_float4(sums[i][0], sums[i][1], sums[i][2], sums[i][3]));
        }
        wait_vector_memory();
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned before = atomicAdd(p.arrive + grp, 1u);
            const int last = before + 1 == (unsigned)KS;
            if (last) atomicExch(p.arrive + grp, 0u);
            last_s = last;
        }
        __syncthreads();
        if (!last_s) return;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * NW * 64;
            if (e >= NE * 64) break;
            v4 sum = v4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < KS; ++q) {
                const float4 v = load_coherent(pt + (size_t)q * NE * 64 + e);
                sum += v4{v.x, v.y, v.z, v.w};
            }
            sums[i] = sum;
        }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NW * 64, t = e >> 6, l = e & 63;
        if (t >= NE) break;
        const int j = t / NP, jb = t % NP, b = 16 * jb + (l & 15);
        if (b >= p.nb || j >= cnt) continue;
        const v4 sum = sums[i];
        const int r0 = 16 * (rt0 + j) + 4 * (l >> 4);  // rows r0 .. r0 + 3 of sequence b
        if (r0 >= p.rows) continue;
        if constexpr (KIND == K_PLAIN) {
            *reinterpret_cast<float4*>(p.out + (size_t)b * p.ldo + r0) = make_float4(sum[0], sum[1], sum[2], sum[3]);
        } else if constexpr (KIND == K_RESID) {
            const float4 o = res[i];
            const float4 v = make_float4(o.x + sum[0], o.y + sum[1], o.z + sum[2], o.w + sum[3]);
            *reinterpret_cast<float4*>(p.x_resid + (size_t)b * p.ldr + r0) = v;
            if (p.out_t) reinterpret_cast<float4*>(p.out_t)[tiled_slot(b, r0, p.rows)] = v;
        } else if constexpr (KIND == K_SWIGLU) {
            // rows (w1 u, w3 u, w1 u+1, w3 u+1), u = r0 / 2: hb = silu(w1 x) (w3 x)
            // ("run.c 逐行解讀" §4 step 2h)
            const float a0 = sum[0], a1 = sum[2];
            const float h0 = a0 * (1.0f / (1.0f + expf(-a0))) * sum[1];
            const float h1 = a1 * (1.0f / (1.0f + expf(-a1))) * sum[3];
            const int u = r0 >> 1;  // even: the pair (u, u + 1) is half of a tiled float4
            *reinterpret_cast<float2*>(p.out_t + 4 * tiled_slot(b, u & ~3, p.rows >> 1) + (u & 3)) = make_float2(h0, h1);
        } else if constexpr (KIND == K_QKV) {
            // RoPE at the sequence's own position on q and k rows (pairs
            // (r0, r0+1) and (r0+2, r0+3)), k and v into its cache row
            // ("run.c 逐行解讀" §4 steps 2b-2d)
            const int pos = p.row_state[b].pos;
            const size_t seq = (size_t)b * p.seq_stride;
            float v[4] = {sum[0], sum[1], sum[2], sum[3]};
            if (r0 < p.seg2) {
                const bool is_q = r0 < p.seg1;
                const int local = is_q ? r0 : r0 - p.seg1;
                const int hs = p.head_size;
#pragma unroll
                for (int h = 0; h < 4; h += 2) {
                    const float2 cs = p.rope[(size_t)pos * (size_t)(hs >> 1) + (((local + h) % hs) >> 1)];
                    const float a = v[h], bb = v[h + 1];
                    v[h] = a * cs.x - bb * cs.y;
                    v[h + 1] = a * cs.y + bb * cs.x;
                }
                const float4 o = make_float4(v[0], v[1], v[2], v[3]);
                if (is_q)
                    *reinterpret_cast<float4*>(p.out + (size_t)b * p.ldo + r0) = o;
                else
                    *reinterpret_cast<float4*>(p.kc + seq + (size_t)pos * p.kv_stride + local) = o;
            } else {
                *reinterpret_cast<float4*>(p.vc + seq + (size_t)pos * p.kv_stride + (r0 - p.seg2)) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

constexpr int kStreamThreads = 256, kStreamU = 16;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const float4* __restrict__ src, long long n4,
                                                                     long long per, float* __restrict__ sums) {
    __shared__ float part[kStreamThreads / 64];
    float acc = 0.f;
    const long long b0 = (long long)blockIdx.x * per;
    const long long b1 = min(n4, b0 + per);
    long long i = b0 + threadIdx.x;
    for (; i + (long long)(kStreamU - 1) * kStreamThreads < b1; i += (long long)kStreamThreads * kStreamU) {
        float4 v[kStreamU];
#pragma unroll
        for (int u = 0; u < kStreamU; ++u) v[u] = load_w(src + i + u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamU; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < b1; i += kStreamThreads) {
        const float4 v = load_w(src + i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamThreads / 64; ++w) t += part[w];
        sums[blockIdx.x] = t;
    }
}

// Argmax of a vector: per-block bests (the reduction the classifier uses),
// then next_token_kernel.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(const float* v, int n, float2* best) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int i = blockIdx.x * kArgmaxThreads + threadIdx.x; i < n; i += gridDim.x * kArgmaxThreads)
        if (better(v[i], i, bv, bi)) {
            bv = v[i];
            bi = i;
        }
    publish_best<kArgmaxThreads>(bv, bi, best);
}

__global__ void set_control_kernel(GenControl* dst, GenControl c) { *dst = c; }

// ---------------------------------------------------------------------------
// A batch of decode steps: row b is sequence b.

// x[b] = E[state[b].token]
__global__ __launch_bounds__(256) void embed_state_kernel(const float* __restrict__ emb,
                                                          const StepState* __restrict__ st, int dim,
                                                          float* __restrict__ x, float* __restrict__ xt) {
    const int b = blockIdx.x;
    const float4* src = reinterpret_cast<const float4*>(emb + (size_t)st[b].token * dim);
    float4* dst = reinterpret_cast<float4*>(x + (size_t)b * dim);
    for (int i = threadIdx.x; i < dim / 4; i += 256) {
        const float4 v = src[i];
        dst[i] = v;
        if (xt) reinterpret_cast<float4*>(xt)[tiled_slot(b, 4 * i, dim)] = v;
    }
}

// The greedy choice of every row of the batch's logits (one block per row, the
// argmax order of the "run.c" page), then the step state of that sequence
// advances as a single sequence's does.
constexpr int kRowsThreads = 1024;

__global__ __launch_bounds__(kRowsThreads) void argmax_rows_kernel(const float* __restrict__ logits, int n,
                                                                   StepState* st, int32_t* tokens_out,
                                                                   int tokens_stride) {
    const int b = blockIdx.x;
    const float* row = logits + (size_t)b * n;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int i = threadIdx.x; i < n; i += kRowsThreads)
        if (better(row[i], i, bv, bi)) {
            bv = row[i];
            bi = i;
        }
    block_best<kRowsThreads>(bv, bi);
    if (threadIdx.x == 0) {
        const int next = bi == INT_MAX ? 0 : bi;  // every value NaN: token 0
        const int pos = st[b].pos;
        st[b].next = next;
        tokens_out[(size_t)b * tokens_stride + pos] = next;
        st[b].token = next;
        st[b].pos = pos + 1;
    }
}

__global__ void set_state_kernel(StepState* st, int token, int pos) {
    st->token = token;
    st->pos = pos;
    st->next = -1;
    st->stopped = 0;
}

// The position of a single attention launch and its zeroed split arrival counts.
__global__ void attn_op_init_kernel(StepState* st, int pos, unsigned* arrive, int n_kv_heads) {
    for (int i = threadIdx.x; i < n_kv_heads; i += blockDim.x) arrive[i] = 0u;
    if (threadIdx.x == 0) {
        st->token = 0;
        st->pos = pos;
        st->next = -1;
        st->stopped = 0;
    }
}

// ---------------------------------------------------------------------------
// Causal grouped-query attention at one position ("run.c 逐行解讀" §4 step
// 2e), split along the key axis (flash-decoding).
//
// The n = pos+1 keys form tiles of CH keys.  Block (g, s) serves kv head g and
// a contiguous run of tiles: the launch has grid.y = nsplit blocks per kv
// head, each split takes at least min_tiles tiles, and blocks past the last
// split exit at once, so one launch shape serves every position up to its
// context.  Every query head h with floor(h*KV/H) = g shares the block's key
// and value reads.  A block folds its keys into a running max m, exp-sum l
// and unnormalised value sum per head (online softmax: when m grows, l and the
// sum are rescaled by 2^{m_old - m_new}; scores are kept in base-2 units,
// s * log2(e) / sqrt(head_size), so every exponential is one exp2).  Each
// block leaves (m, l, sum) as a partial, and they are combined exactly,
// out = sum_s 2^{m_s - M} acc_s / sum_s 2^{m_s - M} l_s, M = max_s m_s:
// by the last block of the kv group to finish (merge_group) when each thread
// of that block folds a few splits, else by attn_merge_kernel, one block per
// query head.  With one split the block writes the output itself.

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32; 0 at -inf

__device__ __forceinline__ void group_of(int g, int H, int KV, int& h_lo, int& G) {
    h_lo = (g * H + KV - 1) / KV;              // ceil(g H / KV)
    G = ((g + 1) * H + KV - 1) / KV - h_lo;    // query heads with floor(h KV / H) = g
}

// Tiles of a position: `per` consecutive tiles per split (at least
// min_tiles), `nact` splits in use.
__host__ __device__ __forceinline__ void split_of(int n, int ch, int nsplit, int min_tiles, int& tiles, int& per,
                                                  int& nact) {
    tiles = (n + ch - 1) / ch;
    per = (tiles + nsplit - 1) / nsplit;
    if (per < min_tiles) per = min_tiles;
    nact = (tiles + per - 1) / per;
}

// Sequence blockIdx.z of a decode batch: its q, output, caches, split
// partials and state (the identity for a single sequence).
template <int HS>
__device__ __forceinline__ AttnParams seq_view(const AttnParams& p) {
    AttnParams v = p;
    const int b = blockIdx.z;
    v.q += (size_t)b * p.q_stride;
    v.out += (size_t)b * p.q_stride;
    v.kc += (size_t)b * p.seq_stride;
    v.vc += (size_t)b * p.seq_stride;
    v.part_ml += (size_t)b * p.n_heads * p.nsplit;
    v.part_acc += (size_t)b * p.n_heads * p.nsplit * HS;
    v.arrive += (size_t)b * p.n_kv_heads;
    v.state += b;
    return v;
}

// Output float4 c of query head h; for a decode batch whose outputs go on to
// the tiled products (out_t), also the tiled copy of sequence blockIdx.z (the
// vectors are n_heads * HS floats).
template <int HS>
__device__ __forceinline__ void put_out(const AttnParams& p, int h, int c, float4 v) {
    reinterpret_cast<float4*>(p.out)[(size_t)h * (HS / 4) + c] = v;
    if (p.out_t) reinterpret_cast<float4*>(p.out_t)[tiled_slot(blockIdx.z, h * HS + 4 * c, p.n_heads * HS)] = v;
}

__device__ __forceinline__ float4 fma4(float a, float4 v, float4 acc) {
    return make_float4(fmaf(a, v.x, acc.x), fmaf(a, v.y, acc.y), fmaf(a, v.z, acc.z), fmaf(a, v.w, acc.w));
}

// Most splits one thread of a merging block folds (the last split block
// merges its kv group only when this covers every split).
constexpr int kMaxFold = 4;

// Exact merge of the split partials of query heads h_lo .. h_lo + G - 1 into
// the output: with M = max_s m_s, out = sum_s 2^{m_s - M} acc_s /
// sum_s 2^{m_s - M} l_s.  Thread (kg, o) of the NT threads takes splits kg,
// kg + KG, ... (at most kMaxFold) of float4 output slot o: it issues all their
// loads at once, then folds them into its own running (m, l, acc); the key
// groups that hold splits are then combined through LDS the same way.
template <int HS, int NT>
__device__ void merge_group(const AttnParams& p, int h_lo, int G, int nact) {
    constexpr int H4 = HS / 4;
    __shared__ float4 acc_s[NT];
    __shared__ float m_s[NT], l_s[NT];
    const int tid = threadIdx.x;
    const int slots = G * H4;  // float4 outputs of the group
    const int KG = slots < NT ? NT / slots : 1;
    const int kgn = KG < nact ? KG : nact;  // key groups that hold a split
    for (int o0 = 0; o0 < slots; o0 += NT) {
        const int o = o0 + (slots < NT ? tid % slots : tid), kg = slots < NT ? tid / slots : 0;
        const int h = h_lo + o / H4, c = o % H4;
        float m = -INFINITY, l = 0.f;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        if (o < slots && kg < kgn) {
            const float2* ml = p.part_ml + (size_t)h * p.nsplit;
            const float4* ah = reinterpret_cast<const float4*>(p.part_acc) + (size_t)h * p.nsplit * H4 + c;
            float2 e[kMaxFold];
            float4 v[kMaxFold];
#pragma unroll
            for (int i = 0; i < kMaxFold; ++i) {  // every load in flight together (a split past nact re-reads the last)
                const int sp = min(kg + i * KG, nact - 1);
                e[i] = load_coherent(ml + sp);
                v[i] = load_coherent(ah + (size_t)sp * H4);
            }
#pragma unroll
            for (int i = 0; i < kMaxFold; ++i) {
                if (kg + i * KG >= nact) break;
                const float mn = fmaxf(m, e[i].x);
                const float r = exp2_fast(m - mn), w = exp2_fast(e[i].x - mn);  // r = 0 for the first split
                l = fmaf(l, r, e[i].y * w);
                a = fma4(w, v[i], make_float4(a.x * r, a.y * r, a.z * r, a.w * r));
                m = mn;
            }
        }
        if (kgn > 1) {
            acc_s[tid] = a;
            m_s[tid] = m;
            l_s[tid] = l;
            __syncthreads();
            if (tid < slots) {
                float M = m;
                for (int k = 1; k < kgn; ++k) M = fmaxf(M, m_s[k * slots + tid]);
                l = 0.f;
                a = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int k = 0; k < kgn; ++k) {
                    const float e = exp2_fast(m_s[k * slots + tid] - M);
                    l = fmaf(l_s[k * slots + tid], e, l);
                    a = fma4(e, acc_s[k * slots + tid], a);
                }
            }
            __syncthreads();  // the next pass reuses the LDS slots
        }
        if (o < slots && (kgn == 1 || tid < slots)) {
            const float il = 1.0f / l;
            put_out<HS>(p, h, c, make_float4(a.x * il, a.y * il, a.z * il, a.w * il));
        }
    }
}

// Called by every thread of a split block after it has stored its partial
// (coherent stores).  Each thread waits for its stores to complete before
// thread 0 counts the block's arrival with an atomic add; the block that
// brings the count to nact resets the counter for the next launch and merges
// the group, whose partials it then reads with coherent loads.  No block waits
// for another, so the grid always drains.
template <int HS, int NT>
__device__ void arrive_and_merge(const AttnParams& p, int g, int h_lo, int G, int nact) {
    __shared__ int last_s;
    wait_vector_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned before = atomicAdd(p.arrive + g, 1u);
        const int last = before + 1 == (unsigned)nact;
        if (last) atomicExch(p.arrive + g, 0u);
        last_s = last;
    }
    __syncthreads();
    if (!last_s) return;
    merge_group<HS, NT>(p, h_lo, G, nact);
}

template <int HS, int CH>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams pb) {
    const AttnParams p = seq_view<HS>(pb);
    constexpr int H4 = HS / 4;
    constexpr int KP = HS + 4;  // padded LDS row
    constexpr int NLOAD = (CH * H4 + kAttnThreads - 1) / kAttnThreads;
    constexpr int NACC = (kMaxGroup * H4 + kAttnThreads - 1) / kAttnThreads;  // float4 outputs per thread
    __shared__ float4 q_s[kMaxGroup][H4];
    __shared__ __align__(16) float k_s[CH * KP];
    __shared__ __align__(16) float v_s[CH * KP];
    __shared__ float p_s[kMaxGroup][CH];
    __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], r_s[kMaxGroup];
    __shared__ float4 red_s[kAttnThreads];

    const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = p.state->pos + 1;
    int tiles, per, nact;
    split_of(n, CH, p.nsplit, p.min_tiles, tiles, per, nact);
    if (s >= nact) return;
    const int tile0 = s * per, tile1 = min(tiles, tile0 + per);
    int h_lo, G;
    group_of(g, p.n_heads, p.n_kv_heads, h_lo, G);
    const float* kbase = p.kc + (size_t)g * HS;
    const float* vbase = p.vc + (size_t)g * HS;

    // first tile's loads, then q
    float4 kk[NLOAD], vv[NLOAD];
    auto load_tile = [&](int tile) {
        const int t0 = tile * CH, nt = min(CH, n - t0);
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int e = tid + i * kAttnThreads;
            const int t = min(e / H4, nt - 1), c = e % H4;  // rows past the tile re-read its last row
            const size_t off = (size_t)(t0 + t) * p.kv_dim + (size_t)c * 4;
            kk[i] = *reinterpret_cast<const float4*>(kbase + off);
            vv[i] = *reinterpret_cast<const float4*>(vbase + off);
        }
    };
    load_tile(tile0);
    const float4* q4 = reinterpret_cast<const float4*>(p.q);
    for (int e = tid; e < G * H4; e += kAttnThreads) q_s[e / H4][e % H4] = q4[(size_t)h_lo * H4 + e];
    if (tid < kMaxGroup) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.f;
    }

    // value-sum mapping: float4 output slot o (head o / H4, column o % H4), key group kg
    const int slots = G * H4;
    const int KG = slots < kAttnThreads ? kAttnThreads / slots : 1;
    const int kg = slots < kAttnThreads ? tid / slots : 0;
    float4 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    // score mapping: tpp threads per (head, key) pair
    const int P = G * CH;
    int tpp = 1;
    while (tpp < 16 && P * tpp * 2 <= kAttnThreads) tpp *= 2;
    const int per_pass = kAttnThreads / tpp, passes = (P + per_pass - 1) / per_pass, sub = tid % tpp;
    const float scale = kLog2e / sqrtf((float)HS);  // base-2 units

    for (int tile = tile0; tile < tile1; ++tile) {
        const int t0 = tile * CH, nt = min(CH, n - t0);
        __syncthreads();  // the previous tile is no longer read from LDS
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int e = tid + i * kAttnThreads;
            if (e < CH * H4) {
                const int t = e / H4, c = e % H4;
                *reinterpret_cast<float4*>(&k_s[t * KP + c * 4]) = kk[i];
                *reinterpret_cast<float4*>(&v_s[t * KP + c * 4]) = vv[i];
            }
        }
        __syncthreads();
        if (tile + 1 < tile1) load_tile(tile + 1);  // in flight while this tile is computed

        // scores s_t = q_h . k_t / sqrt(head_size), times log2(e)
        for (int it = 0; it < passes; ++it) {
            const int pair = it * per_pass + tid / tpp;
            const int hh = pair / CH, t = pair % CH;
            float a = 0.f;
            if (pair < P && t < nt) {
                for (int c = sub; c < H4; c += tpp)
                    a = dot4(*reinterpret_cast<const float4*>(&k_s[t * KP + c * 4]), q_s[hh][c], a);
            }
            for (int off = tpp >> 1; off > 0; off >>= 1) a += __shfl_xor(a, off);
            if (pair < P && sub == 0) p_s[hh][t] = t < nt ? a * scale : -INFINITY;
        }
        __syncthreads();

        // online softmax: new running max, weights 2^{s - m}, rescale factor
        for (int hh = wave; hh < G; hh += kAttnThreads / 64) {
            const float sc = lane < CH ? p_s[hh][lane] : -INFINITY;
            const float m_old = m_s[hh];
            const float m_new = fmaxf(m_old, wave_max(sc));
            const float e = lane < nt ? exp2_fast(sc - m_new) : 0.f;
            const float sum = wave_sum(e);
            if (lane < CH) p_s[hh][lane] = e;
            if (lane == 0) {
                const float r = exp2_fast(m_old - m_new);  // 0 on the first tile
                r_s[hh] = r;
                l_s[hh] = l_s[hh] * r + sum;
                m_s[hh] = m_new;
            }
        }
        __syncthreads();

        // value sum: acc = acc * r + sum_t e_t v_t over this thread's keys
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            const int o = slots < kAttnThreads ? tid % slots : tid + j * kAttnThreads;
            if ((slots < kAttnThreads ? kg < KG : o < slots) && (j == 0 || slots >= kAttnThreads)) {
                const int hh = o / H4, c = o % H4;
                const float r = r_s[hh];
                float4 a = make_float4(acc[j].x * r, acc[j].y * r, acc[j].z * r, acc[j].w * r);
                for (int t = kg; t < nt; t += KG) {
                    const float pw = p_s[hh][t];
                    const float4 v = *reinterpret_cast<const float4*>(&v_s[t * KP + c * 4]);
                    a = make_float4(fmaf(pw, v.x, a.x), fmaf(pw, v.y, a.y), fmaf(pw, v.z, a.z), fmaf(pw, v.w, a.w));
                }
                acc[j] = a;
            }
        }
    }

    // this split's partial: (m, l) per head and the value sum
    float4* part4 = reinterpret_cast<float4*>(p.part_acc);
    if (slots >= kAttnThreads) {
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            const int o = tid + j * kAttnThreads;
            if (o < slots) store_coherent(part4 + ((size_t)(h_lo + o / H4) * p.nsplit + s) * H4 + o % H4, acc[j]);
        }
    } else {
        red_s[tid] = acc[0];
        __syncthreads();
        if (tid < slots) {
            float4 a = acc[0];
            for (int k = 1; k < KG; ++k) {
                const float4 b = red_s[k * slots + tid];
                a = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
            }
            if (nact == 1) {  // one split holds every key: this is the output
                const float il = 1.0f / l_s[tid / H4];
                put_out<HS>(p, h_lo + tid / H4, tid % H4, make_float4(a.x * il, a.y * il, a.z * il, a.w * il));
            } else {
                store_coherent(part4 + ((size_t)(h_lo + tid / H4) * p.nsplit + s) * H4 + tid % H4, a);
            }
        }
        if (nact == 1) return;
    }
    if (nact == 1) {
        // (slots >= threads): outputs written unnormalised above; normalise in place
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            const int o = tid + j * kAttnThreads;
            if (o < slots) {
                const float il = 1.0f / l_s[o / H4];
                const float4 a = acc[j];
                put_out<HS>(p, h_lo + o / H4, o % H4, make_float4(a.x * il, a.y * il, a.z * il, a.w * il));
            }
        }
        return;
    }
    if (tid < G) store_coherent(p.part_ml + (size_t)(h_lo + tid) * p.nsplit + s, make_float2(m_s[tid], l_s[tid]));
    if (p.fuse) arrive_and_merge<HS, kAttnThreads>(p, g, h_lo, G, nact);
}

// Register-only attention for head sizes up to 128.  A key row of HS floats
// is held by LPK lanes (HS/4 float4 columns, rounded up to a power of two;
// lanes past the row re-read its last column and have q = 0 there), so a wave
// holds KPW = 64/LPK keys per load, and U such loads form a wave batch of
// KPW*U keys.  Each of the NW waves is an independent flash-decoding worker
// over its batches: the next batch is loaded while the current one is scored,
// q of every head of the group stays in registers, a score is reduced over
// its LPK lanes with DPP, every lane turns its own key's score into a weight,
// and the running max m is wave-uniform.  No LDS and no barrier in the key
// loop; the waves merge once at the end of the block.  A round of the block
// (every wave one batch) is the tile of CH = NW*KPW*U keys.
__host__ __device__ constexpr int attn_lanes_per_key(int hs) { return hs <= 16 ? 4 : hs <= 32 ? 8 : hs <= 64 ? 16 : 32; }

__device__ __forceinline__ float half_sum(float v) {  // lanes 16-31: sum of 0-31; lanes 48-63: of 32-63
    v += dpp<kQuadSwap1>(0.f, v);
    v += dpp<kQuadSwap2>(0.f, v);
    v += dpp<kRowHalfMirror>(0.f, v);
    v += dpp<kRowMirror>(0.f, v);
    v += dpp<kRowBcast15, 0xa>(0.f, v);
    return v;
}

// Sum over aligned groups of LPK <= 16 lanes, left in every lane of the group.
template <int LPK>
__device__ __forceinline__ float lane_group_sum(float v) {
    v += dpp<kQuadSwap1>(0.f, v);
    v += dpp<kQuadSwap2>(0.f, v);
    if (LPK >= 8) v += dpp<kRowHalfMirror>(0.f, v);
    if (LPK >= 16) v += dpp<kRowMirror>(0.f, v);
    return v;
}

// Block (kv head g, split s) of the register kernel.  STAGED: the tail of the
// fused q/k/v kernel, one split over every key.  q and the key and value rows
// of the current position were written by other blocks of that launch and are
// read from its stage with coherent loads; the rows before the position come
// from the cache (written by earlier launches).  The block's key loop covers
// the cached rows, and wave 0 folds the current position's key in at the end.
template <int HS, int GMAX, int U, int NW, bool STAGED>
__device__ void attend_reg(const AttnParams& p, int g, int s) {
    constexpr int H4 = HS / 4, LPK = attn_lanes_per_key(HS), KPW = 64 / LPK;
    constexpr int BK = KPW * U;  // keys of one wave batch
    constexpr int CH = NW * BK;  // keys of one round of the block
    static_assert(H4 <= LPK && LPK <= 32, "a key row within one lane group of at most half a wave");
    __shared__ float4 acc_s[NW][GMAX][H4];
    __shared__ float ms_s[NW][GMAX], ls_s[NW][GMAX], w_s[NW][GMAX], M_s[GMAX];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, sub = lane / LPK, c = lane % LPK;
    const int cc = c < H4 ? c : H4 - 1;
    int h_lo, G;
    group_of(g, p.n_heads, p.n_kv_heads, h_lo, G);

    // q does not depend on the position: its loads go out beside the state's
    float4 q[GMAX];
    float4 k_cur = make_float4(0.f, 0.f, 0.f, 0.f), v_cur = k_cur;
    if constexpr (STAGED) {
        const float4* st4 = reinterpret_cast<const float4*>(p.q);
        const int sh4 = p.stage_sh / 4;
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh)
            q[hh] = hh < G && c < H4 ? load_coherent(st4 + (size_t)(h_lo + hh) * sh4 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (wave == 0) {
            k_cur = load_coherent(st4 + (size_t)(p.n_heads + g) * sh4 + cc);
            v_cur = load_coherent(st4 + (size_t)(p.n_heads + p.n_kv_heads + g) * sh4 + cc);
        }
    } else {
        const float4* q4 = reinterpret_cast<const float4*>(p.q);
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh)
            q[hh] = hh < G && c < H4 ? q4[(size_t)(h_lo + hh) * H4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int n = p.state->pos + 1;
    int tiles, per, nact;
    split_of(n, CH, p.nsplit, p.min_tiles, tiles, per, nact);
    if (s >= nact) return;
    // this block's keys from the cache (STAGED: all but the current position's)
    const int kb = s * per * CH, ke = min(STAGED ? n - 1 : n, (s + 1) * per * CH);

    const float* kbase = p.kc + (size_t)g * HS + 4 * cc;
    const float* vbase = p.vc + (size_t)g * HS + 4 * cc;
    float4 K[U], V[U];
    auto load = [&](int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(kb + b * BK + u * KPW + sub, ke - 1);  // past the end: re-read the block's last key
            K[u] = *reinterpret_cast<const float4*>(kbase + (size_t)t * p.kv_dim);
            V[u] = *reinterpret_cast<const float4*>(vbase + (size_t)t * p.kv_dim);
        }
    };
    int b = wave;
    if (kb + b * BK < ke) load(b);

    float4 acc[GMAX];
    float m[GMAX], l[GMAX];  // m wave-uniform; l sums this lane's own keys' weights
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) {
        acc[hh] = make_float4(0.f, 0.f, 0.f, 0.f);
        m[hh] = -INFINITY;
        l[hh] = 0.f;
    }
    const float scale = kLog2e / sqrtf((float)HS);  // scores in base-2 units

    for (; kb + b * BK < ke; b += NW) {
        float4 Kc[U], Vc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Kc[u] = K[u];
            Vc[u] = V[u];
        }
        if (kb + (b + NW) * BK < ke) load(b + NW);  // in flight while this batch is scored
        const int key0 = kb + b * BK;
        // every head slot of the template is computed (a slot past the group has
        // q = 0 and is never written), so the loop has no per-head branch
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) {
            float sc[U];
            float mb = -INFINITY;
            if constexpr (LPK == 32) {
                // the two halves hold two keys; their scores become wave-uniform by readlane
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float d = half_sum(dot4(Kc[u], q[hh], 0.f));
                    const float se = key0 + 2 * u < ke
                                         ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), 31)) * scale
                                         : -INFINITY;
                    const float so = key0 + 2 * u + 1 < ke
                                         ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), 63)) * scale
                                         : -INFINITY;
                    sc[u] = sub ? so : se;
                    mb = fmaxf(mb, fmaxf(se, so));
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float d = lane_group_sum<LPK>(dot4(Kc[u], q[hh], 0.f));
                    sc[u] = key0 + u * KPW + sub < ke ? d * scale : -INFINITY;
                    mb = fmaxf(mb, sc[u]);
                }
                mb = wave_max(mb);
            }
            const float mn = fmaxf(m[hh], mb);
            const float r = exp2_fast(m[hh] - mn);  // 0 on the first batch
            float4 a = make_float4(acc[hh].x * r, acc[hh].y * r, acc[hh].z * r, acc[hh].w * r);
            float ls = l[hh] * r;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float e = exp2_fast(sc[u] - mn);
                ls += e;
                a = fma4(e, Vc[u], a);
            }
            acc[hh] = a;
            l[hh] = ls;
            m[hh] = mn;
        }
    }

    if constexpr (STAGED) {
        // the current position's key, scored by every lane group of wave 0
        // (each holds the whole row) and added by key slot 0
        if (wave == 0) {
#pragma unroll
            for (int hh = 0; hh < GMAX; ++hh) {
                float sc;
                if constexpr (LPK == 32)
                    sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(half_sum(dot4(k_cur, q[hh], 0.f))), 31));
                else
                    sc = lane_group_sum<LPK>(dot4(k_cur, q[hh], 0.f));
                sc *= scale;
                const float mn = fmaxf(m[hh], sc);
                const float r = exp2_fast(m[hh] - mn);  // 0 when no cached key came before
                const float e = sub == 0 ? exp2_fast(sc - mn) : 0.f;
                acc[hh] = fma4(e, v_cur, make_float4(acc[hh].x * r, acc[hh].y * r, acc[hh].z * r, acc[hh].w * r));
                l[hh] = fmaf(l[hh], r, e);
                m[hh] = mn;
            }
        }
    }

    // lanes c, c + LPK, ... hold the same column over different keys: add them,
    // then merge the waves through LDS
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) {
#pragma unroll
        for (int off = LPK; off < 64; off *= 2) {
            acc[hh] = make_float4(acc[hh].x + __shfl_xor(acc[hh].x, off), acc[hh].y + __shfl_xor(acc[hh].y, off),
                                  acc[hh].z + __shfl_xor(acc[hh].z, off), acc[hh].w + __shfl_xor(acc[hh].w, off));
            l[hh] += __shfl_xor(l[hh], off);
        }
        if (lane < H4) acc_s[wave][hh][lane] = acc[hh];
        if (lane == 0) {
            ms_s[wave][hh] = m[hh];
            ls_s[wave][hh] = l[hh];
        }
    }
    __syncthreads();
    if (tid < NW * GMAX) {  // each wave's weight 2^{m_w - M} (0 for a wave without keys)
        const int w = tid / GMAX, hh = tid % GMAX;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NW; ++k) M = fmaxf(M, ms_s[k][hh]);
        w_s[w][hh] = exp2_fast(ms_s[w][hh] - M);
        if (w == 0) M_s[hh] = M;
    }
    __syncthreads();
    if (tid < G * H4) {
        const int hh = tid / H4, col = tid % H4;
        float L = 0.f;
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float e = w_s[w][hh];
            L = fmaf(ls_s[w][hh], e, L);
            A = fma4(e, acc_s[w][hh][col], A);
        }
        const int h = h_lo + hh;
        if (nact == 1) {  // one split holds every key: this is the output
            const float il = 1.0f / L;
            put_out<HS>(p, h, col, make_float4(A.x * il, A.y * il, A.z * il, A.w * il));
        } else {
            store_coherent(reinterpret_cast<float4*>(p.part_acc) + ((size_t)h * p.nsplit + s) * H4 + col, A);
            if (col == 0) store_coherent(p.part_ml + (size_t)h * p.nsplit + s, make_float2(M_s[hh], L));
        }
    }
    if (nact > 1 && p.fuse) arrive_and_merge<HS, NW * 64>(p, g, h_lo, G, nact);
}

template <int HS, int GMAX, int U, int NW>
__global__ __launch_bounds__(NW * 64) void attn_reg_kernel(AttnParams pb) {
    const AttnParams p = seq_view<HS>(pb);
    attend_reg<HS, GMAX, U, NW, false>(p, blockIdx.x, blockIdx.y);
}

// The q/k/v product and the layer's attention in one launch ("run.c 逐行解讀"
// §4 steps 2a-2e; kind K_QKV_ATT).  Each block runs the q/k/v GEMV on its row
// groups, which also stores every row to the stage with coherent stores.  It
// then waits until those stores have completed and counts, per kv group, the
// rows it wrote of that group (the q rows of its query heads, its k and v
// rows) into arrive[group] with an atomic add.  The block whose add completes
// a group's (G + 2) * HS rows resets the counter for the next launch and runs
// the group's attention with all its threads (attend_reg, STAGED), reading
// the stage with coherent loads.  No block waits for another, so the grid
// always drains.  One block per kv group streams its keys: the launch serves
// short contexts.
constexpr int kMaxFusedKv = 64;   // kv heads a fused launch covers

// Key loads per lane of a wave batch: 2 for blocks of 4 waves or more (the
// q/k/v product keeps its occupancy), 4 for the narrow blocks of the small
// models' products.
constexpr int fused_u(int nt) { return nt >= 256 ? 2 : 4; }

template <int NT, int NX, int RPI, int HS, int GMAX>
__global__ __launch_bounds__(NT) void qkv_attention_kernel(GemvParams p) {
    gemv_body<NT, NX, RPI, K_QKV_ATT>(p);
    __shared__ int groups_s[kMaxFusedKv];
    __shared__ int ngroups_s;
    const int tid = threadIdx.x;
    const int u0 = (int)(((long long)blockIdx.x * p.units) / gridDim.x);
    const int u1 = (int)(((long long)(blockIdx.x + 1) * p.units) / gridDim.x);
    const int r0 = u0 * RPI, r1 = min(u1 * RPI, p.rows);  // the rows this block wrote
    const int H = p.n_heads, KV = p.n_kv_heads;
    if (tid == 0) ngroups_s = 0;
    wait_vector_memory();
    __syncthreads();
    auto overlap = [&](int a, int b) { return max(0, min(b, r1) - max(a, r0)); };
    for (int g = tid; g < KV; g += NT) {
        int h_lo, G;
        group_of(g, H, KV, h_lo, G);
        const int cnt = overlap(h_lo * HS, (h_lo + G) * HS) + overlap(p.seg1 + g * HS, p.seg1 + (g + 1) * HS) +
                        overlap(p.seg2 + g * HS, p.seg2 + (g + 1) * HS);
        if (cnt > 0) {
            const unsigned before = atomicAdd(p.arrive + g, (unsigned)cnt);
            if (before + (unsigned)cnt == (unsigned)((G + 2) * HS)) {
                atomicExch(p.arrive + g, 0u);
                groups_s[atomicAdd(&ngroups_s, 1)] = g;
            }
        }
    }
    __syncthreads();
    const int ng = ngroups_s;
    if (ng == 0) return;
    AttnParams a{};
    a.q = p.stage;
    a.kc = p.kc;
    a.vc = p.vc;
    a.out = p.att_out;
    a.state = p.state;
    a.n_heads = H;
    a.n_kv_heads = KV;
    a.kv_dim = p.kv_stride;
    a.nsplit = 1;
    a.min_tiles = 1;
    a.stage_sh = p.stage_sh;
    for (int i = 0; i < ng; ++i) {
        attend_reg<HS, GMAX, fused_u(NT), NT / 64, true>(a, groups_s[i], 0);
        __syncthreads();  // the next group reuses the attention's LDS
    }
}

// Exact merge of the split partials of query head blockIdx.x, one block per
// query head, for groups whose partials are too many for one block to fold.
// Wave 0 finds M = max_s m_s and L = sum_s 2^{m_s - M} l_s over the splits
// (lane-strided loads); then every column's float4 is summed over split
// groups, 8 loads in flight per thread, and the groups are added through LDS.
template <int HS>
__global__ __launch_bounds__(kAttnThreads) void attn_merge_kernel(AttnParams pb) {
    const AttnParams p = seq_view<HS>(pb);
    constexpr int H4 = HS / 4;
    constexpr int KG = kAttnThreads / H4;  // split groups (H4 <= 64, so at least 4)
    __shared__ float M_s, L_s;
    __shared__ float4 red_s[kAttnThreads];
    const int tid = threadIdx.x, lane = tid & 63, h = blockIdx.x;
    int tiles, per, nact;
    split_of(p.state->pos + 1, p.chunk, p.nsplit, p.min_tiles, tiles, per, nact);
    if (nact == 1) return;  // the attention kernel wrote the output itself
    const float2* ml = p.part_ml + (size_t)h * p.nsplit;
    if (tid < 64) {
        float m = -INFINITY;
        for (int sp = lane; sp < nact; sp += 64) m = fmaxf(m, ml[sp].x);
        m = wave_max(m);
        float l = 0.f;
        for (int sp = lane; sp < nact; sp += 64) {
            const float2 e = ml[sp];
            l = fmaf(e.y, exp2_fast(e.x - m), l);
        }
        l = wave_sum(l);
        if (lane == 0) {
            M_s = m;
            L_s = l;
        }
    }
    __syncthreads();
    const int c = tid % H4, kg = tid / H4;
    const float M = M_s;
    const float4* acc4 = reinterpret_cast<const float4*>(p.part_acc) + (size_t)h * p.nsplit * H4 + c;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (kg < KG) {
#pragma unroll 8
        for (int sp = kg; sp < nact; sp += KG) {
            const float wgt = exp2_fast(ml[sp].x - M);
            a = fma4(wgt, acc4[(size_t)sp * H4], a);
        }
    }
    red_s[tid] = a;
    __syncthreads();
    if (tid < H4) {
        for (int k = 1; k < KG; ++k) {
            const float4 b = red_s[k * H4 + tid];
            a = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        }
        const float il = 1.0f / L_s;
        put_out<HS>(p, h, tid, make_float4(a.x * il, a.y * il, a.z * il, a.w * il));
    }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.

struct Tpl {
    int nt, nx, rpi;
};


// Ordered by capacity nt*nx float4 (= input floats / 4).  Two groups of
// weights are live at once (the pipelined loads), so rpi*nx stays at 16 or
// below.  The q/k/v and w1/w3 kernels pair rows and use at least 2 rows per
// group.  For 1024 < n <= 4096 and 8192 < n <= 12288 (the 7B shape's
// products and its 11008-wide down projection) the shapes are the fastest of
// those timed on a whole greedy decode: 512 x 2 x 2 and 1024 x 3 x 2 (about
// 1.2% more tokens/s than 256 x 4 x 4 and 1024 x 3 x 4; 256 x 4 x 2 gave
// 0.8%, 512 x 2 x 1 and 1024 x 3 x 1 less, 1024 x 1 x 2/4 and 512 x 2 x 4
// 5-6% less).  Smaller groups and more blocks start every weight stream
// sooner.
// The narrow shapes (the tiny, stories15M- and GQA-small-shaped workloads,
// which are bound by launch latency): one or two rows per group and twice the
// threads of the first version gave 3.5% (tiny) and 3.4-4.2% more tokens/s
// than 64 x 1/2/4 x 4.
#ifndef LD_GEMV_256
#define LD_GEMV_256 {64, 1, 1}
#endif
#ifndef LD_GEMV_512
#define LD_GEMV_512 {128, 1, 2}
#endif
#ifndef LD_GEMV_1024
#define LD_GEMV_1024 {128, 2, 2}
#endif
#ifndef LD_GEMV_4096
#define LD_GEMV_4096 {512, 2, 2}
#endif
#ifndef LD_GEMV_12288
#define LD_GEMV_12288 {1024, 3, 2}
#endif
#ifndef LD_GEMV_8192
#define LD_GEMV_8192 {512, 4, 2}  // the 70B layer's 8192-wide products: +0.75% tokens/s over 256 x 8 x 2
#endif
#ifndef LD_GEMV_28672
#define LD_GEMV_28672 {512, 14, 1}
#endif
// Per-kind shapes for 1024 < n <= 4096, chosen on whole greedy decodes of the
// 7B shape with the round-robin row groups: the q/k/v product 256 x 4 x 2
// (31.9 -> 31.1 us; the same shape for wo was 11.1 -> 11.6 us), the
// classifier one row per group (84.7 -> 83.7 us).
#ifndef LD_GEMV_QKV4096
#define LD_GEMV_QKV4096 {256, 4, 2}
#endif
#ifndef LD_GEMV_CLS4096
#define LD_GEMV_CLS4096 {512, 2, 1}
#endif
// For 4096 < n <= 8192 (the 70B layer's products), the residual products take
// one row per group: wo 41.0-41.1 -> 39.8 us, 229.6-230.0 -> 230.7 tok/s
#ifndef LD_GEMV_RESID8192
#define LD_GEMV_RESID8192 {512, 4, 1}
#endif
constexpr Tpl kTpl[] = {
    LD_GEMV_256,       // n <= 256
    LD_GEMV_512,       // n <= 512
    LD_GEMV_1024,      // n <= 1024
    LD_GEMV_4096,      // n <= 4096
    LD_GEMV_8192,      // n <= 8192
    LD_GEMV_12288,     // n <= 12288
    LD_GEMV_28672,     // n <= 28672
    {512, 16, 1},      // n <= 32768
    LD_GEMV_QKV4096,   // K_QKV in place of entry 3
    LD_GEMV_CLS4096,   // K_CLS in place of entry 3
    LD_GEMV_RESID8192, // K_RESID in place of entry 4
};
constexpr int kNumTpl = sizeof(kTpl) / sizeof(kTpl[0]);
constexpr int kNumWidthTpl = 8;  // entries chosen by input width

// the entry a kind uses in place of width entry t
constexpr int kind_template(int kind, int t) {
    return t == 3 && kind == K_QKV ? 8 : t == 3 && kind == K_CLS ? 9 : t == 4 && kind == K_RESID ? 10 : t;
}

constexpr int rows_per_group(int t, int kind) {
    return (is_qkv_kind(kind) || kind == K_SWIGLU) && kTpl[t].rpi < 2 ? 2 : kTpl[t].rpi;
}

using GemvFn = void (*)(GemvParams);

template <int KIND, int T>
GemvFn gemv_fn_t() {
    return gemv_kernel<kTpl[T].nt, kTpl[T].nx, rows_per_group(T, KIND), KIND>;
}

template <int KIND>
GemvFn gemv_fn(int t) {
    switch (t) {
        case 0: return gemv_fn_t<KIND, 0>();
        case 1: return gemv_fn_t<KIND, 1>();
        case 2: return gemv_fn_t<KIND, 2>();
        case 3: return gemv_fn_t<KIND, 3>();
        case 4: return gemv_fn_t<KIND, 4>();
        case 5: return gemv_fn_t<KIND, 5>();
        case 6: return gemv_fn_t<KIND, 6>();
        case 7: return gemv_fn_t<KIND, 7>();
        case 8: return gemv_fn_t<KIND, 8>();
        case 9: return gemv_fn_t<KIND, 9>();
        case 10: return gemv_fn_t<KIND, 10>();
    }
    return nullptr;
}

GemvFn gemv_fn_kind(int kind, int t) {
    switch (kind) {
        case K_PLAIN: return gemv_fn<K_PLAIN>(t);
        case K_RESID: return gemv_fn<K_RESID>(t);
        case K_QKV: return gemv_fn<K_QKV>(t);
        case K_SWIGLU: return gemv_fn<K_SWIGLU>(t);
        case K_CLS: return gemv_fn<K_CLS>(t);
    }
    return nullptr;
}

// Batch kernel shapes: NB vectors of NX float4 per thread stay in registers,
// so NB * NX stays at 24 or below (and blocks at 512 threads, which leave a
// wave 256 registers).  Two rows per group: four cost more registers than
// the pipelined loads gain (measured on the 7B shape, 4 sequences: 4.83 ms
// per step with 2 rows per group at n <= 4096, 5.35 with 4; 512 x 2 x 2:
// 5.11; one row per group for the residual products: 4.86-4.89).
#ifndef LD_GEMVB_4096
#define LD_GEMVB_4096 {256, 4, 2}
#endif
#ifndef LD_GEMVB_12288
#define LD_GEMVB_12288 {512, 6, 2}
#endif
constexpr Tpl kTplB[] = {
    {64, 1, 4},       // n <= 256
    {256, 1, 4},      // n <= 1024
    LD_GEMVB_4096,    // n <= 4096
    {512, 4, 2},      // n <= 8192
    LD_GEMVB_12288,   // n <= 12288
};
constexpr int kNumTplB = sizeof(kTplB) / sizeof(kTplB[0]);

constexpr int rows_per_group_b(int t, int kind) {
    return (kind == K_QKV || kind == K_SWIGLU) && kTplB[t].rpi < 2 ? 2 : kTplB[t].rpi;
}

// Instances for 1, 2 and kGemvBatch vectors: a batch of one or two
// sequences does not pay for the registers and products of four.
template <int KIND, int T, int NB>
GemvFn gemv_batch_fn_t() {
    return gemv_batch_kernel<kTplB[T].nt, kTplB[T].nx, rows_per_group_b(T, KIND), KIND, NB>;
}

template <int KIND, int NB>
GemvFn gemv_batch_fn(int t) {
    switch (t) {
        case 0: return gemv_batch_fn_t<KIND, 0, NB>();
        case 1: return gemv_batch_fn_t<KIND, 1, NB>();
        case 2: return gemv_batch_fn_t<KIND, 2, NB>();
        case 3: return gemv_batch_fn_t<KIND, 3, NB>();
        case 4: return gemv_batch_fn_t<KIND, 4, NB>();
    }
    return nullptr;
}

template <int NB>
GemvFn gemv_batch_fn_nb(int kind, int t) {
    switch (kind) {
        case K_PLAIN: return gemv_batch_fn<K_PLAIN, NB>(t);
        case K_RESID: return gemv_batch_fn<K_RESID, NB>(t);
        case K_QKV: return gemv_batch_fn<K_QKV, NB>(t);
        case K_SWIGLU: return gemv_batch_fn<K_SWIGLU, NB>(t);
    }
    return nullptr;
}

// nb: the batch's vectors (1, 2, or up to kGemvBatch)
GemvFn gemv_batch_fn_kind(int kind, int t, int nb = kGemvBatch) {
    return nb <= 1 ? gemv_batch_fn_nb<1>(kind, t) : nb <= 2 ? gemv_batch_fn_nb<2>(kind, t) : gemv_batch_fn_nb<kGemvBatch>(kind, t);
}

// The fused q/k/v + attention kernels: GEMV shapes up to n = 4096 (kTpl[0..3]),
// head sizes 16 / 32 / 48 / 64 / 128, one or two query heads per kv head.
constexpr int kFusedTpl = 4;

bool fused_head_size(int hs) { return hs == 16 || hs == 32 || hs == 48 || hs == 64 || hs == 128; }

template <int T, int HS, int GMAX>
GemvFn qkv_att_fn_t() {
    return qkv_attention_kernel<kTpl[T].nt, kTpl[T].nx, rows_per_group(T, K_QKV_ATT), HS, GMAX>;
}

template <int T, int HS>
GemvFn qkv_att_fn_g(int gmax) {
    return gmax <= 1 ? qkv_att_fn_t<T, HS, 1>() : qkv_att_fn_t<T, HS, 2>();
}

template <int T>
GemvFn qkv_att_fn_h(int hs, int gmax) {
    switch (hs) {
        case 16: return qkv_att_fn_g<T, 16>(gmax);
        case 32: return qkv_att_fn_g<T, 32>(gmax);
        case 48: return qkv_att_fn_g<T, 48>(gmax);
        case 64: return qkv_att_fn_g<T, 64>(gmax);
        case 128: return qkv_att_fn_g<T, 128>(gmax);
    }
    return nullptr;
}

GemvFn qkv_att_fn(int t, int hs, int gmax) {
    if (gmax > 2) return nullptr;
    switch (t) {
        case 0: return qkv_att_fn_h<0>(hs, gmax);
        case 1: return qkv_att_fn_h<1>(hs, gmax);
        case 2: return qkv_att_fn_h<2>(hs, gmax);
        case 3: return qkv_att_fn_h<3>(hs, gmax);
    }
    return nullptr;
}

int template_for(const GemvPlan& pl) {
    if (pl.nb) {
        for (int t = 0; t < kNumTplB; ++t)
            if (kTplB[t].nt == pl.nt && kTplB[t].nx == pl.nx && rows_per_group_b(t, pl.kind) == pl.rpi) return t;
        return -1;
    }
    for (int t = 0; t < kNumTpl; ++t)
        if (kTpl[t].nt == pl.nt && kTpl[t].nx == pl.nx && rows_per_group(t, pl.kind) == pl.rpi) return t;
    return -1;
}

// Largest divisor of `units` in [lo, hi], or 0.
int divisor_in(int units, int lo, int hi) {
    for (int g = hi; g >= lo && g >= 1; --g)
        if (units % g == 0) return g;
    return 0;
}

}  // namespace

hipError_t gemv_plan(int kind, int rows, int n, GemvPlan* plan) {
    if (n <= 0 || rows <= 0 || (n & 3) || n > kMaxN) return hipErrorInvalidValue;
    if (kind == K_QKV_ATT) return hipErrorInvalidValue;  // qkv_attention_plan
    const int n4 = n / 4;
    int t = 0;
    while (t < kNumWidthTpl && kTpl[t].nt * kTpl[t].nx < n4) ++t;
    if (t == kNumWidthTpl) return hipErrorInvalidValue;
    t = kind_template(kind, t);
    const Tpl tp = kTpl[t];
    const int rpi = rows_per_group(t, kind);
    const int per_iter = kind == K_SWIGLU ? rpi / 2 : rpi;
    plan->kind = kind;
    plan->nt = tp.nt;
    plan->nx = tp.nx;
    plan->rpi = rpi;
    plan->nb = 0;
    plan->units = (rows + per_iter - 1) / per_iter;

    int dev = 0, cus = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_fn_kind(kind, t), tp.nt, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    // One resident wave of blocks, every slot filled: each block streams an
    // even share of the row groups, to within one group.  (A grid chosen to
    // divide the groups exactly, which can leave a third of the slots empty,
    // was 0.3% slower on the 7B shape's decode now that groups are small.)
    const int slots = cus * occ;
    plan->grid = plan->units <= slots ? plan->units : slots;
    return hipSuccess;
}

hipError_t gemv_plan_batch(int kind, int rows, int n, GemvPlan* plan) {
    if (n <= 0 || rows <= 0 || (n & 3)) return hipErrorInvalidValue;
    if (kind != K_PLAIN && kind != K_RESID && kind != K_QKV && kind != K_SWIGLU) return hipErrorInvalidValue;
    const int n4 = n / 4;
    int t = 0;
    while (t < kNumTplB && kTplB[t].nt * kTplB[t].nx < n4) ++t;
    if (t == kNumTplB) return hipErrorInvalidValue;
    const Tpl tp = kTplB[t];
    const int rpi = rows_per_group_b(t, kind);
    const int per_iter = kind == K_SWIGLU ? rpi / 2 : rpi;
    plan->kind = kind;
    plan->nt = tp.nt;
    plan->nx = tp.nx;
    plan->rpi = rpi;
    plan->nb = kGemvBatch;
    plan->units = (rows + per_iter - 1) / per_iter;
    int dev = 0, cus = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // one grid per instance (kGemvBatch, 1 and 2 vectors): each fills its own slots
    for (int i = 0; i < 3; ++i) {
        const int nbi = i == 0 ? kGemvBatch : i;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_batch_fn_kind(kind, t, nbi), tp.nt, 0);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
        const int slots = cus * occ;
        int grid;
        if (plan->units <= slots) {
            grid = plan->units;
        } else {
            const int even = divisor_in(plan->units, (slots + 1) / 2, slots);
            grid = even ? even : slots;
        }
        if (i == 0)
            plan->grid = grid;
        else
            plan->grid_nb[i - 1] = grid;
    }
    return hipSuccess;
}

bool qkv_attention_supported(int n, int head_size, int n_heads, int n_kv_heads) {
    if (n <= 0 || (n & 3) || head_size <= 0 || n_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > n_heads) return false;
    if (n_kv_heads > kMaxFusedKv || !fused_head_size(head_size)) return false;
    const int group = (n_heads + n_kv_heads - 1) / n_kv_heads;
    return group <= 2 && n <= kTpl[kFusedTpl - 1].nt * kTpl[kFusedTpl - 1].nx * 4;
}

// Measured on whole decode steps (kernel events, positions 0-15): the fused
// launch took 7.5 against 4.5 + 4.3 us per layer for the tiny shape (dim 64,
// single-wave q/k/v blocks), but 10.4 against 4.7 + 4.3 us (stories15M
// shape), 9.5 against 4.3 + 4.3 (GQA-small) and 39.2 against 31.8 + 4.2 (7B
// shape).  The hand-off (stores written through to memory and waited for, the
// arrival count, the coherent loads of the last block) costs more than the
// kernel boundary it replaces wherever the product's blocks have more than one
// wave, so the decode step uses it only where they have one.
bool qkv_attention_pays(int n) { return n > 0 && n <= kTpl[0].nt * kTpl[0].nx * 4; }

int qkv_attention_stage_stride(int head_size) { return (head_size + 63) / 64 * 64; }

size_t qkv_attention_stage_floats(int head_size, int n_heads, int n_kv_heads) {
    return (size_t)(n_heads + 2 * n_kv_heads) * (size_t)qkv_attention_stage_stride(head_size);
}

hipError_t qkv_attention_plan(int n, int head_size, int n_heads, int n_kv_heads, GemvPlan* plan) {
    if (!qkv_attention_supported(n, head_size, n_heads, n_kv_heads)) return hipErrorInvalidValue;
    const int n4 = n / 4;
    int t = 0;
    while (kTpl[t].nt * kTpl[t].nx < n4) ++t;
    const int rows = (n_heads + 2 * n_kv_heads) * head_size;
    const int rpi = rows_per_group(t, K_QKV_ATT);
    plan->kind = K_QKV_ATT;
    plan->nt = kTpl[t].nt;
    plan->nx = kTpl[t].nx;
    plan->rpi = rpi;
    plan->nb = 0;
    plan->units = (rows + rpi - 1) / rpi;
    const int group = (n_heads + n_kv_heads - 1) / n_kv_heads;
    int dev = 0, cus = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, qkv_att_fn(t, head_size, group), plan->nt, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    const int slots = cus * occ;
    plan->grid = plan->units <= slots ? plan->units : slots;
    return hipSuccess;
}

hipError_t qkv_attention_launch(const GemvPlan& plan, const GemvParams& p0, hipStream_t s, hipEvent_t start,
                                hipEvent_t stop) {
    const int t = template_for(plan);
    if (plan.kind != K_QKV_ATT || t < 0 || t >= kFusedTpl) return hipErrorInvalidValue;
    GemvParams p = p0;
    p.units = plan.units;
    if (!p.stage || !p.arrive || !p.att_out || p.stage_sh < p.head_size || (p.stage_sh & 63)) return hipErrorInvalidValue;
    if (!qkv_attention_supported(p.n, p.head_size, p.n_heads, p.n_kv_heads) ||
        p.rows != (p.n_heads + 2 * p.n_kv_heads) * p.head_size || p.seg1 != p.n_heads * p.head_size ||
        p.seg2 != p.seg1 + p.n_kv_heads * p.head_size)
        return hipErrorInvalidValue;
    const int group = (p.n_heads + p.n_kv_heads - 1) / p.n_kv_heads;
    GemvFn fn = qkv_att_fn(t, p.head_size, group);
    if (!fn) return hipErrorInvalidValue;
    if (start || stop)
        hipExtLaunchKernelGGL(fn, dim3(plan.grid), dim3(plan.nt), 0, s, start, stop, 0, p);
    else
        hipLaunchKernelGGL(fn, dim3(plan.grid), dim3(plan.nt), 0, s, p);
    return hipGetLastError();
}

hipError_t tile_weights_launch(int kind, const float* w0, const float* w1, const float* w2, int seg1, int seg2,
                               const float* gain, int rows, int k, float* dst, hipStream_t s) {
    if (rows <= 0 || k <= 0 || rows % 16 || k % 16 || !w0 || !dst) return hipErrorInvalidValue;
    if ((kind == K_QKV && (!w1 || !w2)) || (kind == K_SWIGLU && !w1)) return hipErrorInvalidValue;
    const size_t n4 = (size_t)rows * (size_t)k / 4;
    const size_t blocks = (n4 + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(tile_weights_kernel, dim3(grid), dim3(256), 0, s, kind, w0, w1, w2, seg1, seg2, gain, rows, k,
                       reinterpret_cast<float4*>(dst));
    return hipGetLastError();
}

// Tiled product shapes, in this order:
// - more row tiles than CUs (tiled_one_block): one block per CU holding
//   ceil(row tiles / CUs) row tiles, so each activation load serves that many
//   tiles and no CU runs two blocks (7B shape: q/k/v 256 blocks of 3 tiles,
//   w1/w3 230 of 6, the classifier 250 of 8);
// - otherwise, without the RMSNorm (wo and w2): K split over blocks
//   (tiled_split);
// - otherwise (the narrow products of small models): tiled_shape, the row
//   tiles per block whose busiest CU is fullest.
// Against the earlier rule (tiled_shape for every product: w1/w3 688 blocks of
// two tiles, wo and w2 256 of one), the first two took the 7B-shaped batch
// step of 8 / 16 / 32 / 64 sequences from 4.83 / 4.88 / 6.47 / 9.74 to 4.59 /
// 4.62 / 5.25 / 8.39 ms.  A probe of the w1/w3 product alone at 64 sequences:
// 171 us with 688 blocks of two tiles, 146 with 459 of three, 116 with 230 of
// six.

int cu_count() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
            cus = c;
        else
            return 256;
    }
    return cus;
}

// fraction of the busiest CU's slots the blocks fill, in thousandths
int tiled_balance(int blocks, int cus) {
    const int per = (blocks + cus - 1) / cus;
    return (int)(1000LL * blocks / ((long long)per * cus));
}

// Up to 16 sequences (one plane): 8 waves, 4 steps in flight, 1 to 4 row
// tiles.  17-32 (two planes): 8 waves, 4 steps, 1 or 2 row tiles (registers
// and LDS hold row tiles x planes partial tiles).  33-48 and 49-64 (three and
// four planes): 4 waves, 2 steps, 1 to 4 row tiles.  Before each step's slot
// was refilled as soon as its products were issued, four planes ran at
// 13.5-13.9 ms per 7B-shaped step against 10.8-11.1 ms with the split-K
// products; with the refill, 9.8 against 10.7.
template <int KIND, int NW, int D, int NP, int RT>
void tiled_go(const TiledParams& p, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((tiled_kernel<NW, RT, D, KIND, NP>), dim3(blocks), dim3(NW * 64), 0, s, p);
}

#ifndef LD_TILED_OB
#define LD_TILED_OB 1
#endif
#ifndef LD_TILED_OB_NW1
#define LD_TILED_OB_NW1 8
#endif
#ifndef LD_TILED_OB_D1
#define LD_TILED_OB_D1 2
#endif
#ifndef LD_TILED_OB_NW2
#define LD_TILED_OB_NW2 4
#endif
#ifndef LD_TILED_OB_D2
#define LD_TILED_OB_D2 2
#endif
#ifndef LD_TILED_OB_NW4
#define LD_TILED_OB_NW4 4
#endif
#ifndef LD_TILED_OB_D4
#define LD_TILED_OB_D4 2
#endif
// K split where the row tiles do not outnumber the CUs (wo and w2; not with
// the RMSNorm): KS row tiles per block and K in KS parts, so there are about
// as many blocks as before and each activation load serves KS row tiles.  KS
// is 2 for one plane and 4 for more (7B shape, 8 / 16 / 32 / 64 sequences:
// without the split 4.64 / 4.66 / 5.49 / 8.78 ms per step, KS 2 4.59 / 4.62 /
// 5.50 / 8.39, KS 4 4.73 / 4.76 / 5.25-5.27 / 8.40-8.41).
#ifndef LD_TILED_KS1
#define LD_TILED_KS1 2
#endif
#ifndef LD_TILED_KS
#define LD_TILED_KS 4
#endif
constexpr int kTiledKsMax = 4;
template <int KIND, int NP>
bool tiled_split(const TiledParams& p, hipStream_t s) {
    constexpr int KS = NP == 1 ? LD_TILED_KS1 : LD_TILED_KS, RT = KS;
    if constexpr (KS <= 1) return false;
    static_assert(KS <= kTiledKsMax, "workspace");
    // (three or four planes: 8 waves 3-5% slower, 3 steps in flight 0.5%)
    constexpr int NW = NP == 1 ? LD_TILED_OB_NW1 : NP == 2 ? LD_TILED_OB_NW2 : LD_TILED_OB_NW4;
    constexpr int D = NP == 1 ? LD_TILED_OB_D1 : NP == 2 ? LD_TILED_OB_D2 : 2;
    const int tiles = p.rows / 16, cus = cu_count();
    const int groups = (tiles + RT - 1) / RT;
    if (p.norm || !p.part || !p.arrive || tiles > cus || (p.k >> 4) < KS * NW) return false;
    if ((size_t)groups * KS * RT * NP * 256 > p.part_floats || groups > tiled_arrive_count(cus)) return false;
    hipLaunchKernelGGL((tiled_kernel<NW, RT, D, KIND, NP, KS>), dim3(groups * KS), dim3(NW * 64), 0, s, p);
    return true;
}

size_t tiled_part_floats(int cus) { return (size_t)cus * kTiledKsMax * 4 * 256; }
int tiled_arrive_count(int cus) { return cus; }

template <int KIND, int NW, int D, int NP, int RT_MAX>
void tiled_shape(const TiledParams& p, hipStream_t s) {
    const int tiles = p.rows / 16, cus = cu_count();
    int rt = 1, best = tiled_balance(tiles, cus);
    for (int r = 2; r <= RT_MAX; ++r)
        if (tiles % r == 0 && tiles / r >= cus && tiled_balance(tiles / r, cus) >= best) {
            rt = r;
            best = tiled_balance(tiles / r, cus);
        }
    switch (rt) {
        case 4: if constexpr (RT_MAX >= 4) tiled_go<KIND, NW, D, NP, 4>(p, tiles / 4, s); break;
        case 3: if constexpr (RT_MAX >= 3) tiled_go<KIND, NW, D, NP, 3>(p, tiles / 3, s); break;
        case 2: tiled_go<KIND, NW, D, NP, 2>(p, tiles / 2, s); break;
        default:
            // three or four planes with one block per CU at most (wo and w2):
            // 8 waves and 8 steps in flight instead of 4 and 2 (7B shape, 40 /
            // 64 sequences: 8.07 / 9.78 -> 7.72 / 9.63 ms per step; for one or
            // two planes the same change was 1-2% slower)
            if (tiled_split<KIND, NP>(p, s)) break;
            if constexpr (NP >= 3) {
                if (tiles <= cus) {
                    tiled_go<KIND, 8, 8, NP, 1>(p, tiles, s);
                    break;
                }
            }
            tiled_go<KIND, NW, D, NP, 1>(p, tiles, s);
            break;
    }
}

// One block per CU holding ceil(row tiles / CUs) row tiles (rounded up to 2,
// 3, 4, 6 or 8; the last block's surplus tiles re-read the last tile and
// store nothing).  Returns false where every row tile has a CU of its own.
template <int KIND, int NW, int D, int NP>
bool tiled_one_block(const TiledParams& p, hipStream_t s) {
    const int tiles = p.rows / 16, cus = cu_count();
    const int need = (tiles + cus - 1) / cus;
    if (need <= 1) return false;
    const int rt = need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 6 ? 6 : 8;
    // (a block on every CU instead, the row tiles shared out evenly, need or
    // need - 1 per block, was 1.5-2% slower for one plane, 0-2% for more)
    const int blocks = (tiles + rt - 1) / rt;
    switch (rt) {
        case 2: tiled_go<KIND, NW, D, NP, 2>(p, blocks, s); break;
        case 3: tiled_go<KIND, NW, D, NP, 3>(p, blocks, s); break;
        case 4: tiled_go<KIND, NW, D, NP, 4>(p, blocks, s); break;
        case 6: tiled_go<KIND, NW, D, NP, 6>(p, blocks, s); break;
        default: tiled_go<KIND, NW, (D < 2 ? D : 2), NP, 8>(p, blocks, s); break;
    }
    return true;
}

template <int KIND>
void tiled_dispatch(const TiledParams& p, hipStream_t s) {
#if LD_TILED_OB
    if (p.nb <= 16) {
        if (tiled_one_block<KIND, LD_TILED_OB_NW1, LD_TILED_OB_D1, 1>(p, s)) return;
    } else if (kTiledBatch <= 32 || p.nb <= 32) {
        if (tiled_one_block<KIND, LD_TILED_OB_NW2, LD_TILED_OB_D2, 2>(p, s)) return;
    }
#if LD_TILED_BATCH > 32
    else if (p.nb <= 48) {
        if (tiled_one_block<KIND, LD_TILED_OB_NW4, LD_TILED_OB_D4, 3>(p, s)) return;
    } else {
        if (tiled_one_block<KIND, LD_TILED_OB_NW4, LD_TILED_OB_D4, 4>(p, s)) return;
    }
#endif
#endif
    if (p.nb <= 16)
        tiled_shape<KIND, LD_TILED_NW1, LD_TILED_D1, 1, 4>(p, s);
    else if (kTiledBatch <= 32 || p.nb <= 32)
        tiled_shape<KIND, LD_TILED_NW2, LD_TILED_D2, 2, 2>(p, s);
#if LD_TILED_BATCH > 32
    else if (p.nb <= 48)
        tiled_shape<KIND, LD_TILED_NW4, LD_TILED_D4, 3, LD_TILED_RT4>(p, s);
    else
        tiled_shape<KIND, LD_TILED_NW4, LD_TILED_D4, 4, LD_TILED_RT4>(p, s);
#endif
}

hipError_t tiled_launch(int kind, const TiledParams& p, hipStream_t s) {
    if (!p.w || !p.x || p.nb < 1 || p.nb > kTiledBatch || p.k <= 0 || p.k % 16 || p.rows <= 0 || p.rows % 16)
        return hipErrorInvalidValue;
    switch (kind) {
        case K_PLAIN:
            if (!p.out || p.ldo % 4) return hipErrorInvalidValue;
            tiled_dispatch<K_PLAIN>(p, s);
            break;
        case K_RESID:
            if (!p.x_resid || p.ldr % 4) return hipErrorInvalidValue;
            tiled_dispatch<K_RESID>(p, s);
            break;
        case K_SWIGLU:
            if (!p.out_t || p.rows % 32) return hipErrorInvalidValue;
            tiled_dispatch<K_SWIGLU>(p, s);
            break;
        case K_QKV:
            if (!p.out || !p.kc || !p.vc || !p.rope || !p.row_state || p.head_size % 4 || p.seg1 % 4 || p.seg2 % 4 ||
                p.ldo % 4 || p.kv_stride % 4 || p.seq_stride % 4)
                return hipErrorInvalidValue;
            tiled_dispatch<K_QKV>(p, s);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t gemv_launch(const GemvPlan& plan, const GemvParams& p0, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    if (plan.kind == K_QKV_ATT) return qkv_attention_launch(plan, p0, s, start, stop);
    const int t = template_for(plan);
    if (t < 0) return hipErrorInvalidValue;
    GemvParams p = p0;
    p.units = plan.units;
    if (plan.nb) {
        if (p.nb < 1 || p.nb > plan.nb) return hipErrorInvalidValue;
        const int grid = p.nb <= 2 && plan.grid_nb[p.nb - 1] > 0 ? plan.grid_nb[p.nb - 1] : plan.grid;
        hipLaunchKernelGGL(gemv_batch_fn_kind(plan.kind, t, p.nb), dim3(grid), dim3(plan.nt), 0, s, p);
    } else if (start || stop) {
        // events taken by the dispatch itself: they bracket the kernel's execution
        hipExtLaunchKernelGGL(gemv_fn_kind(plan.kind, t), dim3(plan.grid), dim3(plan.nt), 0, s, start, stop, 0, p);
    } else {
        hipLaunchKernelGGL(gemv_fn_kind(plan.kind, t), dim3(plan.grid), dim3(plan.nt), 0, s, p);
    }
    return hipGetLastError();
}

// ---- attention launch shapes ----
// Head sizes up to 128 take the register kernel; its instance follows the
// query heads per kv head: one or two heads with 4 key loads per wave batch,
// four or eight heads with 2 (registers grow with the heads).  Head size 256
// takes the LDS-staged kernel (16-key tiles).
//
// Blocks have 4 waves where the grid is large.  Where 4-wave blocks would
// make at most kSmallGrid blocks (few kv heads, a short context: the small
// models), a block has 16 waves (8 for eight heads per kv head, whose merge
// slots would not fit 16), so the few blocks cover their keys in fewer rounds.
//
// A split takes at least kSplitBytes of keys and values: the keys of one
// block stream at a few tens of GB/s (one compute unit's share), so a split
// of that size costs about what merging one more split costs.  The grid aims
// at about kAttnBlocks blocks at the longest context (two per compute unit).
constexpr int kSplitBytes = 64 << 10;
constexpr int kAttnBlocks = 512;
constexpr int kSmallGrid = 64;

struct AttnShape {
    int reg;        // 1: register kernel
    int gmax, u, nw;
    int chunk;      // keys per tile (one round of the block)
    int min_tiles;  // fewest tiles of a split
};

AttnShape attn_shape(int hs, int group, int waves) {
    AttnShape a{};
    if (hs <= 128) {
        a.reg = 1;
        a.gmax = group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8;
        a.u = a.gmax <= 2 ? 4 : 2;
        a.nw = waves <= 4 ? 4 : a.gmax <= 4 ? 16 : 8;
        a.chunk = a.nw * (64 / attn_lanes_per_key(hs)) * a.u;
    } else {
        a.nw = kAttnThreads / 64;
        a.chunk = 16;
    }
    const int keys = (kSplitBytes + 8 * hs - 1) / (8 * hs);  // keys whose K and V rows of one head fill a split
    a.min_tiles = (keys + a.chunk - 1) / a.chunk;
    if (a.min_tiles < 1) a.min_tiles = 1;
    return a;
}

int attn_chunk(int hs) {
    switch (hs) {
        case 16: case 32: case 48: case 64: case 80: case 96: case 128: case 256: return attn_shape(hs, 1, 4).chunk;
    }
    return 0;
}

// Whether the last split block of a kv group merges the group's partials:
// when each thread of that block folds at most kMaxFold splits (the merge
// launch costs more than such a tail).  Larger groups of partials go to the
// merge kernel.
bool attn_fused(int hs, int n_heads, int n_kv_heads, int nsplit, int waves) {
    const int group = (n_heads + n_kv_heads - 1) / n_kv_heads;
    const int nt = attn_shape(hs, group, waves).nw * 64;
    const int slots = group * (hs / 4), kg = slots < nt ? nt / slots : 1;
    return nsplit > 1 && (nsplit + kg - 1) / kg <= kMaxFold;
}

#ifndef LD_ATTN_ONE_BLOCK_BYTES
#define LD_ATTN_ONE_BLOCK_BYTES (128 << 10)
#endif

int splits_for(int hs, int seq_len, int n_heads, int n_kv_heads, int waves) {
    const int group = (n_heads + n_kv_heads - 1) / n_kv_heads;
    const AttnShape a = attn_shape(hs, group, waves);
    const int tiles = (seq_len + a.chunk - 1) / a.chunk;
    const int most = (tiles + a.min_tiles - 1) / a.min_tiles;
    int want = (kAttnBlocks + n_kv_heads - 1) / n_kv_heads;
    if (want > most) want = most;
    if (want < 1) want = 1;
    // where the partials would need the merge launch (a few us even with
    // nothing to do) and a kv head's whole cache fits one block, one block per
    // kv head serves it
    if (want > 1 && !attn_fused(hs, n_heads, n_kv_heads, want, waves) &&
        (long long)seq_len * hs * 2 * (long long)sizeof(float) <= LD_ATTN_ONE_BLOCK_BYTES)
        return 1;
    return want;
}

int attn_waves(int hs, int seq_len, int n_heads, int n_kv_heads) {
    if (hs > 128) return kAttnThreads / 64;
    return n_kv_heads * splits_for(hs, seq_len, n_heads, n_kv_heads, 4) <= kSmallGrid ? 16 : 4;
}

int attn_splits(int hs, int seq_len, int n_heads, int n_kv_heads) {
    if (!attn_chunk(hs)) return 0;
    return splits_for(hs, seq_len, n_heads, n_kv_heads, attn_waves(hs, seq_len, n_heads, n_kv_heads));
}

// Splits of a decode batch's attention: the batch brings its own blocks, so
// about kAttnBlocks blocks over all sequences' kv heads.  A split grid sized
// for one sequence would launch tens of thousands of blocks for a large
// batch, and at a short context nearly all of them return at once, which
// cost more than the attention (7B shape, 64 sequences at positions 0-31:
// 26 us per layer with 16 splits).
int attn_batch_splits(int nsplit, int n_kv_heads, int batch) {
    const long long per = (long long)n_kv_heads * (batch > 1 ? batch : 1);
    const int want = (int)((kAttnBlocks + per - 1) / per);
    return want < 1 ? 1 : want < nsplit ? want : nsplit;
}

// Launch one attention kernel (and the merge after it): with events, through
// hipExtLaunchKernelGGL so that `start` is taken by the attention kernel's own
// dispatch and `stop` by the last kernel's, bracketing their execution alone.
template <class K>
void attn_dispatch(K kernel, dim3 grid, int threads, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                   const AttnParams& p) {
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, start, stop, 0, p);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, p);
}

template <int HS, int NW>
void attn_reg_dispatch_nw(int gmax, dim3 grid, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                          const AttnParams& p) {
    switch (gmax) {
        case 1: attn_dispatch(attn_reg_kernel<HS, 1, 4, NW>, grid, NW * 64, s, start, stop, p); break;
        case 2: attn_dispatch(attn_reg_kernel<HS, 2, 4, NW>, grid, NW * 64, s, start, stop, p); break;
        default: attn_dispatch(attn_reg_kernel<HS, 4, 2, NW>, grid, NW * 64, s, start, stop, p); break;
    }
}

template <int HS>
void attn_reg_dispatch(const AttnShape& a, dim3 grid, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                       const AttnParams& p) {
    if (a.gmax == 8) {
        if (a.nw == 4)
            attn_dispatch(attn_reg_kernel<HS, 8, 2, 4>, grid, 256, s, start, stop, p);
        else
            attn_dispatch(attn_reg_kernel<HS, 8, 2, 8>, grid, 512, s, start, stop, p);
    } else if (a.nw == 4) {
        attn_reg_dispatch_nw<HS, 4>(a.gmax, grid, s, start, stop, p);
    } else {
        attn_reg_dispatch_nw<HS, 16>(a.gmax, grid, s, start, stop, p);
    }
}

hipError_t attn_launch(int hs, const AttnParams& p0, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    AttnParams p = p0;
    const int group = (p.n_heads + p.n_kv_heads - 1) / p.n_kv_heads;
    if (group > kMaxGroup || p.nsplit < 1) return hipErrorInvalidValue;
    const int waves = p.waves > 0 ? p.waves : 4;
    const AttnShape a = attn_shape(hs, group, waves);
    p.chunk = a.chunk;
    p.min_tiles = a.min_tiles;
    const unsigned nb = p.batch > 1 ? (unsigned)p.batch : 1u;
    const dim3 grid(p.n_kv_heads, p.nsplit, nb), mgrid(p.n_heads, 1, nb);
    p.fuse = attn_fused(hs, p.n_heads, p.n_kv_heads, p.nsplit, waves);
    if (p.fuse && !p.arrive) return hipErrorInvalidValue;  // split blocks count their arrivals there
    const bool merge = p.nsplit > 1 && !p.fuse;
    hipEvent_t stop1 = merge ? nullptr : stop;  // the attention kernel's own stop event when nothing follows it
    switch (hs) {
#define LD_ATTN_REG_CASE(HS)                                                                            \
    case HS:                                                                                            \
        attn_reg_dispatch<HS>(a, grid, s, start, stop1, p);                                             \
        if (merge) attn_dispatch(attn_merge_kernel<HS>, mgrid, kAttnThreads, s, nullptr, stop, p);       \
        break;
        LD_ATTN_REG_CASE(16)
        LD_ATTN_REG_CASE(32)
        LD_ATTN_REG_CASE(48)
        LD_ATTN_REG_CASE(64)
        LD_ATTN_REG_CASE(80)
        LD_ATTN_REG_CASE(96)
        LD_ATTN_REG_CASE(128)
#undef LD_ATTN_REG_CASE
        case 256:
            attn_dispatch(attn_kernel<256, 16>, grid, kAttnThreads, s, start, stop1, p);
            if (merge) attn_dispatch(attn_merge_kernel<256>, mgrid, kAttnThreads, s, nullptr, stop, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t embed_state_launch(const float* emb, const StepState* st, int batch, int dim, float* x, hipStream_t s,
                              float* xt) {
    if (xt && (batch > kTiledBatch || dim % 16)) return hipErrorInvalidValue;  // (tiled_slot's planes)
    hipLaunchKernelGGL(embed_state_kernel, dim3(batch), dim3(256), 0, s, emb, st, dim, x, xt);
    return hipGetLastError();
}

hipError_t argmax_rows_launch(const float* logits, int batch, int n, StepState* st, int32_t* tokens_out,
                              int tokens_stride, hipStream_t s) {
    hipLaunchKernelGGL(argmax_rows_kernel, dim3(batch), dim3(kRowsThreads), 0, s, logits, n, st, tokens_out,
                       tokens_stride);
    return hipGetLastError();
}

hipError_t set_control_launch(GenControl* dst, const GenControl& c, hipStream_t s) {
    hipLaunchKernelGGL(set_control_kernel, dim3(1), dim3(1), 0, s, dst, c);
    return hipGetLastError();
}

hipError_t attn_op_init_launch(StepState* st, int pos, unsigned* arrive, int n_kv_heads, hipStream_t s) {
    hipLaunchKernelGGL(attn_op_init_kernel, dim3(1), dim3(256), 0, s, st, pos, arrive, n_kv_heads);
    return hipGetLastError();
}

hipError_t set_state_launch(StepState* st, int token, int pos, hipStream_t s) {
    hipLaunchKernelGGL(set_state_kernel, dim3(1), dim3(1), 0, s, st, token, pos);
    return hipGetLastError();
}

int argmax_blocks(int n) {
    int b = (n + kArgmaxThreads * 8 - 1) / (kArgmaxThreads * 8);
    return b < 1 ? 1 : (b > 1024 ? 1024 : b);
}

hipError_t argmax_partial_launch(const float* v, int n, float2* best, int nblocks, hipStream_t s) {
    hipLaunchKernelGGL(argmax_partial_kernel, dim3(nblocks), dim3(kArgmaxThreads), 0, s, v, n, best);
    return hipGetLastError();
}

// The smallest block whose NT threads of E tokens hold the vocabulary: every
// pass of a draw is a block-wide sum, whose cost grows with the waves, and the
// index-order walk takes log2(E) of them.  1024 threads of 32 tokens hold up
// to kMaxSampleVocab; a larger vocabulary is only ever chosen from greedily
// (the kernel checks).
hipError_t next_token_launch(const NextTokenParams& p, hipStream_t s) {
    static_assert(kMaxSampleVocab == 1024 * 32, "sampler register layout");
    if (p.n <= 256)
        hipLaunchKernelGGL((next_token_kernel<256, 1>), dim3(1), dim3(256), 0, s, p);
    else if (p.n <= 1024 * 8)
        hipLaunchKernelGGL((next_token_kernel<1024, 8>), dim3(1), dim3(1024), 0, s, p);
    else
        hipLaunchKernelGGL((next_token_kernel<1024, 32>), dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

hipError_t stream_read_launch(const void* src, size_t bytes, float* sums, hipStream_t s) {
    const long long n4 = (long long)(bytes / 16);
    const long long per = (n4 + kStreamReadBlocks - 1) / kStreamReadBlocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(kStreamThreads), 0, s,
                       static_cast<const float4*>(src), n4, per, sums);
    return hipGetLastError();
}

}  // namespace ld
