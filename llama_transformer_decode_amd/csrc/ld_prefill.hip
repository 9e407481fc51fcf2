// ld_prefill.hip -- gfx950 (CDNA4) kernels of batched prompt prefill: the
// decode step of the "run.c 逐行解讀" page (§4 forward()) applied to T
// consecutive prompt tokens at once, as the R/Keras page's call_with_cache
// does for a whole prompt under a causal mask.  With T tokens every weight is
// used T times, so the projections are dense fp32 contractions
// (2 flops per weight per token) and run on the matrix cores:
//
//   gemm_kernel     C(T x N) = A(T x K) * B(N x K)^T with v_mfma_f32_32x32x2f32
//                   (or 16x16x4f32 for batches of up to 16 decode steps),
//                   epilogues: plain store, residual add, RoPE + cache append,
//                   SwiGLU (the same epilogues as the decode GEMVs)
//   attn_prefill    causal grouped-query attention of T queries over the
//                   cache rows with v_mfma_f32_16x16x4f32 (flash-attention
//                   style: online softmax, scores never leave registers)
//   embed           the per-token gather (the RMSNorms are fused into the
//                   products that follow them)
//
// All arithmetic is fp32 (products and sums), as in the decode kernels.
#include "ld_internal.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

namespace ld {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Embedding gather.

__global__ __launch_bounds__(256) void embed_kernel(const float* __restrict__ emb, const int32_t* __restrict__ tokens,
                                                    int dim, float* __restrict__ x) {
    const int t = blockIdx.x;
    const float4* src = reinterpret_cast<const float4*>(emb + (size_t)tokens[t] * dim);
    float4* dst = reinterpret_cast<float4*>(x + (size_t)t * dim);
    for (int i = threadIdx.x; i < dim / 4; i += 256) dst[i] = src[i];
}


// RMSNorm of every token row ("run.c 逐行解讀" §4 rmsnorm): out = g * (x *
// 1/sqrt(mean(x^2) + eps)), one block per row, for the prompt products that
// read a normalised copy of the residual stream.
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* __restrict__ x, const float* __restrict__ gain,
                                                           float eps, int dim, float* __restrict__ out) {
    __shared__ float part[4];
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)blockIdx.x * dim);
    const float4* g4 = reinterpret_cast<const float4*>(gain);
    float4* o = reinterpret_cast<float4*>(out + (size_t)blockIdx.x * dim);
    const int n4 = dim / 4;
    float ss = 0.f;
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 v = xr[i];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)dim + eps);
    for (int i = threadIdx.x; i < n4; i += 256) {
        const float4 v = xr[i], g = g4[i];
        o[i] = make_float4(g.x * (r * v.x), g.y * (r * v.y), g.z * (r * v.z), g.w * (r * v.w));
    }
}

// ---------------------------------------------------------------------------
// C = A * B^T on the matrix cores.
//
// A block of 256 threads (4 waves) computes a BM x 128 tile of C on the
// matrix cores (BM and the MFMA shape per product, see gemm_kernel).  K is
// walked in slabs of BK (16 or 32): both operand slabs go global -> registers
// -> LDS (row-major, K contiguous, rows padded by 4 floats), double-buffered
// with one barrier per slab, while the next slabs' global loads are in
// flight.  Within a slab, lane group g of an MFMA step supplies k position
// HK g + s at step s (HK = BK / lane groups), so each lane reads HK
// consecutive floats of its row with 16-byte LDS loads; every k is still used
// exactly once.  Rows of A past M and of B past N are clamped (their results
// are not stored); k past the end reads as zero.

constexpr int kBN = 128, kGemmThreads = 256;

// K slab depth and slabs in flight per row tile.  Prompts (BM = 128) gain
// about 2% from BK = 32 (fewer barriers per flop).  Decode batches, bound by
// the weight stream, run faster with 2 slabs in flight, and with BK = 32 for
// the 16- and 32-row tiles (a whole 128-byte line of each weight row per
// slab) but 16 for the 64-row tile (measured on the 7B shape: 6.8 vs 7.2 ms
// per step at 16 rows, 8.0 vs 8.1 at 32, 11.5 vs 12.3 at 64).
#ifndef LD_GEMM_BK128
#define LD_GEMM_BK128 32
#endif
#ifndef LD_GEMM_BK_M16
#define LD_GEMM_BK_M16 32
#endif
#ifndef LD_GEMM_BK_M32
#define LD_GEMM_BK_M32 32
#endif
#ifndef LD_GEMM_BK_M64
#define LD_GEMM_BK_M64 16
#endif
// 128-row tiles (prompts) take gemm_dtl_kernel (1) or gemm_kernel (0)
#ifndef LD_GEMM_DTL
#define LD_GEMM_DTL 1
#endif
#ifndef LD_GEMM_R_BATCH
#define LD_GEMM_R_BATCH 2
#endif

template <int KIND>
__device__ __forceinline__ const float* b_row(const GemmParams& p, int r) {
    if constexpr (KIND == G_SWIGLU) return ((r & 1) ? p.w1 : p.w0) + (size_t)(r >> 1) * p.k;
    if constexpr (KIND == G_QKV) {
        if (r < p.seg1) return p.w0 + (size_t)r * p.k;
        if (r < p.seg2) return p.w1 + (size_t)(r - p.seg1) * p.k;
        return p.w2 + (size_t)(r - p.seg2) * p.k;
    }
    return p.w0 + (size_t)r * p.k;
}

}  // namespace

// Zeros read in place of k past the end of a product's K, and ones in place of
// an RMSNorm gain where there is none.  Never written; their external linkage
// keeps the compiler from folding their values.
__device__ __attribute__((aligned(16))) float gemm_zero4[4];
__device__ __attribute__((aligned(16))) float gemm_one4[4] = {1.f, 1.f, 1.f, 1.f};

namespace {

// 4 floats of a row at k, zero from kend on.  Past the end the load takes the
// address of gemm_zero4 instead of selecting on the loaded value: with a
// select the compiler turns the load into a branch, and a load that may not
// have been issued makes every later wait one for all loads in flight.
__device__ __forceinline__ float4 load_k4(const float* row, int k, int kend) {
    const float* a = k < kend ? row + k : gemm_zero4;
    return *reinterpret_cast<const float4*>(a);
}

// 4 gains at k (clamped to the last 4 of K: past the end the A values they
// scale are zero); ones without a gain
__device__ __forceinline__ float4 load_gain4(const float* gain, int k, int K) {
    const float* a = gain ? gain + min(k, K - 4) : gemm_one4;
    return *reinterpret_cast<const float4*>(a);
}

// Blocks are dealt to the 8 XCDs round-robin; renumber them so that each XCD
// runs a contiguous range of tiles (tiles that share a B slab then share an L2).
__device__ __forceinline__ int xcd_local_block(int b, int nb) {
    const int q = nb / 8, r = nb % 8, x = b % 8;
    return x * q + min(x, r) + b / 8;
}

// C(gm, gn) = v, with other = C(gm, gn ^ 1), the pair partner.
template <int KIND>
__device__ __forceinline__ void epilogue(const GemmParams& p, int gm, int gn, float v, float other) {
    if constexpr (KIND == G_SWIGLU) {
        // hb = silu(w1 x) * (w3 x), silu(u) = u * 1/(1 + e^-u)
        if (!(gn & 1)) {
            float a = v;
            a *= 1.0f / (1.0f + expf(-a));
            a *= other;
            p.out[(size_t)gm * p.ldo + (gn >> 1)] = a;
        }
    } else if constexpr (KIND == G_QKV) {
        // prompt: position pos0 + m of one sequence; batch: row m is sequence m
        // at its own position
        const bool odd = gn & 1;
        const int pos = p.row_state ? p.row_state[gm].pos : p.pos0 + gm;
        const size_t seq = p.row_state ? (size_t)gm * p.seq_stride : 0;
        if (gn < p.seg2) {
            const bool is_q = gn < p.seg1;
            const int local = is_q ? gn : gn - p.seg1;
            const int hs = p.head_size;
            const float2 cs = p.rope[(size_t)pos * (size_t)(hs >> 1) + ((local % hs) >> 1)];
            const float a = odd ? other : v;  // element 2j
            const float b = odd ? v : other;  // element 2j+1
            const float rv = odd ? (a * cs.y + b * cs.x) : (a * cs.x - b * cs.y);
            if (is_q)
                p.out[(size_t)gm * p.ldo + gn] = rv;
            else
                p.kc[seq + (size_t)pos * p.kv_stride + local] = rv;
        } else {
            p.vc[seq + (size_t)pos * p.kv_stride + (gn - p.seg2)] = v;
        }
    } else if constexpr (KIND == G_RESID) {
        p.out[(size_t)gm * p.ldo + gn] += v;
    } else {
        p.out[(size_t)gm * p.ldo + gn] = v;
    }
}

// Matrix-core shapes: MT = 32 is v_mfma_f32_32x32x2f32 (k advances 2 per
// step), MT = 16 is v_mfma_f32_16x16x4f32 (k advances 4).  Lane l supplies
// row l % MT of A and of B; the G = 64 / MT lane groups supply the step's k
// positions.
template <int MT>
struct Mfma;
template <>
struct Mfma<32> {
    typedef v16f acc;
    static __device__ __forceinline__ acc step(float a, float b, acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // row of register r in lane group g (the column is l % 32)
    static __device__ __forceinline__ int row(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }
};
template <>
struct Mfma<16> {
    typedef v4f acc;
    static __device__ __forceinline__ acc step(float a, float b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int r, int g) { return g * 4 + r; }
};

// Tiles: BM = 128 rows (prompt prefill; gemm_dtl_kernel below runs these
// unless LD_GEMM_DTL is 0), 2 x 2 waves of 64 x 64 with MT = 32.
// A decode batch, where the weight stream is the cost, takes the smallest
// tile that holds its rows: BM = 16 (1 x 4 waves of 16 x 32, MT = 16), 32
// (1 x 4 waves of 32 x 32) or 64 (2 x 2 waves of 32 x 64).  The matrix-core
// work per weight byte grows with BM: at BM = 32 streaming the weights at
// 8 TB/s would keep the fp32 matrix cores 80% busy, at BM = 16 40%.
//
// Pipeline: R register sets hold the next R slabs' global loads, so R slabs
// per block are in flight while slab kt is multiplied out of LDS; at the end
// of iteration kt the set holding slab kt+1 goes to the other LDS buffer and
// is refilled with slab kt+1+R.
//
// NORM: C = RMSNorm(A) B^T with the gain p.gain ("run.c 逐行解讀" §4, the
// rmsnorm before the q/k/v and w1/w3 products and the classifier).  The norm's
// row scale is a common factor of a row of C, so A is multiplied by the gain
// on its way to LDS, the blocks accumulate each row's sum of squares from the
// same A values, and the scale 1/sqrt(mean(a^2) + eps) multiplies the row's
// products before the epilogue: here when the block holds all of K, in
// gemm_reduce_kernel (which sums the squares' split partials too) otherwise.
template <int KIND, int BM, int BK, int MT, int R, bool NORM>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(GemmParams p) {
    constexpr int WAVES_M = BM / MT >= 2 ? 2 : 1, WAVES_N = 4 / WAVES_M;
    constexpr int TM = BM / (MT * WAVES_M), TN = kBN / (MT * WAVES_N);  // MT x MT tiles per wave
    constexpr int G = 64 / MT;                                           // lane groups (k per step)
    constexpr int HK = BK / G;                                           // k per lane and slab
    constexpr int NR = MT * MT / 64;                                     // accumulator registers per tile
    constexpr int ROW = BK + 4;                                          // padded LDS row
    constexpr int Q4 = BK / 4;                                           // float4 per row and slab
    constexpr int A_PER = (BM * Q4 + kGemmThreads - 1) / kGemmThreads;  // A float4 loads per thread and slab
    constexpr int B_PER = kBN * Q4 / kGemmThreads;
    static_assert(HK % 4 == 0 && TM >= 1 && TN >= 1, "tile shape");
    typedef typename Mfma<MT>::acc acc_t;
    __shared__ __attribute__((aligned(16))) float As[2][BM][ROW];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBN][ROW];
    __shared__ float row_scale[NORM ? BM : 1];

    const int mtiles = (p.m + BM - 1) / BM;
    const int lb = xcd_local_block(blockIdx.x, gridDim.x);
    const int ks = lb % p.splits, tile = lb / p.splits;  // split ks of K for this tile
    const int m0 = (tile % mtiles) * BM, n0 = (tile / mtiles) * kBN;
    const int kbeg = ks * p.kchunk, kend = min(p.k, kbeg + p.kchunk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane % MT, lg = lane / MT;
    const int wm = (wave % WAVES_M) * (TM * MT), wn = (wave / WAVES_M) * (TN * MT);

    // this thread's rows and k quads of every slab: float4 number q of a slab is
    // row q / Q4, k 4 (q % Q4)
    const float* arow[A_PER];
    int alrow[A_PER], alk[A_PER];
    bool aon[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int q = tid + kGemmThreads * i;
        aon[i] = q < BM * Q4;
        alrow[i] = min(q / Q4, BM - 1);
        alk[i] = (q % Q4) * 4;
        arow[i] = p.a + (size_t)min(m0 + alrow[i], p.m - 1) * p.lda;
    }
    const float* brow[B_PER];
    int blrow[B_PER], blk[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int q = tid + kGemmThreads * i;
        blrow[i] = q / Q4;
        blk[i] = (q % Q4) * 4;
        brow[i] = b_row<KIND>(p, min(n0 + blrow[i], p.n - 1));
    }

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;

    // register sets: A, its gains (NORM), B
    constexpr int GS = NORM ? R : 1, GP = NORM ? A_PER : 1;
    float4 ra[R][A_PER], rg[GS][GP], rb[R][B_PER];
    float sq[A_PER];  // NORM: this thread's part of its A rows' sums of squares
#pragma unroll
    for (int i = 0; i < A_PER; ++i) sq[i] = 0.f;

    // Whole slabs (K chunk / BK of them) go through plain pointer offsets.
    // The loop runs a whole number of register-set turns; slabs past the last
    // whole one reload that one (always in bounds) with A scaled by zero, so
    // they add nothing and no load of the loop sits behind a branch (a load
    // that may not have been issued makes every later wait one for all loads
    // in flight).  A ragged end of K is one masked slab after the loop.
    const int nfull = (kend - kbeg) / BK;
    const int nmain = (nfull + R - 1) / R * R;
    const float* pa[A_PER];
    const float* pg[GP];
    const float* pb[B_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) pa[i] = arow[i] + kbeg + alk[i];
#pragma unroll
    for (int i = 0; i < GP; ++i) pg[i] = NORM ? (p.gain ? p.gain + kbeg + alk[i] : gemm_one4) : nullptr;
#pragma unroll
    for (int i = 0; i < B_PER; ++i) pb[i] = brow[i] + kbeg + blk[i];
    const size_t gstep = NORM && p.gain ? BK : 0;  // the ones vector does not advance
    auto load_whole = [&](float4(&xa)[A_PER], float4(&xg)[GP], float4(&xb)[B_PER], int slab) {
        const size_t off = (size_t)min(slab, nfull - 1) * BK;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) xa[i] = *reinterpret_cast<const float4*>(pa[i] + off);
        if constexpr (NORM) {
            const size_t goff = (size_t)min(slab, nfull - 1) * gstep;
#pragma unroll
            for (int i = 0; i < A_PER; ++i) xg[i] = *reinterpret_cast<const float4*>(pg[i] + goff);
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) xb[i] = *reinterpret_cast<const float4*>(pb[i] + off);
    };
    // keep: 1 for a slab of this split, 0 for a padding slab
    auto store_slab = [&](const float4(&xa)[A_PER], const float4(&xg)[GP], const float4(&xb)[B_PER], int buf,
                          float keep) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            float4 v = make_float4(keep * xa[i].x, keep * xa[i].y, keep * xa[i].z, keep * xa[i].w);
            if constexpr (NORM) {
                sq[i] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                const float4 g = xg[i];
                v = make_float4(g.x * v.x, g.y * v.y, g.z * v.z, g.w * v.w);
            }
            if (aon[i]) *reinterpret_cast<float4*>(&As[buf][alrow[i]][alk[i]]) = v;
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) *reinterpret_cast<float4*>(&Bs[buf][blrow[i]][blk[i]]) = xb[i];
    };
    auto multiply = [&](int buf) {
        // the MFMA's k positions of step s are k = HK g + s (lane group g):
        // each lane reads HK consecutive floats of its row
        float av[TM][HK], bv[TN][HK];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < HK; q += 4) {
                const float4 x = *reinterpret_cast<const float4*>(&As[buf][wm + i * MT + li][lg * HK + q]);
                av[i][q] = x.x; av[i][q + 1] = x.y; av[i][q + 2] = x.z; av[i][q + 3] = x.w;
            }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < HK; q += 4) {
                const float4 y = *reinterpret_cast<const float4*>(&Bs[buf][wn + j * MT + li][lg * HK + q]);
                bv[j][q] = y.x; bv[j][q + 1] = y.y; bv[j][q + 2] = y.z; bv[j][q + 3] = y.w;
            }
#pragma unroll
        for (int st = 0; st < HK; ++st)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<MT>::step(av[i][st], bv[j][st], acc[i][j]);
    };

    if (nfull > 0) {
#pragma unroll
        for (int s = 0; s < R; ++s) load_whole(ra[s], rg[s % GS], rb[s], s);
        store_slab(ra[0], rg[0], rb[0], 0, 1.f);
        load_whole(ra[0], rg[0], rb[0], R);
        __syncthreads();
        for (int kt0 = 0; kt0 < nmain; kt0 += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int kt = kt0 + u;
                const int buf = kt & 1;
                multiply(buf);
                // slab kt+1 to the other buffer (read in the previous
                // iteration, before the barrier), then its register set
                // takes slab kt+1+R
                store_slab(ra[(u + 1) % R], rg[(u + 1) % R % GS], rb[(u + 1) % R], buf ^ 1, kt + 1 < nfull ? 1.f : 0.f);
                load_whole(ra[(u + 1) % R], rg[(u + 1) % R % GS], rb[(u + 1) % R], kt + 1 + R);
                __syncthreads();
            }
        }
    }
    if (kbeg + nfull * BK < kend) {  // the ragged end of K: one slab, zero past kend
        const int k = kbeg + nfull * BK;
        const int buf = nmain & 1;  // not read since the last barrier
#pragma unroll
        for (int i = 0; i < A_PER; ++i) ra[0][i] = load_k4(arow[i], k + alk[i], kend);
        if constexpr (NORM) {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) rg[0][i] = load_gain4(p.gain, k + alk[i], p.k);
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) rb[0][i] = load_k4(brow[i], k + blk[i], kend);
        store_slab(ra[0], rg[0], rb[0], buf, 1.f);
        __syncthreads();
        multiply(buf);
    }

    if constexpr (NORM) {
        // the Q4 consecutive lanes of an A row hold its sum of squares over
        // this split's k in parts; the first column tile publishes them
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            float v = sq[i];
#pragma unroll
            for (int o = 1; o < Q4; o <<= 1) v += __shfl_xor(v, o);
            const int q = tid + kGemmThreads * i, gm = m0 + alrow[i];
            if (aon[i] && q % Q4 == 0) {
                if (p.splits > 1) {
                    if (n0 == 0 && gm < p.m) p.part[(size_t)p.splits * p.m * p.n + (size_t)ks * p.m + gm] = v;
                } else {
                    row_scale[alrow[i]] = 1.0f / sqrtf(v / (float)p.k + p.eps);
                }
            }
        }
        if (p.splits == 1) __syncthreads();
    }

    // Epilogue.  Register r of tile (i, j) in lane group g holds C(row, col)
    // with row = wm + MT i + Mfma<MT>::row(r, g) and col = wn + MT j + l % MT:
    // lanes 2c and 2c+1 hold the adjacent columns (2c, 2c+1) of one row, the
    // pair RoPE rotates and the (w1, w3) pair SwiGLU combines.  With split K
    // the block stores its partial tile instead; gemm_reduce_kernel sums the
    // splits in order and applies the epilogue.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int gm = m0 + wm + i * MT + Mfma<MT>::row(r, lg);
                const int gn = n0 + wn + j * MT + li;
                float v = acc[i][j][r];
                if constexpr (NORM) {
                    if (p.splits == 1) v *= row_scale[gm - m0];
                }
                if (p.splits > 1) {
                    if (gm < p.m && gn < p.n) p.part[((size_t)ks * p.m + gm) * p.n + gn] = v;
                    continue;
                }
                const float other = (KIND == G_QKV || KIND == G_SWIGLU) ? __shfl_xor(v, 1) : 0.f;
                if (gm < p.m && gn < p.n) epilogue<KIND>(p, gm, gn, v, other);
            }
}

// ---------------------------------------------------------------------------
// Prompt products (128-row tiles) with the slabs loaded straight into LDS.
//
// The same 128 x 128 tile, 2 x 2 waves of 64 x 64 and v_mfma_f32_32x32x2f32
// as gemm_kernel, but the K slabs (BK deep) go from global memory to LDS by
// the load-to-LDS form of the global load (global_load_lds_dwordx4: each
// lane's 16 bytes land at the wave's LDS base + 16 x lane), so no register
// holds a slab on its way.  ST LDS buffers keep ST - 1 slabs in flight
// behind the one being multiplied.  Built with BK = 32, ST = 2: 66 KB of LDS
// and 142 registers, two blocks per CU (two waves per SIMD).  Measured on the
// 7B-shaped prompt of 2048 tokens: 224.6 ms against 228.4 for gemm_kernel;
// slabs of 16 with 2-4 buffers 228.6-229.9 ms; one block per CU (BK = 32,
// ST = 3 or 4) 257-259 ms.
//
// Slab layout: row r, k quad c (4 floats) sits at quad position
// c ^ ((r / SH) % QPR) of its row (QPR = BK / 4 quads; rows SH = 16 / QPR
// apart share LDS banks).  A fragment read (one k quad of 16 consecutive
// rows per 16 lanes) then covers every bank once.  A load instruction fills
// 64 / QPR rows: lane l takes row l / QPR and position l % QPR.
//
// Per slab kt a wave runs its MFMAs in groups of 4 k per lane (16 each).
// The LDS reads of the next group and the loads of slab kt + ST - 1 are
// issued one at a time between the MFMAs (a wave issues in order, so a burst
// of them would hold back its next MFMA).  Before the last group a wave
// waits for its loads of slab kt + 1 (later slabs stay in flight) and its
// LDS reads of slab kt, then the block barrier: slab kt + 1 is then visible
// to every wave, and slab kt's buffer free for the loads of the next
// iteration.  The last group, already in registers, covers the reads of
// slab kt + 1's first group.
//
// NORM: the RMSNorm gain is staged per slab in LDS too (each wave its own
// copies of the slab's gains, one 4-byte load per lane) and multiplies the A
// fragments after they are read; the row sums of squares are taken from the
// same fragments before the gain.

#ifndef LD_GEMM_DTL_STAGES
#define LD_GEMM_DTL_STAGES 2
#endif
#ifndef LD_GEMM_DTL_BK
#define LD_GEMM_DTL_BK 32
#endif

__device__ __forceinline__ float f4c(const float4& v, int t) { return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w; }

// LDS byte address of a shared-memory pointer
__device__ __forceinline__ unsigned lds_addr(const float* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) float*)p;
}

// One load of 16 bytes per lane straight into LDS at lds + 16 x lane (lds
// wave-uniform).  Inline assembly, so that the compiler does not take the
// LDS write as pending at every later LDS read; the kernel counts these
// loads itself before each barrier.  M0 is set here; nothing else in these
// kernels uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// the same with 4 bytes per lane (at lds + 4 x lane)
__device__ __forceinline__ void lds_load4(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector memory loads are in flight and
// all its LDS reads are done, then the block barrier.
template <int N>
__device__ __forceinline__ void slab_barrier() {
    static_assert(N >= 0 && N <= 63, "vector memory count");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int KIND, bool NORM, int BK, int ST>
__global__ __launch_bounds__(kGemmThreads, ST * BK <= 64 ? 2 : 1) void gemm_dtl_kernel(GemmParams p) {
    constexpr int MT = 32, TM = 2, TN = 2, NR = 16;
    constexpr int QPR = BK / 4;          // k quads per slab row
    constexpr int RPI = 64 / QPR;        // rows per load instruction
    constexpr int NI = 128 / RPI / 4;    // load instructions per operand, wave and slab
    constexpr int SH = 16 / QPR;         // rows apart that share LDS banks
    constexpr int HK = BK / 2;           // k per lane group and slab
    constexpr int NG = HK / 4;           // groups of 4 k per slab
    constexpr int NL = 2 * NI + (NORM ? 1 : 0);  // loads per slab and lane
    static_assert((BK == 16 || BK == 32) && ST >= 2 && ST <= 4, "shape");
    typedef Mfma<MT>::acc acc_t;
    __shared__ __attribute__((aligned(1024))) float As[ST][128 * BK];
    __shared__ __attribute__((aligned(1024))) float Bs[ST][128 * BK];
    __shared__ __attribute__((aligned(16))) float Gs[NORM ? ST : 1][NORM ? 256 : 4];
    __shared__ float row_scale[NORM ? 128 : 1];

    const int mtiles = (p.m + 127) / 128;
    const int lb = xcd_local_block(blockIdx.x, gridDim.x);
    const int ks = lb % p.splits, tile = lb / p.splits;
    const int m0 = (tile % mtiles) * 128, n0 = (tile / mtiles) * kBN;
    const int kbeg = ks * p.kchunk, kend = min(p.k, kbeg + p.kchunk);
    const int nslab = (kend - kbeg + BK - 1) / BK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lg = lane >> 5;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;

    // slab loads: instruction i of a wave fills rows 32 wave + RPI i ..; lane
    // l takes row r = 32 wave + RPI i + l / QPR at position l % QPR, which
    // holds k quad (l % QPR) ^ ((r / SH) % QPR)
    int lq[NI];
    const float* ga[NI];
    const float* gb[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = 32 * wave + RPI * i + lane / QPR;
        lq[i] = (lane % QPR) ^ ((r / SH) % QPR);
        ga[i] = p.a + (size_t)min(m0 + r, p.m - 1) * p.lda + 4 * lq[i];
        gb[i] = b_row<KIND>(p, min(n0 + r, p.n - 1)) + 4 * lq[i];
    }
    // load u of slab s (into buffer s % ST): u < NI the A rows of instruction
    // u, u < 2 NI the B rows of instruction u - NI, u = 2 NI the gains (each
    // wave its own copies: lane l takes gain k % BK); k past kend reads zeros
    auto issue_one = [&](int s, int u) {
        const int st = s % ST;
        const int kk = kbeg + BK * s;
        if (u < 2 * NI) {
            const int i = u % NI;
            const bool in = kk + 4 * lq[i] < kend;
            const float* src = u < NI ? ga[i] + kk : gb[i] + kk;
            const float* dst = u < NI ? &As[st][(32 * wave + RPI * i) * BK] : &Bs[st][(32 * wave + RPI * i) * BK];
            lds_load16(in ? (const void*)src : (const void*)gemm_zero4, lds_addr(dst));
        } else if constexpr (NORM) {
            lds_load4(p.gain + min(kk + lane % BK, p.k - 1), lds_addr(&Gs[st][64 * wave]));
        }
    };

    // fragment offsets (floats in a slab): rows wm + 32 i + li and
    // wn + 32 j + li; group g reads k quad NG lg + g, at position
    // (NG lg + g) ^ ((li / SH) % QPR)
    const int xq = (NG * lg) ^ ((li / SH) % QPR);
    int aoff[TM], boff[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) aoff[i] = (wm + 32 * i + li) * BK;
#pragma unroll
    for (int j = 0; j < TN; ++j) boff[j] = (wn + 32 * j + li) * BK;

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;
    float sq[TM] = {};
    float4 fa[2][TM], fb[2][TN], gv[2];  // two fragment sets (gains: NORM)

    // LDS read r of group g of buffer st into a fragment set: r = 0, 1 the A
    // tiles, 2, 3 the B tiles, 4 the gains
    constexpr int NRD = NORM ? 5 : 4;
    auto read_one = [&](int st, int g, int set, int r) {
        const int q = (xq ^ g) << 2;
        if (r < 2) fa[set][r] = *reinterpret_cast<const float4*>(&As[st][aoff[r] + q]);
        else if (r < 4) fb[set][r - 2] = *reinterpret_cast<const float4*>(&Bs[st][boff[r - 2] + q]);
        else if constexpr (NORM) gv[set] = *reinterpret_cast<const float4*>(&Gs[st][64 * wave + HK * lg + 4 * g]);
    };
    // NORM: A tile i's rows' sums of squares, then the gain
    auto prep = [&](int set, int i) {
        if constexpr (NORM) {
            const float4 g = gv[set];
            float4& a = fa[set][i];
            sq[i] += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
            a = make_float4(a.x * g.x, a.y * g.y, a.z * g.z, a.w * g.w);
        }
    };
    // product idx (0..15) of a group: k step idx / 4, tiles ((idx / 2) % 2, idx % 2)
    auto mfma_one = [&](int set, int idx) {
        const int s = idx >> 2, i = (idx >> 1) & 1, j = idx & 1;
        acc[i][j] = Mfma<MT>::step(f4c(fa[set][i], s), f4c(fb[set][j], s), acc[i][j]);
    };
    // group g of slab kt from fragment set g % 2: the reads of (rst, rg) into
    // the other set after its first products, and in the groups before the
    // barrier the loads of slab kt + ST - 1 (if any) after every other product
    auto group = [&](int kt, int g, int rst, int rg) {
        const int set = g & 1;
        const int ls = kt + ST - 1;
        const bool more = ls < nslab;
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
            if (idx == 0) prep(set, 0);
            mfma_one(set, idx);
            if (idx == 0) prep(set, 1);
            if (idx < NRD) read_one(rst, rg, set ^ 1, idx);
            if (g < NG - 1 && (idx & 1)) {
                const int u = 8 * g + (idx >> 1);
                if (u < NL && more) issue_one(ls, u);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    static_assert(8 * (NG - 1) >= NL, "load slots");
    // waits for slab kt + 1 with the loads of later slabs in flight
    auto end_slab = [&](int kt) {
        int after = 0;
#pragma unroll
        for (int d = 2; d < ST; ++d) after += kt + d < nslab;
        if (after == 2) slab_barrier<2 * NL>();
        else if (after == 1) slab_barrier<NL>();
        else slab_barrier<0>();
    };

    for (int s = 0; s < ST - 1 && s < nslab; ++s)
        for (int u = 0; u < NL; ++u) issue_one(s, u);
    end_slab(-1);
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(0, 0, 0, r);
    for (int kt = 0; kt < nslab; ++kt) {
        const int st = kt % ST;
#pragma unroll
        for (int g = 0; g < NG - 1; ++g) group(kt, g, st, g + 1);
        end_slab(kt);
        group(kt, NG - 1, (kt + 1) % ST, 0);  // after the last slab the reads are stale and not used
    }

    if constexpr (NORM) {
        // lanes li and li + 32 hold row wm + 32 i + li's sum in two halves;
        // the waves of the first column half publish it
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const float v = sq[i] + __shfl_xor(sq[i], 32);
            const int r = wm + 32 * i + li, gm = m0 + r;
            if (wn == 0 && lg == 0) {
                if (p.splits > 1) {
                    if (n0 == 0 && gm < p.m) p.part[(size_t)p.splits * p.m * p.n + (size_t)ks * p.m + gm] = v;
                } else {
                    row_scale[r] = 1.0f / sqrtf(v / (float)p.k + p.eps);
                }
            }
        }
        if (p.splits == 1) __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int gm = m0 + wm + i * MT + Mfma<MT>::row(r, lg);
                const int gn = n0 + wn + j * MT + li;
                float v = acc[i][j][r];
                if constexpr (NORM) {
                    if (p.splits == 1) v *= row_scale[gm - m0];
                }
                if (p.splits > 1) {
                    if (gm < p.m && gn < p.n) p.part[((size_t)ks * p.m + gm) * p.n + gn] = v;
                    continue;
                }
                const float other = (KIND == G_QKV || KIND == G_SWIGLU) ? __shfl_xor(v, 1) : 0.f;
                if (gm < p.m && gn < p.n) epilogue<KIND>(p, gm, gn, v, other);
            }
}

// Sum of the split partials of C, in split order, then the epilogue: one
// thread per (row, column pair).  The loads of 8 splits are issued before
// their sums.  With a norm gain the row's sum of squares is summed the same
// way and its scale multiplies the two sums.
template <int KIND>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmParams p) {
    const int pairs = (p.n + 1) / 2;
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long long)p.m * pairs) return;
    const int gm = (int)(e / pairs), c = (int)(e % pairs), gn = 2 * c;
    const bool two = gn + 1 < p.n;
    const size_t stride = (size_t)p.m * p.n;
    const float* src = p.part + (size_t)gm * p.n + gn;
    const int d1 = two ? 1 : 0;  // without a second column v1 is never used
    const float* sqs = p.gain ? p.part + (size_t)p.splits * stride + gm : src;
    const size_t sq_stride = p.gain ? (size_t)p.m : stride;
    float v0 = 0.f, v1 = 0.f, ss = 0.f;
    constexpr int U = 8;
    int ks = 0;
    for (; ks + U <= p.splits; ks += U) {
        float a[U], b[U], q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = src[(ks + u) * stride];
            b[u] = src[(ks + u) * stride + d1];
            q[u] = sqs[(ks + u) * sq_stride];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v0 += a[u];
            v1 += b[u];
            ss += q[u];
        }
    }
    for (; ks < p.splits; ++ks) {
        v0 += src[ks * stride];
        v1 += src[ks * stride + d1];
        ss += sqs[ks * sq_stride];
    }
    if (p.gain) {
        const float r = 1.0f / sqrtf(ss / (float)p.k + p.eps);
        v0 *= r;
        v1 *= r;
    }
    epilogue<KIND>(p, gm, gn, v0, v1);
    if (two) epilogue<KIND>(p, gm, gn + 1, v1, v0);
}

// ---------------------------------------------------------------------------
// Causal attention of T queries at positions pos0 .. pos0 + T - 1 over the
// cache rows 0 .. pos0 + T - 1 ("run.c 逐行解讀" §4 step 2e for every query),
// on the matrix cores with v_mfma_f32_16x16x4f32.
//
// A block (4 waves) takes two tiles of 64 consecutive queries of one head h,
// one after the other (a short and a long one); each wave 16 of a tile's.
// Key tiles of 32 rows of K (as rows) and V (transposed: Vt[d][key]) of kv
// head g(h) are staged in LDS by the whole block.  Per 16 keys a wave
// computes the transposed score tile S^T (16 keys x 16 queries) = K Q^T:
// lane l then holds 4 keys of query
// l % 16, so the online softmax statistics (m, l) of a query live in the four
// lanes l % 16 + 16c and need two lane exchanges.  The same registers are
// the B operand of O^T (hs x 16 queries) += V^T P^T, whose result keeps the
// query in l % 16, so the rescale by e^(m_old - m_new) needs no exchange.
// Scores are kept in base-2
// units (q scaled by log2(e) / sqrt(hs)), so the weights come from the native
// 2^x.
// Q (hs/4 floats per lane) and O^T (hs/4) stay in registers.  The MFMA's four
// k positions per step are k = (hs/4) c + s for lane quarter c in the score
// product, and key 4c + s in the value product.

constexpr int kAQ = 64;       // queries per block
constexpr float kLog2eP = 1.4426950408889634f;  // log2(e)
constexpr int kAK = 32;       // keys per LDS tile
constexpr int kAPad = 4;

#ifndef LD_APF_PAIR
#define LD_APF_PAIR 1
#endif

template <int HS>
// (three blocks per CU where the head fits: 126 registers at head size 128,
// against 172 at two, which left the 70B layer's 1792 blocks a third fewer
// slots: 951 against 1099 us per layer of its 3584-token prompt)
__global__ __launch_bounds__(256, HS <= 128 ? 3 : 1) void attn_prefill_kernel(AttnPrefillParams p) {
    constexpr int Q4 = HS / 4;    // d per lane quarter
    constexpr int CT = HS / 16;   // 16-wide column tiles of the output
    constexpr int ROW = HS + kAPad;
    constexpr int VROW = kAK + 4;  // keys per row of the transposed value tile (+4: no bank conflicts)
    __shared__ __attribute__((aligned(16))) float Ks[kAK][ROW];
    __shared__ __attribute__((aligned(16))) float Vt[HS][VROW];

    const int h = blockIdx.y;
    const int g = (int)(((long long)h * p.n_kv_heads) / p.n_heads);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 15, lc = lane >> 4;
    // scores in base-2 units: q is scaled by log2(e) / sqrt(hs), so that
    // e^(s - m) is 2^(s2 - m2) on the native exponential
    const float scale = kLog2eP / sqrtf((float)HS);
    const float* kbase = p.kc + (size_t)g * HS;
    const float* vbase = p.vc + (size_t)g * HS;
    const int ntiles = (p.t + kAQ - 1) / kAQ;

    // Causal work grows with the query tile, so a block takes tile b and tile
    // ntiles - 1 - b: every block then has about the same number of key tiles,
    // instead of the last blocks running alone at the end (7B shape, 2048
    // tokens: 23 -> 13 ms of attention per prompt).
    for (int pass = 0; pass < (LD_APF_PAIR ? 2 : 1); ++pass) {
        const int qt = pass == 0 ? (int)blockIdx.x : ntiles - 1 - (int)blockIdx.x;
        if (pass == 1 && qt <= (int)blockIdx.x) break;  // the middle tile of an odd count is done once
        const int q0 = qt * kAQ;          // first query (token index in the chunk) of the tile
        const int wq0 = q0 + wave * 16;   // first query of the wave
        const int tq = min(wq0 + lq, p.t - 1);  // this lane's query (clamped; results past T are not stored)
        const int qpos = p.pos0 + tq;

        // Q row quarter: Q[tq][h*HS + lc*Q4 + s], pre-scaled
        float qv[Q4];
        {
            const float4* q4 = reinterpret_cast<const float4*>(p.q + (size_t)tq * p.ldq + (size_t)h * HS + lc * Q4);
#pragma unroll
            for (int s = 0; s < Q4 / 4; ++s) {
                const float4 v = q4[s];
                qv[4 * s] = v.x * scale;
                qv[4 * s + 1] = v.y * scale;
                qv[4 * s + 2] = v.z * scale;
                qv[4 * s + 3] = v.w * scale;
            }
        }
        v4f o[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) o[c] = v4f{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f;

        const int last_q = min(q0 + kAQ, p.t) - 1;  // last query of the tile
        const int n_keys = p.pos0 + last_q + 1;
        const int wave_last_pos = p.pos0 + min(wq0 + 15, p.t - 1);

        for (int k0 = 0; k0 < n_keys; k0 += kAK) {
            // stage keys k0 .. k0 + 31 (rows past the last key read the last key;
            // they are masked): K as rows, V transposed (Vt[d][key]), so that a
            // lane's four values of one output column are one 16-byte read.
            // All of a thread's loads go out before its LDS writes (one round
            // trip per tile).  V item e: dims 4 c4 .. 4 c4 + 3 of keys 4 kg ..
            // 4 kg + 3 (kg fastest across lanes: two-way bank conflicts at most).
            __syncthreads();
            {
                // items past the end are clamped to the last one: loaded and
                // written twice with the same values, with no branch (a load
                // behind a branch is waited for on its own)
                constexpr int NKE = kAK * (HS / 4), NVE = (kAK / 4) * (HS / 4);
                constexpr int NKI = (NKE + 255) / 256, NVI = (NVE + 255) / 256;
                float4 kr[NKI], vr[NVI][4];
#pragma unroll
                for (int i = 0; i < NKI; ++i) {
                    const int e = min(tid + 256 * i, NKE - 1);
                    const int r = e / (HS / 4), c4 = e % (HS / 4);
                    const size_t row = (size_t)min(k0 + r, n_keys - 1) * p.kv_stride;
                    kr[i] = reinterpret_cast<const float4*>(kbase + row)[c4];
                }
#pragma unroll
                for (int i = 0; i < NVI; ++i) {
                    const int e = min(tid + 256 * i, NVE - 1);
                    const int kg = e % (kAK / 4), c4 = e / (kAK / 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const size_t row = (size_t)min(k0 + 4 * kg + j, n_keys - 1) * p.kv_stride;
                        vr[i][j] = reinterpret_cast<const float4*>(vbase + row)[c4];
                    }
                }
#pragma unroll
                for (int i = 0; i < NKI; ++i) {
                    const int e = min(tid + 256 * i, NKE - 1);
                    *reinterpret_cast<float4*>(&Ks[e / (HS / 4)][4 * (e % (HS / 4))]) = kr[i];
                }
#pragma unroll
                for (int i = 0; i < NVI; ++i) {
                    const int e = min(tid + 256 * i, NVE - 1);
                    const int kg = e % (kAK / 4), c4 = e / (kAK / 4);
                    *reinterpret_cast<float4*>(&Vt[4 * c4 + 0][4 * kg]) =
                        make_float4(vr[i][0].x, vr[i][1].x, vr[i][2].x, vr[i][3].x);
                    *reinterpret_cast<float4*>(&Vt[4 * c4 + 1][4 * kg]) =
                        make_float4(vr[i][0].y, vr[i][1].y, vr[i][2].y, vr[i][3].y);
                    *reinterpret_cast<float4*>(&Vt[4 * c4 + 2][4 * kg]) =
                        make_float4(vr[i][0].z, vr[i][1].z, vr[i][2].z, vr[i][3].z);
                    *reinterpret_cast<float4*>(&Vt[4 * c4 + 3][4 * kg]) =
                        make_float4(vr[i][0].w, vr[i][1].w, vr[i][2].w, vr[i][3].w);
                }
            }
            __syncthreads();
            if (k0 > wave_last_pos) continue;  // every key of the tile is after every query of this wave

#pragma unroll
            for (int sub = 0; sub < kAK / 16; ++sub) {
                // S^T(16 keys x 16 queries): A = K rows (key lq), B = Q^T (query lq)
                v4f st = v4f{0.f, 0.f, 0.f, 0.f};
                const float* krow = &Ks[sub * 16 + lq][lc * Q4];
#pragma unroll
                for (int s = 0; s < Q4; s += 4) {
                    const float4 kk = *reinterpret_cast<const float4*>(krow + s);
                    st = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.x, qv[s], st, 0, 0, 0);
                    st = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.y, qv[s + 1], st, 0, 0, 0);
                    st = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.z, qv[s + 2], st, 0, 0, 0);
                    st = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.w, qv[s + 3], st, 0, 0, 0);
                }
                // register r: key k0 + 16 sub + 4 lc + r of query tq; causal mask
                float sc[4];
                float tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kpos = k0 + sub * 16 + lc * 4 + r;
                    sc[r] = kpos <= qpos ? st[r] : -INFINITY;
                    tmax = fmaxf(tmax, sc[r]);
                }
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                const float m_new = fmaxf(m, tmax);  // finite: key 0 is in the first tile of every query
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);
                float psum = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sc[r] = __builtin_amdgcn_exp2f(sc[r] - m_new);
                    psum += sc[r];
                }
                psum += __shfl_xor(psum, 16);
                psum += __shfl_xor(psum, 32);
                l = l * alpha + psum;
                m = m_new;
                // O^T(hs x 16 queries) += V^T P^T: A = V^T (column 16 c + lq,
                // keys 4 lc + r, one 16-byte read), B = P^T
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    o[c] *= alpha;
                    const float4 vv = *reinterpret_cast<const float4*>(&Vt[c * 16 + lq][sub * 16 + lc * 4]);
                    o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.x, sc[0], o[c], 0, 0, 0);
                    o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.y, sc[1], o[c], 0, 0, 0);
                    o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.z, sc[2], o[c], 0, 0, 0);
                    o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.w, sc[3], o[c], 0, 0, 0);
                }
            }
        }
        // O^T register r of tile c: column 16 c + 4 lc + r of query tq
        if (wq0 + lq < p.t) {
            const float inv = 1.0f / l;
            float* out = p.out + (size_t)tq * p.ldo + (size_t)h * HS;
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[c * 16 + lc * 4 + r] = o[c][r] * inv;
        }
    }
}

}  // namespace

hipError_t embed_launch(const float* emb, const int32_t* tokens, int t, int dim, float* x, hipStream_t s) {
    hipLaunchKernelGGL(embed_kernel, dim3(t), dim3(256), 0, s, emb, tokens, dim, x);
    return hipGetLastError();
}

hipError_t rmsnorm_rows_launch(const float* x, const float* gain, float eps, int t, int dim, float* out,
                               hipStream_t s) {
    if (t <= 0 || dim <= 0 || dim % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(t), dim3(256), 0, s, x, gain, eps, dim, out);
    return hipGetLastError();
}

namespace {

hipError_t gemm_reduce_launch(int kind, const GemmParams& p, hipStream_t s);

template <int BM, int BK, int MT, int R, bool NORM>
void gemm_launch_kind(int kind, const GemmParams& p, dim3 grid, dim3 block, hipStream_t s) {
    switch (kind) {
        case G_PLAIN: hipLaunchKernelGGL((gemm_kernel<G_PLAIN, BM, BK, MT, R, NORM>), grid, block, 0, s, p); break;
        case G_RESID: hipLaunchKernelGGL((gemm_kernel<G_RESID, BM, BK, MT, R, NORM>), grid, block, 0, s, p); break;
        case G_QKV: hipLaunchKernelGGL((gemm_kernel<G_QKV, BM, BK, MT, R, NORM>), grid, block, 0, s, p); break;
        case G_SWIGLU: hipLaunchKernelGGL((gemm_kernel<G_SWIGLU, BM, BK, MT, R, NORM>), grid, block, 0, s, p); break;
    }
}

template <int BM, int BK, int MT, int R>
hipError_t gemm_launch_bm(int kind, const GemmParams& p, hipStream_t s) {
    const long long blocks = (long long)((p.m + BM - 1) / BM) * ((p.n + kBN - 1) / kBN) * p.splits;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    if (kind != G_PLAIN && kind != G_RESID && kind != G_QKV && kind != G_SWIGLU) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kGemmThreads);
    if (p.gain)
        gemm_launch_kind<BM, BK, MT, R, true>(kind, p, grid, block, s);
    else
        gemm_launch_kind<BM, BK, MT, R, false>(kind, p, grid, block, s);
    return gemm_reduce_launch(kind, p, s);
}

template <bool NORM>
void gemm_dtl_kind(int kind, const GemmParams& p, dim3 grid, hipStream_t s) {
    const dim3 block(kGemmThreads);
    switch (kind) {
        case G_PLAIN: hipLaunchKernelGGL((gemm_dtl_kernel<G_PLAIN, NORM, LD_GEMM_DTL_BK, LD_GEMM_DTL_STAGES>), grid, block, 0, s, p); break;
        case G_RESID: hipLaunchKernelGGL((gemm_dtl_kernel<G_RESID, NORM, LD_GEMM_DTL_BK, LD_GEMM_DTL_STAGES>), grid, block, 0, s, p); break;
        case G_QKV: hipLaunchKernelGGL((gemm_dtl_kernel<G_QKV, NORM, LD_GEMM_DTL_BK, LD_GEMM_DTL_STAGES>), grid, block, 0, s, p); break;
        case G_SWIGLU: hipLaunchKernelGGL((gemm_dtl_kernel<G_SWIGLU, NORM, LD_GEMM_DTL_BK, LD_GEMM_DTL_STAGES>), grid, block, 0, s, p); break;
    }
}

// 128-row tiles with direct-to-LDS slabs
hipError_t gemm_dtl_launch(int kind, const GemmParams& p, hipStream_t s) {
    const long long blocks = (long long)((p.m + 127) / 128) * ((p.n + kBN - 1) / kBN) * p.splits;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    if (kind != G_PLAIN && kind != G_RESID && kind != G_QKV && kind != G_SWIGLU) return hipErrorInvalidValue;
    if (p.gain)
        gemm_dtl_kind<true>(kind, p, dim3((unsigned)blocks), s);
    else
        gemm_dtl_kind<false>(kind, p, dim3((unsigned)blocks), s);
    return gemm_reduce_launch(kind, p, s);
}

// the sum of split partials and the epilogue (after either product kernel)
hipError_t gemm_reduce_launch(int kind, const GemmParams& p, hipStream_t s) {
    const dim3 block(kGemmThreads);
    if (p.splits > 1) {
        const long long threads = (long long)p.m * ((p.n + 1) / 2);
        const dim3 rgrid((unsigned)((threads + 255) / 256));
        switch (kind) {
            case G_PLAIN: hipLaunchKernelGGL(gemm_reduce_kernel<G_PLAIN>, rgrid, block, 0, s, p); break;
            case G_RESID: hipLaunchKernelGGL(gemm_reduce_kernel<G_RESID>, rgrid, block, 0, s, p); break;
            case G_QKV: hipLaunchKernelGGL(gemm_reduce_kernel<G_QKV>, rgrid, block, 0, s, p); break;
            case G_SWIGLU: hipLaunchKernelGGL(gemm_reduce_kernel<G_SWIGLU>, rgrid, block, 0, s, p); break;
        }
    }
    return hipGetLastError();
}

}  // namespace

// Row tile of a product of m rows: the smallest of 16, 32, 64 that holds a
// decode batch (m <= 64, where the weight stream is the cost and the
// matrix-core work per weight byte grows with the tile), 128 above.
int gemm_tile_rows(int m) { return m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : 128; }

// Splits of K for a product with few row tiles (a decode batch): with whole K
// each block would stream its weight rows alone, and a few hundred blocks
// leave most of the chip idle; splitting K gives about 768 blocks (at least
// 256 of K each): three per CU, as many as the 16- and 32-row tiles' LDS lets
// a CU hold, so every block streams from the start and none runs in a second
// round (7B shape: 6.5 against 6.9 ms per step at 16 sequences with 1024
// blocks, 7.3 against 8.0 at 32, 10.7 against 11.4 at 64).  Used only where
// the caller provides the partials' workspace.
#ifndef LD_GEMM_SPLIT_BLOCKS
#define LD_GEMM_SPLIT_BLOCKS 768
#endif
#ifndef LD_GEMM_SPLIT_MINK
#define LD_GEMM_SPLIT_MINK 256
#endif

int gemm_splits(int m, int n, int k) {
    const int bm = gemm_tile_rows(m);
    const long long tiles = (long long)((m + bm - 1) / bm) * ((n + kBN - 1) / kBN);
    if (tiles >= LD_GEMM_SPLIT_BLOCKS) return 1;
    const int sp = (int)((LD_GEMM_SPLIT_BLOCKS + tiles - 1) / tiles);
    return max(1, min(sp, k / LD_GEMM_SPLIT_MINK));
}

// the product partials (splits x m x n) and the row sums of squares of a
// normed product (splits x m)
size_t gemm_part_floats(int m, int n, int k) {
    const int sp = gemm_splits(m, n, k);
    return sp > 1 ? (size_t)sp * m * (n + 1) : 0;
}

// Tiles of gemm_tile_rows rows; split K when a workspace is given
hipError_t gemm_launch(int kind, const GemmParams& p0, hipStream_t s) {
    GemmParams p = p0;
    if (p.m <= 0 || p.n <= 0 || p.k < 4 || (p.k % 4)) return hipErrorInvalidValue;
    p.splits = p.part ? gemm_splits(p.m, p.n, p.k) : 1;
    const int chunk = (p.k + p.splits - 1) / p.splits;
    p.kchunk = (chunk + 31) / 32 * 32;  // a whole number of slabs of either depth
    p.splits = (p.k + p.kchunk - 1) / p.kchunk;
    if (p.splits > 1 && (size_t)p.splits * p.m * (p.n + 1) > p.part_floats) return hipErrorInvalidValue;
    switch (gemm_tile_rows(p.m)) {
        case 16: return gemm_launch_bm<16, LD_GEMM_BK_M16, 16, LD_GEMM_R_BATCH>(kind, p, s);
        case 32: return gemm_launch_bm<32, LD_GEMM_BK_M32, 32, LD_GEMM_R_BATCH>(kind, p, s);
        case 64: return gemm_launch_bm<64, LD_GEMM_BK_M64, 32, LD_GEMM_R_BATCH>(kind, p, s);
    }
#if LD_GEMM_DTL
    return gemm_dtl_launch(kind, p, s);
#else
    return gemm_launch_bm<128, LD_GEMM_BK128, 32, 1>(kind, p, s);
#endif
}

bool attn_prefill_supported(int hs) {
    switch (hs) {
        case 16: case 32: case 48: case 64: case 80: case 96: case 128: case 256: return true;
    }
    return false;
}

hipError_t attn_prefill_launch(int hs, const AttnPrefillParams& p, hipStream_t s) {
    const int ntiles = (p.t + kAQ - 1) / kAQ;
    const dim3 grid((unsigned)(LD_APF_PAIR ? (ntiles + 1) / 2 : ntiles), (unsigned)p.n_heads), block(256);
    switch (hs) {
        case 16: hipLaunchKernelGGL(attn_prefill_kernel<16>, grid, block, 0, s, p); break;
        case 32: hipLaunchKernelGGL(attn_prefill_kernel<32>, grid, block, 0, s, p); break;
        case 48: hipLaunchKernelGGL(attn_prefill_kernel<48>, grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, block, 0, s, p); break;
        case 80: hipLaunchKernelGGL(attn_prefill_kernel<80>, grid, block, 0, s, p); break;
        case 96: hipLaunchKernelGGL(attn_prefill_kernel<96>, grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, block, 0, s, p); break;
        case 256: hipLaunchKernelGGL(attn_prefill_kernel<256>, grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ld
