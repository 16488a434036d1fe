// Softmax + cross-entropy over the vocabulary, for gfx950.
//
// The pages list softmax_forward, crossentropy_forward and the fused
// crossentropy_softmax_backward (huxiu page "llm.c：Andrej Karpathy带你从零复现LLM",
// 核心代码解读 item 1).  Rows are V = 50257 floats.  The LM-head forward GEMM's
// epilogue leaves, for each tile and row, the (max, sum of exp) of its columns; here
// those partials are merged into lse = max + log(sum) per row, and the loss is
// lse - z[target] = -log softmax(z)[target].  Nothing else is written: the
// probabilities exp(z - lse) and the logits' gradient (p - onehot)/rows are formed by
// the LM-head backward GEMMs as they load the logits, which saves writing and
// re-reading two 1.6 GB tensors.  Rows are padded to a multiple of 64 floats so every
// row starts 256-byte aligned.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

// Log-sum-exp from the LM-head forward's partials: (max, sum) pairs in base 2, stored
// [part][row].  A block takes 64 rows; wave q merges parts q, q+16, ... of each row (a
// wave's loads cover 64 consecutive rows: 512 contiguous bytes), then the sixteen waves'
// results are merged in LDS, in order.  With 8192 rows and ~800 parts a row, sixteen
// waves per block keep each thread's chain of dependent loads short (four waves: 26 us
// per launch, about 2.5x a copy of the same bytes).
constexpr int LC_ROWS = 64, LC_WAVES = 16;
GPT2_DEV void merge2(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = s * __builtin_amdgcn_exp2f(m - M) + s2 * __builtin_amdgcn_exp2f(m2 - M);
    m = M;
}

__global__ __launch_bounds__(LC_ROWS * LC_WAVES) void lse_combine_kernel(
    const float2* __restrict__ part, int parts, const float* __restrict__ logits, long ld, float* __restrict__ lse,
    float* __restrict__ losses, const int32_t* __restrict__ targets, int N, int V, int* flags) {
    __shared__ float sm_m[LC_WAVES][LC_ROWS], sm_s[LC_WAVES][LC_ROWS];
    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int row = blockIdx.x * LC_ROWS + lane;
    float m = -INFINITY, s = 0.f;
    if (row < N) {
        int pi = q;
        for (; pi + LC_WAVES * 7 < parts; pi += LC_WAVES * 8) {
            float2 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = part[(long)(pi + LC_WAVES * u) * N + row];
#pragma unroll
            for (int u = 0; u < 8; u++) merge2(m, s, v[u].x, v[u].y);
        }
        for (; pi < parts; pi += LC_WAVES) {
            const float2 v = part[(long)pi * N + row];
            merge2(m, s, v.x, v.y);
        }
    }
    sm_m[q][lane] = m;
    sm_s[q][lane] = s;
    __syncthreads();
    if (q == 0 && row < N) {
        for (int w = 1; w < LC_WAVES; w++) merge2(m, s, sm_m[w][lane], sm_s[w][lane]);
        const float L = (m + __builtin_amdgcn_logf(s)) * 0.6931471805599453f;
        lse[row] = L;
        if (targets) {
            const int tgt = targets[row];
            if (tgt < 0 || tgt >= V) {
                atomicOr(flags, ERR_BAD_TARGET_TOKEN);
                losses[row] = NAN;
            } else {
                losses[row] = L - logits[(long)row * ld + tgt];
            }
        }
    }
}

// Mean in double, fixed order: strided per-thread sums, then a tree in LDS.
__global__ __launch_bounds__(256) void loss_mean_kernel(float* out, const float* __restrict__ losses, int N) {
    __shared__ double sm[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < N; i += 256) s += (double)losses[i];
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = (float)(sm[0] / (double)N);
}

// Next-token sampling (the pages' sample_mult: huxiu page "llm.c：Andrej Karpathy带你从零复现
// LLM", 核心代码解读 item 5): the token is the smallest index j whose cumulative
// probability sum_{k<=j} p_k exceeds the coin (the last index when rounding leaves the
// total below it).  One 1024-thread block per request: p_k = exp(z_k - lse) in fp32
// from the stored log-sum-exp; each thread sums a contiguous chunk in fp64, a block scan
// gives every chunk its starting cumulative sum, and the thread whose range holds the
// coin walks its chunk.  The decision is taken on fp64 sums of the fp32 probabilities,
// so it does not depend on the chunking beyond ~1e-16.
constexpr int SAMPLE_THREADS = 1024;

__global__ __launch_bounds__(SAMPLE_THREADS) void sample_kernel(const float* __restrict__ logits, long ld,
                                                                const float* __restrict__ lse,
                                                                const int32_t* __restrict__ rows,
                                                                const float* __restrict__ coins, int V,
                                                                int32_t* __restrict__ tokens) {
    __shared__ double part[SAMPLE_THREADS];
    const int t = threadIdx.x;
    const long row = rows[blockIdx.x];
    const double coin = coins[blockIdx.x];
    const float* z = logits + row * ld;
    const float L = lse[row];
    const int chunk = (V + SAMPLE_THREADS - 1) / SAMPLE_THREADS;
    const int j0 = min(V, t * chunk), j1 = min(V, j0 + chunk);
    double s = 0.0;
    for (int j = j0; j < j1; j++) s += (double)expf(z[j] - L);
    // inclusive scan of the chunk sums (fixed order: Hillis-Steele over the block)
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < SAMPLE_THREADS; off <<= 1) {
        const double add = t >= off ? part[t - off] : 0.0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    // chunk t covers [part[t-1], part[t]): consecutive ranges share their bounds exactly
    const double hi = part[t], lo = t > 0 ? part[t - 1] : 0.0;
    const double total = part[SAMPLE_THREADS - 1];
    if (coin >= total) {
        if (t == 0) tokens[blockIdx.x] = V - 1;
        return;
    }
    if (lo <= coin && coin < hi) {
        // exactly one thread's [lo, hi) holds the coin
        double c = lo;
        int pick = j1 - 1;
        for (int j = j0; j < j1; j++) {
            c += (double)expf(z[j] - L);
            if (coin < c) {
                pick = j;
                break;
            }
        }
        tokens[blockIdx.x] = pick;
    }
}

}  // namespace

hipError_t sample_tokens(const float* logits, long ld, const float* lse, const int32_t* rows, const float* coins,
                         int n, int V, int32_t* tokens, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    ProfScope ps(st, "sample_kernel", 0.0, 4.0 * n * ((double)V + 3));
    hipLaunchKernelGGL(sample_kernel, dim3(n), dim3(SAMPLE_THREADS), 0, st, logits, ld, lse, rows, coins, V, tokens);
    return hipGetLastError();
}


hipError_t lse_combine(const float* lse_part, int parts, const float* logits, long ld, float* lse, float* losses,
                       const int32_t* targets, int N, int V, int* flags, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    if (parts <= 0 || ((uintptr_t)lse_part & 7)) return hipErrorInvalidValue;
    ProfScope ps(st, "lse_combine_kernel", 0.0, 8.0 * (double)N * parts + 12.0 * N);
    hipLaunchKernelGGL(lse_combine_kernel, dim3((N + LC_ROWS - 1) / LC_ROWS), dim3(LC_ROWS * LC_WAVES), 0, st,
                       reinterpret_cast<const float2*>(lse_part), parts, logits, ld, lse, losses, targets, N, V,
                       flags);
    return hipGetLastError();
}

hipError_t loss_mean(float* out, const float* losses, int N, hipStream_t st) {
    hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(256), 0, st, out, losses, N);
    return hipGetLastError();
}

}  // namespace gpt2k
