// Softmax + cross-entropy over the vocabulary, for gfx950.
//
// The pages list softmax_forward, crossentropy_forward and the fused
// crossentropy_softmax_backward (huxiu page "llm.c：Andrej Karpathy带你从零复现LLM",
// 核心代码解读 item 1).  Rows are V = 50257 floats, far too long for one wave, so a
// 256-thread block owns a row and keeps a running (max, sum of exp) per thread
// (rescaling the sum when the max grows); the block merges the pairs into
// lse = max + log(sum).  The loss is lse - z[target] = -log softmax(z)[target].
// Nothing else is written: the probabilities exp(z - lse) and the logits' gradient
// (p - onehot)/rows are formed by the LM-head backward GEMMs as they load the logits,
// which saves writing and re-reading two 1.6 GB tensors.  Rows are padded to a multiple
// of 64 floats so every row starts 256-byte aligned.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int SX_THREADS = 256;

GPT2_DEV void online_add(float& m, float& s, float x) {
    if (x > m) {
        s = s * expf(m - x) + 1.0f;
        m = x;
    } else {
        s += expf(x - m);
    }
}

GPT2_DEV void online_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = s * expf(m - M) + s2 * expf(m2 - M);
    m = M;
}

__global__ __launch_bounds__(SX_THREADS) void lse_xent_kernel(const float* __restrict__ logits, long ld,
                                                              float* __restrict__ lse, float* __restrict__ losses,
                                                              const int32_t* __restrict__ targets, int V,
                                                              int* flags) {
    __shared__ float sm_m[SX_THREADS / 64], sm_s[SX_THREADS / 64];
    const long row = blockIdx.x;
    const float* z = logits + row * ld;
    const int V4 = V >> 2;
    float m = -INFINITY, s = 0.f;
    for (int i = threadIdx.x; i < V4; i += SX_THREADS) {
        const float4 v = reinterpret_cast<const float4*>(z)[i];
        online_add(m, s, v.x);
        online_add(m, s, v.y);
        online_add(m, s, v.z);
        online_add(m, s, v.w);
    }
    for (int i = 4 * V4 + threadIdx.x; i < V; i += SX_THREADS) online_add(m, s, z[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        online_merge(m, s, m2, s2);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        sm_m[wave] = m;
        sm_s[wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = sm_m[0], S = sm_s[0];
        for (int w = 1; w < SX_THREADS / 64; w++) online_merge(M, S, sm_m[w], sm_s[w]);
        const float L = logf(S) + M;
        lse[row] = L;
        if (targets) {
            const int tgt = targets[row];
            if (tgt < 0 || tgt >= V) {
                atomicOr(flags, ERR_BAD_TARGET_TOKEN);
                losses[row] = NAN;
            } else {
                losses[row] = L - z[tgt];
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

hipError_t lse_xent_forward(const float* logits, long ld, float* lse, float* losses, const int32_t* targets,
                            int N, int V, int* flags, hipStream_t st) {
    if (ld % 4 || ld < V) return hipErrorInvalidValue;
    if (N == 0) return hipSuccess;
    ProfScope ps(st, "lse_xent_kernel", 0.0, 4.0 * ((double)N * V + 2.0 * N));
    hipLaunchKernelGGL(lse_xent_kernel, dim3(N), dim3(SX_THREADS), 0, st, logits, ld, lse, losses, targets, V, flags);
    return hipGetLastError();
}

hipError_t sample_tokens(const float* logits, long ld, const float* lse, const int32_t* rows, const float* coins,
                         int n, int V, int32_t* tokens, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    ProfScope ps(st, "sample_kernel", 0.0, 4.0 * n * ((double)V + 3));
    hipLaunchKernelGGL(sample_kernel, dim3(n), dim3(SAMPLE_THREADS), 0, st, logits, ld, lse, rows, coins, V, tokens);
    return hipGetLastError();
}

hipError_t loss_mean(float* out, const float* losses, int N, hipStream_t st) {
    hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(256), 0, st, out, losses, N);
    return hipGetLastError();
}

}  // namespace gpt2k
