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

}  // namespace

hipError_t lse_xent_forward(const float* logits, long ld, float* lse, float* losses, const int32_t* targets,
                            int N, int V, int* flags, hipStream_t st) {
    if (ld % 4 || ld < V) return hipErrorInvalidValue;
    if (N == 0) return hipSuccess;
    ProfScope ps(st, "lse_xent_kernel", 0.0, 4.0 * ((double)N * V + 2.0 * N));
    hipLaunchKernelGGL(lse_xent_kernel, dim3(N), dim3(SX_THREADS), 0, st, logits, ld, lse, losses, targets, V, flags);
    return hipGetLastError();
}

hipError_t loss_mean(float* out, const float* losses, int N, hipStream_t st) {
    hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(256), 0, st, out, losses, N);
    return hipGetLastError();
}

}  // namespace gpt2k
