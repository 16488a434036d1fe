// Causal multi-head self-attention, forward and backward, for gfx950.
//
// The pages name the layer (attention_forward / attention_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1; multi-head in section
// 傻瓜式复现GPT-2).  Per (batch b, head h, query t):
//   s_u = (q_t . k_u) / sqrt(hs) for u <= t,  p = softmax(s),  o_t = sum_u p_u v_u.
// The forward keeps only o and lse_t = max + log(sum exp) per row (O(T) instead of the
// plain O(T^2) score tensors); the backward recomputes p_u = exp(s_u - lse_t).
// Backward: D_t = dO_t . o_t;  dp_u = dO_t . v_u;  ds_u = p_u (dp_u - D_t);
//   dq_t = scale sum_u ds_u k_u;  dk_u = scale sum_t ds_tu q_t;  dv_u = sum_t p_tu dO_t.
// One wave64 per query row (forward, dq) or key row (dk, dv); every output element is
// written by exactly one lane, so no atomics are needed.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

namespace {

GPT2_DEV float dot_row(const float* __restrict__ a_lds, const float* __restrict__ b, int hs) {
    float s = 0.f;
    for (int i = 0; i < hs; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(b + i);
        s += a_lds[i] * v.x + a_lds[i + 1] * v.y + a_lds[i + 2] * v.z + a_lds[i + 3] * v.w;
    }
    return s;
}

__global__ __launch_bounds__(64) void attn_fwd_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                      const float* __restrict__ qkv, int T, int C, int NH) {
    extern __shared__ float sm[];
    float* q = sm;         // [64]
    float* p = sm + 64;    // [T]
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.0f / sqrtf((float)hs);
    const float* base = qkv + (long)b * T * C3;
    if (lane < hs) q[lane] = base[(long)t * C3 + h * hs + lane];
    __syncthreads();
    float mx = -INFINITY;
    for (int u = lane; u <= t; u += 64) {
        const float s = dot_row(q, base + (long)u * C3 + C + h * hs, hs) * scale;
        p[u] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int u = lane; u <= t; u += 64) {
        const float e = expf(p[u] - mx);
        p[u] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    __syncthreads();
    if (lane < hs) {
        float o = 0.f;
        const float* vb = base + 2 * C + h * hs + lane;
        for (int u = 0; u <= t; u++) o += p[u] * vb[(long)u * C3];
        out[((long)b * T + t) * C + h * hs + lane] = o / sum;
    }
    if (lane == 0) lse[((long)b * NH + h) * T + t] = mx + logf(sum);
}

__global__ __launch_bounds__(64) void attn_bwd_dq_kernel(float* __restrict__ dqkv, float* __restrict__ delta,
                                                         const float* __restrict__ dout, const float* __restrict__ qkv,
                                                         const float* __restrict__ out, const float* __restrict__ lse,
                                                         int T, int C, int NH) {
    extern __shared__ float sm[];
    float* q = sm;          // [64]
    float* dO = sm + 64;    // [64]
    float* ds = sm + 128;   // [T]
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.0f / sqrtf((float)hs);
    const float* base = qkv + (long)b * T * C3;
    const long orow = ((long)b * T + t) * C + h * hs;
    float dd = 0.f;
    if (lane < hs) {
        q[lane] = base[(long)t * C3 + h * hs + lane];
        const float g = dout[orow + lane];
        dO[lane] = g;
        dd = g * out[orow + lane];
    }
    const float D = wave_sum(dd);
    __syncthreads();
    const float L = lse[((long)b * NH + h) * T + t];
    for (int u = lane; u <= t; u += 64) {
        const float s = dot_row(q, base + (long)u * C3 + C + h * hs, hs) * scale;
        const float pr = expf(s - L);
        const float dp = dot_row(dO, base + (long)u * C3 + 2 * C + h * hs, hs);
        ds[u] = pr * (dp - D);
    }
    __syncthreads();
    if (lane < hs) {
        float acc = 0.f;
        const float* kb = base + C + h * hs + lane;
        for (int u = 0; u <= t; u++) acc += ds[u] * kb[(long)u * C3];
        dqkv[(long)b * T * C3 + (long)t * C3 + h * hs + lane] = acc * scale;
    }
    if (lane == 0) delta[((long)b * NH + h) * T + t] = D;
}

__global__ __launch_bounds__(64) void attn_bwd_dkdv_kernel(float* __restrict__ dqkv, const float* __restrict__ delta,
                                                           const float* __restrict__ dout, const float* __restrict__ qkv,
                                                           const float* __restrict__ lse, int T, int C, int NH) {
    __shared__ float k[64], v[64], P[64], DS[64];
    const int u = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int hs = C / NH, C3 = 3 * C;
    const float scale = 1.0f / sqrtf((float)hs);
    const float* base = qkv + (long)b * T * C3;
    if (lane < hs) {
        k[lane] = base[(long)u * C3 + C + h * hs + lane];
        v[lane] = base[(long)u * C3 + 2 * C + h * hs + lane];
    }
    __syncthreads();
    float dk = 0.f, dv = 0.f;
    for (int t0 = u; t0 < T; t0 += 64) {
        const int t = t0 + lane;
        float pr = 0.f, dsv = 0.f;
        if (t < T) {
            const float s = dot_row(k, base + (long)t * C3 + h * hs, hs) * scale;
            pr = expf(s - lse[((long)b * NH + h) * T + t]);
            const float dp = dot_row(v, dout + ((long)b * T + t) * C + h * hs, hs);
            dsv = pr * (dp - delta[((long)b * NH + h) * T + t]);
        }
        P[lane] = pr;
        DS[lane] = dsv;
        __syncthreads();
        if (lane < hs) {
            const int n = min(64, T - t0);
            for (int j = 0; j < n; j++) {
                const long r = (long)b * T + t0 + j;
                dv += P[j] * dout[r * C + h * hs + lane];
                dk += DS[j] * base[(long)(t0 + j) * C3 + h * hs + lane];
            }
        }
        __syncthreads();
    }
    if (lane < hs) {
        float* d = dqkv + (long)b * T * C3 + (long)u * C3;
        d[C + h * hs + lane] = dk * scale;
        d[2 * C + h * hs + lane] = dv;
    }
}

}  // namespace

hipError_t attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                             hipStream_t st) {
    const int hs = C / NH;
    if (C % NH || hs > 64 || hs % 4 || T > 65535 || NH > 65535 || B > 65535) return hipErrorInvalidValue;
    if (B * T == 0) return hipSuccess;
    const size_t lds = (64 + (size_t)T) * sizeof(float);
    hipLaunchKernelGGL(attn_fwd_kernel, dim3(T, NH, B), dim3(64), lds, st, out, lse, qkv, T, C, NH);
    return hipGetLastError();
}

hipError_t attention_backward(float* dqkv, float* delta, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C, int NH,
                              hipStream_t st) {
    const int hs = C / NH;
    if (C % NH || hs > 64 || hs % 4 || T > 65535 || NH > 65535 || B > 65535) return hipErrorInvalidValue;
    if (B * T == 0) return hipSuccess;
    const size_t lds = (128 + (size_t)T) * sizeof(float);
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(T, NH, B), dim3(64), lds, st, dqkv, delta, dout, qkv, out, lse, T, C, NH);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(T, NH, B), dim3(64), 0, st, dqkv, (const float*)delta, dout, qkv, lse, T, C, NH);
    return hipGetLastError();
}

}  // namespace gpt2k
