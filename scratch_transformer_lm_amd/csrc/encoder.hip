// Token + position embedding, forward and backward, for gfx950.
//
// The pages name the layer (encoder_forward / encoder_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1): out = wte[token] + wpe[t].
// The backward is a scatter-add into the wte rows that were read.  Token frequencies
// are skewed (a few ids fill a large share of the positions), so instead of float
// atomics, which would serialise on the hot rows and make the sums order-dependent,
// the backward finds the first position of every distinct id and lets one block own
// that id: it walks the later positions in order and adds their rows.  Results are
// therefore bitwise reproducible.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int STAGE = 4096;  // tokens staged in LDS per pass

__global__ __launch_bounds__(256) void encoder_fwd_kernel(float* __restrict__ out, const int32_t* __restrict__ tok,
                                                          const float* __restrict__ wte, const float* __restrict__ wpe,
                                                          int BT, int T, int C, int V, int* flags) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= BT) return;
    int id = tok[row];
    if (id < 0 || id >= V) {
        if (lane == 0) atomicOr(flags, ERR_BAD_INPUT_TOKEN);
        id = 0;
    }
    const int t = row % T;
    const float4* we = reinterpret_cast<const float4*>(wte + (long)id * C);
    const float4* pe = reinterpret_cast<const float4*>(wpe + (long)t * C);
    float4* o = reinterpret_cast<float4*>(out + (long)row * C);
    for (int i = lane; i < C / 4; i += 64) {
        const float4 a = we[i], b = pe[i];
        o[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
}

// dwpe[t] += sum_b dout[b, t] (b in order); one thread per 4 channels of one t.
__global__ __launch_bounds__(256) void wpe_bwd_kernel(float* __restrict__ dwpe, const float* __restrict__ dout,
                                                      int B, int T, int C) {
    const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
    const int C4 = C / 4;
    if (i >= (long)T * C4) return;
    const int t = (int)(i / C4), c4 = (int)(i - (long)t * C4);
    float4 acc = reinterpret_cast<float4*>(dwpe + (long)t * C)[c4];
    for (int b = 0; b < B; b++) {
        const float4 d = reinterpret_cast<const float4*>(dout + ((long)b * T + t) * C)[c4];
        acc.x += d.x;
        acc.y += d.y;
        acc.z += d.z;
        acc.w += d.w;
    }
    reinterpret_cast<float4*>(dwpe + (long)t * C)[c4] = acc;
}

// For each position p, is it the first position holding its token id?  Such positions
// are appended to list (slot order does not matter: each one is processed alone).
// work[0] is the list length and must be 0 on entry.
__global__ __launch_bounds__(256) void first_occurrence_kernel(int* work, const int32_t* __restrict__ tok, int BT) {
    __shared__ int s[STAGE];
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    const int v = p < BT ? tok[p] : -1;
    const int pmax = min(BT, (int)((blockIdx.x + 1) * blockDim.x));
    int found = 0;
    for (int base = 0; base < pmax; base += STAGE) {
        const int n = min(STAGE, pmax - base);
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) s[i] = tok[base + i];
        __syncthreads();
        const int lim = min(n, p - base);
        for (int i = 0; i < lim; i++) found |= (s[i] == v);
    }
    if (p < BT && !found) {
        const int slot = atomicAdd(work, 1);
        work[1 + slot] = p;
    }
}

// Block k owns the k-th listed first position p: dwte[tok[p]] += sum of dout[q] over
// q >= p with the same id, q increasing.
__global__ __launch_bounds__(256) void wte_bwd_kernel(float* __restrict__ dwte, const float* __restrict__ dout,
                                                      const int32_t* __restrict__ tok, const int* __restrict__ work,
                                                      int BT, int C) {
    __shared__ unsigned long long masks[4];
    if ((int)blockIdx.x >= work[0]) return;
    const int p = work[1 + blockIdx.x];
    const int v = tok[p];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int C4 = C / 4;
    float4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = p; base < BT; base += 256) {
        const int q = base + threadIdx.x;
        const bool hit = q < BT && tok[q] == v;
        const unsigned long long m = __ballot(hit);
        if (lane == 0) masks[wave] = m;
        __syncthreads();
        for (int w = 0; w < 4; w++) {
            unsigned long long mm = masks[w];
            while (mm) {
                const int bit = __ffsll((long long)mm) - 1;
                mm &= mm - 1;
                const float4* row = reinterpret_cast<const float4*>(dout + (long)(base + w * 64 + bit) * C);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int c = threadIdx.x + 256 * j;
                    if (c < C4) {
                        const float4 d = row[c];
                        acc[j].x += d.x;
                        acc[j].y += d.y;
                        acc[j].z += d.z;
                        acc[j].w += d.w;
                    }
                }
            }
        }
        __syncthreads();
    }
    float4* dst = reinterpret_cast<float4*>(dwte + (long)v * C);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int c = threadIdx.x + 256 * j;
        if (c < C4) {
            float4 o = dst[c];
            o.x += acc[j].x;
            o.y += acc[j].y;
            o.z += acc[j].z;
            o.w += acc[j].w;
            dst[c] = o;
        }
    }
}

__global__ void zero_int_kernel(int* x) { *x = 0; }

}  // namespace

hipError_t encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe,
                           int B, int T, int C, int V, int* flags, hipStream_t st) {
    const int BT = B * T;
    if (C % 4) return hipErrorInvalidValue;
    if (BT == 0) return hipSuccess;
    ProfScope ps(st, "encoder_fwd_kernel", 0.0, 4.0 * ((double)BT * C * 3 + BT));
    hipLaunchKernelGGL(encoder_fwd_kernel, dim3((BT + 3) / 4), dim3(256), 0, st, out, tok, wte, wpe, BT, T, C, V, flags);
    return hipGetLastError();
}

// `work` is an int scratch of 1 + B*T entries.
hipError_t encoder_backward_ws(float* dwte, float* dwpe, const float* dout, const int32_t* tok,
                               int B, int T, int C, int* work, hipStream_t st) {
    const int BT = B * T;
    if (C % 4 || C > 4096) return hipErrorInvalidValue;
    if (BT == 0) return hipSuccess;
    const long n = (long)T * (C / 4);
    {
        ProfScope ps(st, "wpe_bwd_kernel", 0.0, 4.0 * ((double)BT * C + 2.0 * T * C));
        hipLaunchKernelGGL(wpe_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dwpe, dout, B, T, C);
    }
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, work);
    {
        ProfScope ps(st, "first_occurrence_kernel", 0.0, 4.0 * BT);
        hipLaunchKernelGGL(first_occurrence_kernel, dim3((BT + 255) / 256), dim3(256), 0, st, work, tok, BT);
    }
    // rows of dout read once; each touched wte row read and written once (at most BT rows)
    ProfScope ps(st, "wte_bwd_kernel", 0.0, 4.0 * ((double)BT * C + BT));
    hipLaunchKernelGGL(wte_bwd_kernel, dim3(BT), dim3(256), 0, st, dwte, dout, tok, (const int*)work, BT, C);
    return hipGetLastError();
}

}  // namespace gpt2k
