// Measurement probes: the chip's ceilings at its running clock, which the benchmark
// reports beside the datasheet peaks its roofline fractions use.  Not part of the
// training step.
//   probe_mfma_kernel: independent matrix-core products held in registers (no memory
//     traffic), fp32 16x16x4 or bf16 16x16x32, the shapes the step's kernels use;
//   probe_copy_kernel: a plain float4 copy over a grid of a given size, the bandwidth a
//     streaming kernel can reach.
#include "common.h"
#include "gpt2.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int PROBE_CHAINS = 16;        // independent accumulators per wave
constexpr int PROBE_MAX_BLOCKS = 4096;  // 256-thread blocks: 4 per CU = 4 waves per SIMD
constexpr int PROBE_THREADS = 256;
constexpr int COPY_UNROLL = 4;          // float4s per thread and round of the copy, all loaded first

template <bool BF16>
__global__ __launch_bounds__(PROBE_THREADS) void probe_mfma_kernel(float* __restrict__ out, int iters) {
    f32x4 acc[PROBE_CHAINS];
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float a = 1e-3f * (float)(threadIdx.x & 15), b = 1e-3f * (float)(threadIdx.x >> 4);
    bf16x8 av, bv;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        av[e] = (__bf16)(a + (float)e);
        bv[e] = (__bf16)(b - (float)e);
    }
    for (int i = 0; i < iters; i++) {
#pragma unroll
        for (int j = 0; j < PROBE_CHAINS; j++) {
            if constexpr (BF16)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < PROBE_CHAINS; j++) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
    out[(size_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

// grid-stride copy: each thread moves COPY_UNROLL float4s per round, all loaded before
// any is stored; nontemporal accesses (build option COPY_NT, on: 5.33 against 4.90 TB/s
// at the best grid size)
#ifndef COPY_NT
#define COPY_NT 1
#endif
typedef float cp4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void probe_copy_kernel(float4* __restrict__ dst, const float4* __restrict__ src,
                                                         size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (COPY_UNROLL - 1) * stride < n4; i += COPY_UNROLL * stride) {
        float4 v[COPY_UNROLL];
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; u++) {
            if (COPY_NT) {
                const cp4 t = __builtin_nontemporal_load(reinterpret_cast<const cp4*>(src + i + u * stride));
                v[u] = make_float4(t.x, t.y, t.z, t.w);
            } else {
                v[u] = src[i + u * stride];
            }
        }
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; u++) {
            if (COPY_NT)
                __builtin_nontemporal_store(cp4{v[u].x, v[u].y, v[u].z, v[u].w}, reinterpret_cast<cp4*>(dst + i + u * stride));
            else
                dst[i + u * stride] = v[u];
        }
    }
    for (; i < n4; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

size_t gpt2_probe_mfma_out_floats(void) { return (size_t)PROBE_MAX_BLOCKS * PROBE_THREADS; }

int gpt2_probe_mfma(int kind, int iters, int blocks, float* out, double* flops, void* stream) {
    if ((kind != 0 && kind != 1) || iters < 1 || blocks < 1 || blocks > PROBE_MAX_BLOCKS || !out || !flops)
        return GPT2_EINVAL;
    const double per_mfma = kind == 0 ? 2.0 * 16 * 16 * 4 : 2.0 * 16 * 16 * 32;
    *flops = per_mfma * PROBE_CHAINS * (double)iters * ((double)blocks * (PROBE_THREADS / 64));
    if (kind == 0)
        hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3(blocks), dim3(PROBE_THREADS), 0, (hipStream_t)stream, out,
                           iters);
    else
        hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3(blocks), dim3(PROBE_THREADS), 0, (hipStream_t)stream, out,
                           iters);
    return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_EDEVICE;
}

int gpt2_probe_copy(float* dst, const float* src, size_t n, int blocks, void* stream) {
    if (!dst || !src || n % 4 || blocks < 1 || blocks > 65536 || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15))
        return GPT2_EINVAL;
    if (n == 0) return GPT2_OK;
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<float4*>(dst), reinterpret_cast<const float4*>(src), n / 4);
    return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_EDEVICE;
}

}  // extern "C"
