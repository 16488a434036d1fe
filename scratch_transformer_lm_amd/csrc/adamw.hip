// AdamW over the flat parameter buffer, and a zero fill, for gfx950.
//
// The update is the pages' gpt2_update (AdamW: huxiu page "llm.c：Andrej Karpathy带你从零
// 复现LLM", 核心代码解读 item 3).  One pass reads p, g, m, v and writes p, m, v
// (28 bytes per parameter), float4-wide with a grid-stride loop sized to the chip.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

GPT2_DEV void adam_one(float& p, float g, float& m, float& v, float lr, float b1, float b2, float eps,
                       float wd, float bc1, float bc2) {
    m = b1 * m + (1.0f - b1) * g;
    v = b2 * v + (1.0f - b2) * g * g;
    const float mh = m / bc1;
    const float vh = v / bc2;
    p -= lr * (mh / (sqrtf(vh) + eps) + wd * p);
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, size_t n,
                                                    float lr, float b1, float b2, float eps, float wd, float bc1,
                                                    float bc2) {
    const size_t n4 = n / 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 pp = reinterpret_cast<float4*>(p)[i];
        const float4 gg = reinterpret_cast<const float4*>(g)[i];
        float4 mm = reinterpret_cast<float4*>(m)[i];
        float4 vv = reinterpret_cast<float4*>(v)[i];
        adam_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, bc1, bc2);
        reinterpret_cast<float4*>(p)[i] = pp;
        reinterpret_cast<float4*>(m)[i] = mm;
        reinterpret_cast<float4*>(v)[i] = vv;
    }
    for (size_t i = 4 * n4 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride)
        adam_one(p[i], g[i], m[i], v[i], lr, b1, b2, eps, wd, bc1, bc2);
}

// The same update over up to ADAM_MAX_SEGS disjoint slices of the flat buffers (one
// layer's parameter tensors), all starting on float4 boundaries with lengths that are
// multiples of 4: float4 index i of the concatenation lies in the segment whose running
// start is the last one <= i.
__global__ __launch_bounds__(256) void adamw_segments_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                             float* __restrict__ m, float* __restrict__ v,
                                                             AdamSegments segs, float lr, float b1, float b2,
                                                             float eps, float wd, float bc1, float bc2) {
    const size_t total = segs.start4[segs.n];
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += stride) {
        int s = 0;
        while (s + 1 < segs.n && segs.start4[s + 1] <= i) s++;
        const size_t j = segs.off4[s] + (i - segs.start4[s]);
        float4 pp = reinterpret_cast<float4*>(p)[j];
        const float4 gg = reinterpret_cast<const float4*>(g)[j];
        float4 mm = reinterpret_cast<float4*>(m)[j];
        float4 vv = reinterpret_cast<float4*>(v)[j];
        adam_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, bc1, bc2);
        adam_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, bc1, bc2);
        reinterpret_cast<float4*>(p)[j] = pp;
        reinterpret_cast<float4*>(m)[j] = mm;
        reinterpret_cast<float4*>(v)[j] = vv;
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ x, size_t n) {
    const size_t n4 = n / 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += stride)
        reinterpret_cast<float4*>(x)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (size_t i = 4 * n4 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

unsigned grid_for(size_t n4) {
    // Enough blocks for 8 waves on each of the 256 CUs, fewer for small buffers.
    const size_t want = (n4 + 255) / 256;
    return (unsigned)std::max<size_t>(1, std::min<size_t>(want, 256 * 8));
}

}  // namespace

hipError_t adamw(float* p, const float* g, float* m, float* v, size_t n, float lr, float b1,
                 float b2, float eps, float wd, float bc1, float bc2, hipStream_t st) {
    if (n == 0) return hipSuccess;
    ProfScope ps(st, "adamw_kernel", 0.0, 28.0 * (double)n);
    hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(n / 4 + 1)), dim3(256), 0, st, p, g, m, v, n, lr, b1, b2, eps, wd, bc1, bc2);
    return hipGetLastError();
}

hipError_t adamw_segments(float* p, const float* g, float* m, float* v, const size_t* off, const size_t* len, int n,
                          float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t st) {
    if (n < 0 || n > ADAM_MAX_SEGS) return hipErrorInvalidValue;
    AdamSegments segs{};
    segs.n = n;
    size_t total = 0;
    for (int i = 0; i < n; i++) {
        if (off[i] % 4 || len[i] % 4) return hipErrorInvalidValue;
        segs.off4[i] = off[i] / 4;
        segs.start4[i] = total;
        total += len[i] / 4;
    }
    segs.start4[n] = total;
    if (total == 0) return hipSuccess;
    ProfScope ps(st, "adamw_segments_kernel", 0.0, 28.0 * 4.0 * (double)total);
    hipLaunchKernelGGL(adamw_segments_kernel, dim3(grid_for(total)), dim3(256), 0, st, p, g, m, v, segs, lr, b1, b2,
                       eps, wd, bc1, bc2);
    return hipGetLastError();
}

hipError_t fill_zero(float* x, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    ProfScope ps(st, "zero_kernel", 0.0, 4.0 * (double)n);
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n / 4 + 1)), dim3(256), 0, st, x, n);
    return hipGetLastError();
}

}  // namespace gpt2k
