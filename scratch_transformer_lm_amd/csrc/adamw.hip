// AdamW over the flat parameter buffer, and a zero fill, for gfx950.
//
// The update is the pages' gpt2_update (AdamW: huxiu page "llm.c：Andrej Karpathy带你从零
// 复现LLM", 核心代码解读 item 3).  One pass reads p, g, m, v and writes p, m, v
// (28 bytes per parameter), float4-wide, each block one tile of 1024 float4s with all of
// a thread's loads issued before its arithmetic.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

// Build option: the optimizer-only streams (g read; m, v read and written) as nontemporal
// accesses (1), or as ordinary ones (0).  Measured over the 124M buffer: 5.69 against
// 5.36 TB/s.  p stays ordinary: the next forward reads it.
#ifndef ADAM_NT
#define ADAM_NT 1
#endif
typedef float nt4 __attribute__((ext_vector_type(4)));
GPT2_DEV float4 ld_s(const float4* a) {
    if (ADAM_NT) {
        const nt4 t = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(a));
        return make_float4(t.x, t.y, t.z, t.w);
    }
    return *a;
}
GPT2_DEV void st_s(float4* a, float4 v) {
    if (ADAM_NT) __builtin_nontemporal_store(nt4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt4*>(a));
    else *a = v;
}

// One element.  ibc1, ibc2 are the reciprocals of the bias corrections 1 - b^t.
GPT2_DEV void adam_one(float& p, float g, float& m, float& v, float lr, float b1, float b2, float eps,
                       float wd, float ibc1, float ibc2) {
    m = b1 * m + (1.0f - b1) * g;
    v = b2 * v + (1.0f - b2) * g * g;
    const float mh = m * ibc1;
    const float vh = v * ibc2;
    p -= lr * (mh / (sqrtf(vh) + eps) + wd * p);
}

GPT2_DEV void adam_four(float4* __restrict__ p, const float4* __restrict__ g, float4* __restrict__ m,
                        float4* __restrict__ v, size_t j, float lr, float b1, float b2, float eps, float wd,
                        float ibc1, float ibc2, float4& pp, float4 gg, float4& mm, float4& vv) {
    adam_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, ibc1, ibc2);
    adam_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, ibc1, ibc2);
    adam_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, ibc1, ibc2);
    adam_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, ibc1, ibc2);
    p[j] = pp;
    st_s(m + j, mm);
    st_s(v + j, vv);
}

// A block updates one tile of ADAM_TILE float4s of one contiguous range: ADAM_UNROLL
// float4s of each of p, g, m, v per thread, all requested before any is used.
constexpr int ADAM_UNROLL = 4;
constexpr int ADAM_TILE = 256 * ADAM_UNROLL;

GPT2_DEV void adam_tile(float* p_, const float* g_, float* m_, float* v_, size_t base4, size_t end4, float lr,
                        float b1, float b2, float eps, float wd, float ibc1, float ibc2) {
    float4* p = reinterpret_cast<float4*>(p_);
    const float4* g = reinterpret_cast<const float4*>(g_);
    float4* m = reinterpret_cast<float4*>(m_);
    float4* v = reinterpret_cast<float4*>(v_);
    float4 pp[ADAM_UNROLL], gg[ADAM_UNROLL], mm[ADAM_UNROLL], vv[ADAM_UNROLL];
#pragma unroll
    for (int u = 0; u < ADAM_UNROLL; u++) {
        const size_t j = base4 + (size_t)u * 256 + threadIdx.x;
        if (j < end4) {
            pp[u] = p[j];
            gg[u] = ld_s(g + j);
            mm[u] = ld_s(m + j);
            vv[u] = ld_s(v + j);
        }
    }
#pragma unroll
    for (int u = 0; u < ADAM_UNROLL; u++) {
        const size_t j = base4 + (size_t)u * 256 + threadIdx.x;
        if (j < end4) adam_four(p, g, m, v, j, lr, b1, b2, eps, wd, ibc1, ibc2, pp[u], gg[u], mm[u], vv[u]);
    }
}

// The whole flat buffer: block b takes float4s [b ADAM_TILE, (b+1) ADAM_TILE); the last
// n % 4 floats go to block 0 one by one.
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, size_t n,
                                                    float lr, float b1, float b2, float eps, float wd, float ibc1,
                                                    float ibc2) {
    const size_t n4 = n / 4;
    adam_tile(p, g, m, v, (size_t)blockIdx.x * ADAM_TILE, n4, lr, b1, b2, eps, wd, ibc1, ibc2);
    if (blockIdx.x == 0)
        for (size_t i = 4 * n4 + threadIdx.x; i < n; i += blockDim.x)
            adam_one(p[i], g[i], m[i], v[i], lr, b1, b2, eps, wd, ibc1, ibc2);
}

// The same update over up to ADAM_MAX_SEGS disjoint slices of the flat buffers (one
// layer's parameter tensors), all starting on float4 boundaries with lengths that are
// multiples of 4.  Each slice is cut into ADAM_TILE-float4 tiles; segs.start4[s] holds
// the first tile of slice s (and start4[n] the tile count), so a block finds its slice
// with one scan.
__global__ __launch_bounds__(256) void adamw_segments_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                             float* __restrict__ m, float* __restrict__ v,
                                                             AdamSegments segs, float lr, float b1, float b2,
                                                             float eps, float wd, float ibc1, float ibc2) {
    const size_t t = blockIdx.x;
    int s = 0;
    while (s + 1 < segs.n && segs.start4[s + 1] <= t) s++;
    const size_t base4 = segs.off4[s] + (t - segs.start4[s]) * ADAM_TILE;
    adam_tile(p, g, m, v, base4, segs.off4[s] + segs.len4[s], lr, b1, b2, eps, wd, ibc1, ibc2);
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
    const size_t tiles = std::max<size_t>(1, (n / 4 + ADAM_TILE - 1) / ADAM_TILE);
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    ProfScope ps(st, "adamw_kernel", 0.0, 28.0 * (double)n);
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)tiles), dim3(256), 0, st, p, g, m, v, n, lr, b1, b2, eps, wd,
                       1.0f / bc1, 1.0f / bc2);
    return hipGetLastError();
}

hipError_t adamw_segments(float* p, const float* g, float* m, float* v, const size_t* off, const size_t* len, int n,
                          float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t st) {
    if (n < 0 || n > ADAM_MAX_SEGS) return hipErrorInvalidValue;
    AdamSegments segs{};
    segs.n = n;
    size_t tiles = 0, total = 0;
    for (int i = 0; i < n; i++) {
        if (off[i] % 4 || len[i] % 4) return hipErrorInvalidValue;
        segs.off4[i] = off[i] / 4;
        segs.len4[i] = len[i] / 4;
        segs.start4[i] = tiles;
        tiles += (len[i] / 4 + ADAM_TILE - 1) / ADAM_TILE;
        total += len[i] / 4;
    }
    segs.start4[n] = tiles;
    if (tiles == 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    ProfScope ps(st, "adamw_segments_kernel", 0.0, 28.0 * 4.0 * (double)total);
    hipLaunchKernelGGL(adamw_segments_kernel, dim3((unsigned)tiles), dim3(256), 0, st, p, g, m, v, segs, lr, b1, b2,
                       eps, wd, 1.0f / bc1, 1.0f / bc2);
    return hipGetLastError();
}

hipError_t fill_zero(float* x, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    ProfScope ps(st, "zero_kernel", 0.0, 4.0 * (double)n);
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n / 4 + 1)), dim3(256), 0, st, x, n);
    return hipGetLastError();
}

}  // namespace gpt2k
