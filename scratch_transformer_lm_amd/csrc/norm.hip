// LayerNorm forward/backward for gfx950.
//
// LayerNorm is the pages' worked example of a hand-written layer ("OpenAI创始大神手搓
// 千行C代码训练GPT", 手动实现每个层前向 / 反向传播; 新智元 article, 教程).  Both
// directions are HBM-bound: one wave64 owns a row, holds it in registers as float4s,
// and reduces with cross-lane shuffles; nothing is re-read from memory.  The
// cross-row sums (dgamma, dbeta) go through per-block partial rows that a
// second kernel adds in a fixed order, so results are deterministic.
//
// RMS = true gives RMSNorm, the Llama-style variant (published definition; the pages only
// name those model families): no mean subtraction and no bias, r = 1/sqrt(mean(x^2) +
// eps), y = x r w; the mean slot is written as 0, so the backward's x_hat = (x - mean) r
// is the same expression, and dx = r (g - x_hat mean(g x_hat)) with no dbeta.
#include <mutex>

#include "common.h"
#include "gpt2.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int ROWS_PER_BLOCK = 4;  // one wave per row, 256 threads
// The backward's grid is capped: each block leaves one partial [dgamma | dbeta] row.
#ifndef LN_BWD_MAX_BLOCKS
#define LN_BWD_MAX_BLOCKS 512
#endif
constexpr int LN_MAX_BLOCKS = LN_BWD_MAX_BLOCKS;
// Waves (rows in flight) per block of the backward (8 measured no faster at 8192 x 768:
// 21.0 against 20.8 us per launch).
#ifndef LN_BWD_WAVES
#define LN_BWD_WAVES 4
#endif
constexpr int BWD_WAVES = LN_BWD_WAVES;

// Rows per wave of the forward: a wave loads all of its rows before reducing any, so
// more bytes are in flight per wave and fewer blocks are dispatched.
#ifndef LN_FWD_ROWS
#define LN_FWD_ROWS 1
#endif

template <int VPL, bool RMS, int RPW>
__global__ __launch_bounds__(256) void ln_fwd_kernel(float* __restrict__ y, uint16_t* __restrict__ yb,
                                                     float* __restrict__ mean,
                                                     float* __restrict__ rstd, const float* __restrict__ x,
                                                     const float* __restrict__ w, const float* __restrict__ b,
                                                     int N, int C, float eps) {
    const int row0 = (blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6)) * RPW;
    const int lane = threadIdx.x & 63;
    if (row0 >= N) return;
    const int C4 = C >> 2;
    float4 v[RPW][VPL];
#pragma unroll
    for (int q = 0; q < RPW; q++) {
        const float4* xr = reinterpret_cast<const float4*>(x + (long)(row0 + q) * C);
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            v[q][j] = (i < C4 && row0 + q < N) ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const float4* w4 = reinterpret_cast<const float4*>(w);
    const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
    for (int q = 0; q < RPW; q++) {
        const int row = row0 + q;
        if (row >= N) break;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < VPL; j++) s += (v[q][j].x + v[q][j].y) + (v[q][j].z + v[q][j].w);
        const float m = RMS ? 0.f : wave_sum(s) / (float)C;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            if (i < C4) {
                const float a = v[q][j].x - m, bb = v[q][j].y - m, c = v[q][j].z - m, d = v[q][j].w - m;
                ss += (a * a + bb * bb) + (c * c + d * d);
            }
        }
        const float var = wave_sum(ss) / (float)C;
        const float r = 1.0f / sqrtf(var + eps);
        float4* yr = reinterpret_cast<float4*>(y + (long)row * C);
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            if (i < C4) {
                const float4 ww = w4[i], bv = RMS ? make_float4(0.f, 0.f, 0.f, 0.f) : b4[i];
                float4 o;
                o.x = (v[q][j].x - m) * r * ww.x + bv.x;
                o.y = (v[q][j].y - m) * r * ww.y + bv.y;
                o.z = (v[q][j].z - m) * r * ww.z + bv.z;
                o.w = (v[q][j].w - m) * r * ww.w + bv.w;
                yr[i] = o;
                if (yb)
                    reinterpret_cast<uint2*>(yb + (long)row * C)[i] =
                        make_uint2(bf16_pack2(o.x, o.y), bf16_pack2(o.z, o.w));
            }
        }
        if (lane == 0) {
            mean[row] = m;
            rstd[row] = r;
        }
    }
}

// dx = rstd * (g - mean(g) - xh * mean(g*xh)), g = w*dy, xh = (x-mean)*rstd.
// Each block also leaves one partial row [dw | db] (2C floats) in `partial`.
template <int VPL, bool RMS>
__global__ __launch_bounds__(64 * BWD_WAVES) void ln_bwd_kernel(float* __restrict__ dx, float* __restrict__ partial,
                                                     const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ w, const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, int N, int C, int accumulate) {
    extern __shared__ float red[];  // [BWD_WAVES][C]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int C4 = C >> 2;
    const float4* w4 = reinterpret_cast<const float4*>(w);
    float4 wv[VPL], pdw[VPL], pdb[VPL];
#pragma unroll
    for (int j = 0; j < VPL; j++) {
        const int i = lane + 64 * j;
        wv[j] = i < C4 ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        pdw[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        pdb[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int row = blockIdx.x * BWD_WAVES + wave; row < N; row += gridDim.x * BWD_WAVES) {
        const float4* xr = reinterpret_cast<const float4*>(x + (long)row * C);
        const float4* dr = reinterpret_cast<const float4*>(dy + (long)row * C);
        float4* o = reinterpret_cast<float4*>(dx + (long)row * C);
        const float m = mean[row], r = rstd[row];
        float4 xh[VPL], g[VPL], ov[VPL];
        float sg = 0.f, sgx = 0.f;
        // the row's x, dy and (when accumulating) old dx are all requested before the
        // reductions, so a row costs one memory latency
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            ov[j] = (accumulate && i < C4) ? o[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), dv = xv;
            if (i < C4) {
                xv = xr[i];
                dv = dr[i];
            }
            xh[j] = make_float4((xv.x - m) * r, (xv.y - m) * r, (xv.z - m) * r, (xv.w - m) * r);
            if (i >= C4) xh[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            g[j] = make_float4(wv[j].x * dv.x, wv[j].y * dv.y, wv[j].z * dv.z, wv[j].w * dv.w);
            sg += (g[j].x + g[j].y) + (g[j].z + g[j].w);
            sgx += (g[j].x * xh[j].x + g[j].y * xh[j].y) + (g[j].z * xh[j].z + g[j].w * xh[j].w);
            pdw[j].x += dv.x * xh[j].x;
            pdw[j].y += dv.y * xh[j].y;
            pdw[j].z += dv.z * xh[j].z;
            pdw[j].w += dv.w * xh[j].w;
            pdb[j].x += dv.x;
            pdb[j].y += dv.y;
            pdb[j].z += dv.z;
            pdb[j].w += dv.w;
        }
        const float mg = RMS ? 0.f : wave_sum(sg) / (float)C;
        const float mgx = wave_sum(sgx) / (float)C;
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            if (i < C4) {
                float4 d;
                d.x = r * (g[j].x - mg - xh[j].x * mgx);
                d.y = r * (g[j].y - mg - xh[j].y * mgx);
                d.z = r * (g[j].z - mg - xh[j].z * mgx);
                d.w = r * (g[j].w - mg - xh[j].w * mgx);
                if (accumulate) {
                    d.x += ov[j].x;
                    d.y += ov[j].y;
                    d.z += ov[j].z;
                    d.w += ov[j].w;
                }
                o[i] = d;
            }
        }
    }
    // Combine the waves' partials in wave order, then write the block's partial row
    // ([dw | db], or [dw] for RMSNorm).
    constexpr int PARTS = RMS ? 1 : 2;
    for (int part = 0; part < PARTS; part++) {
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int i = lane + 64 * j;
            if (i < C4) reinterpret_cast<float4*>(red + wave * C)[i] = part == 0 ? pdw[j] : pdb[j];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < C; c += blockDim.x) {
            float s = red[c];
#pragma unroll
            for (int q = 1; q < BWD_WAVES; q++) s += red[q * C + c];
            partial[(long)blockIdx.x * PARTS * C + part * C + c] = s;
        }
        __syncthreads();
    }
}

// out[w] (+)= sum_r part[r*W + w] over R rows (W % 4 == 0).  A block covers 16 columns as
// 4 float4 columns x 64 row groups (so the grid has W/16 blocks: 96 for LayerNorm's
// [dgamma | dbeta] rows at C = 768); group j adds rows j, j+64, ... in order.  The 64
// group sums of a column are then added as a fixed tree: within a wave (16 groups: lane
// bits 2..5) by row rotations of 4 and 8 lanes and the two permlane swaps, then the four
// waves' sums in wave order through LDS.  Columns w < W1 go to out_lo[w], the rest to
// out_hi[w - W1].
constexpr int RR_GROUPS = 64;
GPT2_DEV float rr_wave_sum(float x) {
    x += dpp_f<DPP_ROR4>(x);  // lanes i, i+4 of each 16-lane row (same column, bits 0..1)
    x += dpp_f<DPP_ROR8>(x);  // ... and i+8, i+12
    return rows4_sum(x);      // ... and the same lane of the other three rows
}
__global__ __launch_bounds__(256) void reduce_rows_kernel(float* out_lo, float* out_hi, int W1,
                                                          const float* __restrict__ part, int R, int W,
                                                          int accumulate) {
    __shared__ float4 s[4][4];
    const int c4 = threadIdx.x & 3, grp = threadIdx.x >> 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int w = blockIdx.x * 16 + c4 * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (w < W) {
#pragma unroll 8
        for (int r = grp; r < R; r += RR_GROUPS) {
            const float4 v = *reinterpret_cast<const float4*>(part + (long)r * W + w);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    acc.x = rr_wave_sum(acc.x);
    acc.y = rr_wave_sum(acc.y);
    acc.z = rr_wave_sum(acc.z);
    acc.w = rr_wave_sum(acc.w);
    if (lane < 4) s[wave][c4] = acc;
    __syncthreads();
    if (threadIdx.x < 4 && w < W) {
        float4 tot = s[0][c4];
#pragma unroll
        for (int j = 1; j < 4; j++) {
            const float4 v = s[j][c4];
            tot.x += v.x;
            tot.y += v.y;
            tot.z += v.z;
            tot.w += v.w;
        }
        const float t4[4] = {tot.x, tot.y, tot.z, tot.w};
        for (int e = 0; e < 4; e++) {
            const int we = w + e;
            float* dst = we < W1 ? out_lo + we : out_hi + (we - W1);
            *dst = accumulate ? *dst + t4[e] : t4[e];
        }
    }
}

int ln_blocks(int N) { return std::min((N + BWD_WAVES - 1) / BWD_WAVES, LN_MAX_BLOCKS); }

}  // namespace

namespace {

template <bool RMS>
hipError_t norm_forward(float* y, float* mean, float* rstd, const float* x, const float* w, const float* b, int N,
                        int C, float eps, hipStream_t st, uint16_t* yb) {
    if (C % 4 || C > 4096 || N < 0 || ((uintptr_t)yb & 7)) return hipErrorInvalidValue;
    if (N == 0) return hipSuccess;
    const int vpl = (C / 4 + 63) / 64;
    // several rows per wave only where the rows are short enough to keep in registers
    const int rpw = vpl <= 4 ? LN_FWD_ROWS : 1;
    dim3 grid((N + ROWS_PER_BLOCK * rpw - 1) / (ROWS_PER_BLOCK * rpw)), block(256);
    ProfScope ps(st, RMS ? "rms_fwd_kernel" : "ln_fwd_kernel", 0.0,
                 4.0 * ((double)N * C * (yb ? 2.5 : 2.0) + 2.0 * N + (RMS ? 1.0 : 2.0) * C));
#define LN_FWD(V, R) hipLaunchKernelGGL((ln_fwd_kernel<V, RMS, R>), grid, block, 0, st, y, yb, mean, rstd, x, w, b, N, C, eps)
    switch (vpl) {
        case 1: LN_FWD(1, LN_FWD_ROWS); break;
        case 2: LN_FWD(2, LN_FWD_ROWS); break;
        case 3: LN_FWD(3, LN_FWD_ROWS); break;
        case 4: LN_FWD(4, LN_FWD_ROWS); break;
        case 5: case 6: case 7: case 8: LN_FWD(8, 1); break;
        default: LN_FWD(16, 1); break;
    }
#undef LN_FWD
    return hipGetLastError();
}

template <bool RMS>
hipError_t norm_backward(float* dx, float* dw, float* db, const float* dy, const float* x, const float* w,
                         const float* mean, const float* rstd, int N, int C, bool accumulate_dx,
                         bool accumulate_dwdb, float* partial, hipStream_t st, hipStream_t st_red = nullptr,
                         hipEvent_t ev = nullptr) {
    if (C % 4 || C > 4096 || N < 0) return hipErrorInvalidValue;
    if (N == 0) {
        if (!accumulate_dwdb) {
            hipError_t e = fill_zero(dw, C, st);
            if (e != hipSuccess || RMS) return e;
            return fill_zero(db, C, st);
        }
        return hipSuccess;
    }
    constexpr int PARTS = RMS ? 1 : 2;
    const int vpl = (C / 4 + 63) / 64;
    const int G = ln_blocks(N);
    const size_t lds = (size_t)BWD_WAVES * C * sizeof(float);
    {
        ProfScope ps(st, RMS ? "rms_bwd_kernel" : "ln_bwd_kernel", 0.0,
                     4.0 * ((double)N * C * (accumulate_dx ? 4 : 3) + 2.0 * N + C + (double)PARTS * G * C));
#define LN_BWD(V) hipLaunchKernelGGL((ln_bwd_kernel<V, RMS>), dim3(G), dim3(64 * BWD_WAVES), lds, st, dx, partial, dy, x, w, mean, rstd, N, C, (int)accumulate_dx)
        switch (vpl) {
            case 1: LN_BWD(1); break;
            case 2: LN_BWD(2); break;
            case 3: LN_BWD(3); break;
            case 4: LN_BWD(4); break;
            case 5: case 6: case 7: case 8: LN_BWD(8); break;
            default: LN_BWD(16); break;
        }
#undef LN_BWD
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipStream_t sr = st;
    if (st_red && ev && st_red != st) {
        if ((e = hipEventRecord(ev, st)) != hipSuccess || (e = hipStreamWaitEvent(st_red, ev, 0)) != hipSuccess)
            return e;
        sr = st_red;
    }
    ProfScope ps2(sr, "reduce_rows_kernel", 0.0,
                  4.0 * ((double)G * PARTS * C + (double)PARTS * C * (accumulate_dwdb ? 2 : 1)));
    hipLaunchKernelGGL(reduce_rows_kernel, dim3((PARTS * C + 15) / 16), dim3(256), 0, sr, dw, db, C,
                       (const float*)partial, G, PARTS * C, (int)accumulate_dwdb);
    return hipGetLastError();
}

}  // namespace

hipError_t layernorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w,
                             const float* b, int N, int C, float eps, hipStream_t st, uint16_t* yb) {
    return norm_forward<false>(y, mean, rstd, x, w, b, N, C, eps, st, yb);
}

hipError_t rmsnorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w, int N, int C,
                           float eps, hipStream_t st, uint16_t* yb) {
    return norm_forward<true>(y, mean, rstd, x, w, nullptr, N, C, eps, st, yb);
}

size_t layernorm_partial_floats(int N, int C) { return (size_t)ln_blocks(N) * 2 * C; }

hipError_t layernorm_backward(float* dx, float* dw, float* db, const float* dy, const float* x,
                              const float* w, const float* mean, const float* rstd, int N, int C,
                              bool accumulate_dx, bool accumulate_dwdb, float* partial,
                              hipStream_t st, hipStream_t st_red, hipEvent_t ev) {
    return norm_backward<false>(dx, dw, db, dy, x, w, mean, rstd, N, C, accumulate_dx, accumulate_dwdb, partial,
                                st, st_red, ev);
}

hipError_t rmsnorm_backward(float* dx, float* dw, const float* dy, const float* x, const float* w,
                            const float* mean, const float* rstd, int N, int C, bool accumulate_dx,
                            bool accumulate_dw, float* partial, hipStream_t st, hipStream_t st_red, hipEvent_t ev) {
    return norm_backward<true>(dx, dw, nullptr, dy, x, w, mean, rstd, N, C, accumulate_dx, accumulate_dw, partial,
                               st, st_red, ev);
}

}  // namespace gpt2k

// ---------------------------------------------------------------------------------------
// gpt2_layernorm_backward_noalloc: the standalone LayerNorm backward for callers that
// cannot allocate (code under HIP graph capture, tight serving loops).  Its partial rows
// live in a fixed device array of this library instead of a caller workspace.  In host
// code `scratch` names a host-side stand-in, never the device memory: the device address
// is looked up once per device with hipGetSymbolAddress and only that address is used.
// ---------------------------------------------------------------------------------------
namespace {

constexpr size_t NOALLOC_SCRATCH_FLOATS = (size_t)4 << 20;  // 16 MiB per device
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

std::mutex g_scratch_mu;
float* g_scratch_ptr[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the current device (looked up on its first use there),
// or nullptr on failure.
float* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = static_cast<float*>(ptr);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t gpt2_layernorm_backward_noalloc_max_floats(void) { return NOALLOC_SCRATCH_FLOATS; }

int gpt2_layernorm_backward_noalloc(float* dx, float* dw, float* db, const float* dy, const float* x,
                                    const float* w, const float* mean, const float* rstd, int N, int C,
                                    void* stream) {
    auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    if (!dw || !db || N < 0 || C <= 0 || C % 4 || C > 4096) return GPT2_EINVAL;
    if (N > 0 && (!dx || !dy || !x || !w || !mean || !rstd)) return GPT2_EINVAL;
    if (N > 0 && (!al(dx) || !al(dy) || !al(x) || !al(w))) return GPT2_EINVAL;
    if (gpt2k::layernorm_partial_floats(N, C) > NOALLOC_SCRATCH_FLOATS) return GPT2_ESCRATCH;
    float* ptr = device_scratch();
    if (!ptr) return GPT2_EDEVICE;
    return gpt2k::layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, N, C, false, false, ptr,
                                     (hipStream_t)stream) == hipSuccess
               ? GPT2_OK
               : GPT2_EDEVICE;
}

}  // extern "C"
