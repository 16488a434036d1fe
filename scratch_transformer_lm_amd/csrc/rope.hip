// Rotary position embedding for the Llama-style layer variant, on gfx950.
//
// The pages name the Llama family as another target of llm.c (新智元 article, 纯CUDA也可训;
// lianzai README, 项目简介) but give no formula: this is the published RoPE (Su et al.,
// 2021).  In every head of q and k, the dimension pair (2i, 2i+1) at position t (0 at
// the start of every row) is rotated by the angle t * 10000^(-2i/hs); v is untouched.
// The backward applies the transpose, the rotation by -angle, to dq and dk.
//
// Both directions are elementwise and HBM-bound: one thread per pair reads a float2 of
// the (B, T, 3C) tensor and the pair's (cos, sin) from a table of maxT x hs/2 entries
// built once per model in float64 (so an angle like 1023 rad keeps its full precision
// before rounding to fp32), and writes the rotated float2 in place.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

__global__ void rope_table_kernel(float2* __restrict__ table, int maxT, int half, int hs) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)maxT * half) return;
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double ang = (double)t * exp(-(double)(2 * i) / (double)hs * log(10000.0));
    table[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// SIGN = +1: forward rotation; -1: its transpose (backward).
template <int SIGN>
__global__ __launch_bounds__(256) void rope_kernel(float* __restrict__ qkv, const float2* __restrict__ table, int T,
                                                   int C, int hs, long pairs) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= pairs) return;
    // idx = (row, c2) with c2 the pair index over the 2C columns of q and k
    const long row = idx / C;
    const int c2 = (int)(idx - row * C);
    const int t = (int)(row % T);
    const int col = 2 * c2;                 // column in [0, 2C): q then k
    const int i = (col % hs) >> 1;          // pair index inside the head
    const float2 cs = table[(long)t * (hs >> 1) + i];
    float2* p = reinterpret_cast<float2*>(qkv + row * 3L * C + col);
    const float2 v = *p;
    const float sn = SIGN * cs.y;
    *p = make_float2(v.x * cs.x - v.y * sn, v.x * sn + v.y * cs.x);
}

}  // namespace

size_t rope_table_floats(int maxT, int hs) { return (size_t)maxT * hs; }

hipError_t rope_table(float* table, int maxT, int hs, hipStream_t st) {
    if (hs % 2 || maxT <= 0) return hipErrorInvalidValue;
    const long n = (long)maxT * (hs / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float2*>(table), maxT, hs / 2, hs);
    return hipGetLastError();
}

template <int SIGN>
static hipError_t rope_apply(float* qkv, const float* table, int B, int T, int C, int NH, hipStream_t st,
                             const char* name) {
    if (C % NH || (C / NH) % 2 || B < 0 || T < 0) return hipErrorInvalidValue;
    const long pairs = (long)B * T * C;  // 2C columns of q and k per row, two per pair
    if (pairs == 0) return hipSuccess;
    ProfScope ps(st, name, 0.0, 4.0 * ((double)B * T * 2 * C * 2 + (double)T * (C / NH)));
    hipLaunchKernelGGL(rope_kernel<SIGN>, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, st, qkv,
                       reinterpret_cast<const float2*>(table), T, C, C / NH, pairs);
    return hipGetLastError();
}

hipError_t rope_forward(float* qkv, const float* table, int B, int T, int C, int NH, hipStream_t st) {
    return rope_apply<1>(qkv, table, B, T, C, NH, st, "rope_kernel<1>");
}

hipError_t rope_backward(float* dqkv, const float* table, int B, int T, int C, int NH, hipStream_t st) {
    return rope_apply<-1>(dqkv, table, B, T, C, NH, st, "rope_kernel<-1>");
}

}  // namespace gpt2k
