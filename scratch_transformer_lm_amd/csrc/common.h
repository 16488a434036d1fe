// Internal helpers shared by the gfx950 kernels of the GPT-2 step (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GPT2_DEV __device__ __forceinline__

namespace gpt2k {

constexpr int WAVE = 64;

GPT2_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

GPT2_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

GPT2_DEV double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Tanh-form GELU and its derivative (same constants as the model definition).
constexpr float GELU_K0 = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_K1 = 0.044715f;

// tanh z = 1 - 2 / (e^{2z} + 1), with e^x and 1/x on the hardware transcendental unit
// (v_exp_f32, v_rcp_f32: a few ulp; e^{2z} overflowing to +inf still gives exactly 1).
GPT2_DEV float tanh_fast(float z) { return 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(2.0f * z) + 1.0f); }

GPT2_DEV float gelu_f(float u) {
    float z = GELU_K0 * (u + GELU_K1 * u * u * u);
    return 0.5f * u * (1.0f + tanh_fast(z));
}

GPT2_DEV float gelu_grad_f(float u) {
    float z = GELU_K0 * (u + GELU_K1 * u * u * u);
    float th = tanh_fast(z);
    float dz = GELU_K0 * (1.0f + 3.0f * GELU_K1 * u * u);
    return 0.5f * (1.0f + th) + 0.5f * u * (1.0f - th * th) * dz;
}

// fp32 pair -> packed bfloat16 (low half = lo), round to nearest, ties to even: one
// v_cvt_pk_bf16_f32.
GPT2_DEV uint32_t bf16_pack2(float lo, float hi) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// bf16 copy of two rows of a 16x16 matrix-core accumulator (lane: column c = lane % 16,
// rows 4 (lane / 16) + v), written as 4-byte pairs: each lane swaps one value with its
// neighbour (DPP quad_perm 1,0,3,2), then even lanes write row v, columns (c, c+1), and
// odd lanes row v+1, columns (c-1, c).  p0 and p1 point at this lane's element of rows v
// and v+1; ok0, ok1 say whether those rows exist.  Every lane of the wave must call it;
// the fragment's first column must be even and rows 4-byte aligned.
GPT2_DEV void bf16_store_rows2(uint16_t* p0, uint16_t* p1, float x0, float x1, bool ok0, bool ok1) {
    const bool odd = threadIdx.x & 1;
    const float send = odd ? x0 : x1;
    const float recv = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
    if (!odd) {
        if (ok0) *reinterpret_cast<uint32_t*>(p0) = bf16_pack2(x0, recv);
    } else if (ok1) {
        *reinterpret_cast<uint32_t*>(p1 - 1) = bf16_pack2(recv, x1);
    }
}

// Error flag bits written by kernels into the scratch header.
constexpr int ERR_BAD_INPUT_TOKEN = 1;
constexpr int ERR_BAD_TARGET_TOKEN = 2;

// Layout of the small header at the start of grad_scratch (in 4-byte words).
constexpr int HDR_LOSS = 0;     // float: mean loss of the last forward
constexpr int HDR_FLAGS = 1;    // int: error bits
constexpr int HDR_WORDS = 64;   // header size (keeps what follows 256-byte aligned)

}  // namespace gpt2k
