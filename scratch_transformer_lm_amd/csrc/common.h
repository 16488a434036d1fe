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

// Error flag bits written by kernels into the scratch header.
constexpr int ERR_BAD_INPUT_TOKEN = 1;
constexpr int ERR_BAD_TARGET_TOKEN = 2;

// Layout of the small header at the start of grad_scratch (in 4-byte words).
constexpr int HDR_LOSS = 0;     // float: mean loss of the last forward
constexpr int HDR_FLAGS = 1;    // int: error bits
constexpr int HDR_WORDS = 64;   // header size (keeps what follows 256-byte aligned)

}  // namespace gpt2k
