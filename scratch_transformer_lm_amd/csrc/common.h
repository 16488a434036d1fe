// Internal helpers shared by the gfx950 kernels of the GPT-2 step (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GPT2_DEV __device__ __forceinline__

namespace gpt2k {

constexpr int WAVE = 64;

// Cross-lane reductions on the VALU (DPP and the gfx950 permlane swaps, no LDS round trip),
// each in the tree of the shuffle-xor steps it stands for, so sums are bitwise the same:
//  rows4_*: over lanes i, i^16, i^32, i^48.  v_permlane16_swap exchanges rows 1, 3 of its
//    first operand with rows 0, 2 of its second, v_permlane32_swap the upper half of the
//    first with the lower half of the second; with both operands the value, each lane holds
//    its own and its partner's value: (r0 + r1) + (r2 + r3) in every lane.
//  row16_*: over the 16 lanes of each row, xor 1, 2, 4, 8.  After the two quad steps the
//    values are equal within each quad, after the half-row mirror within each 8 lanes, so
//    the mirrors pair the same values as xor 4 and xor 8.
//  wave_*: xor 32 then 16 as permlane swaps (v_permlane32_swap pairs lanes i and i^32 the
//    same way), then 8, 4, 2, 1 as row rotations: after the xor-8 step the values are equal
//    within each residue class mod 8 of the lane, and rotating by 4, 2, 1 reaches the class
//    that xor 4, 2, 1 would.
template <int CTRL>
GPT2_DEV float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_ROR1 = 0x121, DPP_ROR2 = 0x122, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;
GPT2_DEV float xpair16_a(float x, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    b = __uint_as_float(r[1]);
    return __uint_as_float(r[0]);
}
GPT2_DEV float xpair32_a(float x, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    b = __uint_as_float(r[1]);
    return __uint_as_float(r[0]);
}
GPT2_DEV float rows4_sum(float x) {
    float b;
    x = xpair16_a(x, b) + b;
    x = xpair32_a(x, b) + b;
    return x;
}
GPT2_DEV float rows4_max(float x) {
    float b;
    x = fmaxf(xpair16_a(x, b), b);
    x = fmaxf(xpair32_a(x, b), b);
    return x;
}
GPT2_DEV float row16_sum(float x) {
    x += dpp_f<DPP_XOR1>(x);
    x += dpp_f<DPP_XOR2>(x);
    x += dpp_f<DPP_HALF_MIRROR>(x);
    return x + dpp_f<DPP_MIRROR>(x);
}
GPT2_DEV float row16_max(float x) {
    x = fmaxf(x, dpp_f<DPP_XOR1>(x));
    x = fmaxf(x, dpp_f<DPP_XOR2>(x));
    x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
    return fmaxf(x, dpp_f<DPP_MIRROR>(x));
}

GPT2_DEV float wave_sum(float v) {
    float b;
    v = xpair32_a(v, b) + b;
    v = xpair16_a(v, b) + b;
    v += dpp_f<DPP_ROR8>(v);
    v += dpp_f<DPP_ROR4>(v);
    v += dpp_f<DPP_ROR2>(v);
    return v + dpp_f<DPP_ROR1>(v);
}

GPT2_DEV float wave_max(float v) {
    float b;
    v = fmaxf(xpair32_a(v, b), b);
    v = fmaxf(xpair16_a(v, b), b);
    v = fmaxf(v, dpp_f<DPP_ROR8>(v));
    v = fmaxf(v, dpp_f<DPP_ROR4>(v));
    v = fmaxf(v, dpp_f<DPP_ROR2>(v));
    return fmaxf(v, dpp_f<DPP_ROR1>(v));
}

GPT2_DEV double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Tanh-form GELU and its derivative (same constants as the model definition),
//   GELU(u) = 0.5 u (1 + tanh z),  z = K0 (u + K1 u^3),
// evaluated through the logistic form 0.5 (1 + tanh z) = s = 1 / (1 + e^{-2z}):
// GELU(u) = u s and GELU'(u) = s + u s (1 - s) 2 dz/du, with the factor -2 log2 e folded
// into the constants of one base-2 exponential, on the hardware transcendental unit
// (v_exp_f32, v_rcp_f32: a few ulp).  e^{-2z} overflowing to +inf gives s = 0 exactly,
// underflowing to 0 gives s = 1.
constexpr float GELU_K0 = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_K1 = 0.044715f;
constexpr float GELU_C0 = -2.0f * 1.4426950408889634f * GELU_K0;            // u^1 term of -2 z log2 e
constexpr float GELU_C1 = -2.0f * 1.4426950408889634f * GELU_K0 * GELU_K1;  // u^3 term
GPT2_DEV float gelu_s(float u, float w) {  // w = u^2
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * fmaf(GELU_C1, w, GELU_C0)));
}
GPT2_DEV float gelu_f(float u) { return u * gelu_s(u, u * u); }

GPT2_DEV float gelu_grad_f(float u) {
    const float w = u * u;
    const float s = gelu_s(u, w);
    const float dz2 = fmaf(6.0f * GELU_K0 * GELU_K1, w, 2.0f * GELU_K0);  // 2 dz/du
    return fmaf(u * s, (1.0f - s) * dz2, s);
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
