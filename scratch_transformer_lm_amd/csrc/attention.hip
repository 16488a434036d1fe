// Causal multi-head self-attention, forward and backward, on gfx950 matrix cores.
//
// The pages name the layer (attention_forward / attention_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1; multi-head in section
// 傻瓜式复现GPT-2).  Per (batch b, head h, query t):
//   s_u = (q_t . k_u) / sqrt(hs) for u <= t,  p = softmax(s),  o_t = sum_u p_u v_u.
// The forward keeps o and lse_t = max + log(sum exp) per row (O(T) instead of the
// plain (B,NH,T,T) score tensors); the backward recomputes p_u = exp(s_u - lse_t):
//   D_t = dO_t . o_t;  dp_u = dO_t . v_u;  ds_u = p_u (dp_u - D_t);
//   dq_t = scale sum_u ds_u k_u;  dk_u = scale sum_t ds_tu q_t;  dv_u = sum_t p_tu dO_t.
//
// Tiling for CDNA4: a block is 4 wave64s over a 64-row tile, each wave 16 rows, and
// every product is a v_mfma_f32_16x16x4f32 chain (A[i][k] from lane i + 16k, B[k][j]
// from lane j + 16k, C[i][j] in lane j + 16(i/4), register i%4).  The score tile is
// computed transposed where that puts the probabilities directly into the A-operand
// layout of the next product, so P never goes through LDS.  Inside each group of 16
// head dimensions a lane feeds 4 consecutive dimensions to 4 consecutive MFMAs (a
// reordering of the dot product), which makes every operand read one 16-byte LDS
// read.  K/V (or Q/dO) tiles are double-buffered in LDS with register prefetch.
// dq and dk/dv come from two kernels (query-tile and key-tile ownership) so every
// output element has one writer: no atomics, bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 64;

GPT2_DEV f32x4 mfma4(float a, float b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

GPT2_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

GPT2_DEV float comp(const float4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// Softmax arithmetic runs in base 2 on the hardware transcendental unit (v_exp_f32,
// v_log_f32): exp(x) = 2^(x log2 e), with log2 e folded into the score scale and the
// stored log-sum-exp converted back to natural log.
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
GPT2_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
GPT2_DEV float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Loads a 64-row x HS tile of rows [r0, r0+64) (row stride ld floats, rows >= T are
// zero) into registers: thread t covers row t/(HS/4) + (256/(HS/4))*j, float4 column t%(HS/4).
template <int HS>
GPT2_DEV void tile_load(float4 (&reg)[HS / 16], const float* src, long ld, int r0, int T) {
    constexpr int C4 = HS / 4, RPP = 256 / C4;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < HS / 16; j++) {
        const int r = r0 + t / C4 + RPP * j;
        reg[j] = r < T ? *reinterpret_cast<const float4*>(src + (long)r * ld + (t % C4) * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int HS>
GPT2_DEV void tile_store(float* S, const float4 (&reg)[HS / 16]) {
    constexpr int C4 = HS / 4, RPP = 256 / C4, LD = HS + 4;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < HS / 16; j++)
        *reinterpret_cast<float4*>(S + (t / C4 + RPP * j) * LD + (t % C4) * 4) = reg[j];
}

// ---------------------------------------------------------------------------- forward
template <int HS>
__global__ __launch_bounds__(256) void attn_fwd_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                       const float* __restrict__ qkv, int B, int T, int C, int NH,
                                                       float scale) {
    constexpr int DG = HS / 16, LD = HS + 4;
    __shared__ __attribute__((aligned(16))) float Ks[2][TILE * LD];
    __shared__ __attribute__((aligned(16))) float Vs[2][TILE * LD];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int qt = nqt - 1 - (int)(blockIdx.x / (B * NH));  // longest rows first
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const long ld = 3L * C;
    const float* base = qkv + (long)b * T * ld;
    const int q0 = qt * TILE + wave * 16;
    const int tq = q0 + i16;

    float4 qreg[DG];
#pragma unroll
    for (int g = 0; g < DG; g++)
        qreg[g] = tq < T ? *reinterpret_cast<const float4*>(base + (long)tq * ld + h * HS + 16 * g + 4 * g4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    f32x4 o[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) o[d] = zero4();
    float m = -INFINITY, l = 0.f;  // running max (base 2) and sum of this lane's query row
    const float scale2 = scale * LOG2E;

    float4 kreg[DG], vreg[DG];
    const int nkt = qt + 1;
    tile_load<HS>(kreg, base + C + h * HS, ld, 0, T);
    tile_load<HS>(vreg, base + 2 * C + h * HS, ld, 0, T);
    tile_store<HS>(Ks[0], kreg);
    tile_store<HS>(Vs[0], vreg);
    __syncthreads();
    // one key tile; only the diagonal tile (kt == qt) has keys after the query
    auto step = [&](int kt, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const int cur = kt & 1;
        if (kt + 1 < nkt) {
            tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
            tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
        }
        const float* K = Ks[cur];
        const float* V = Vs[cur];
        // S^T[key][query] = K Q^T for 4 blocks of 16 keys.
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            s[kb] = zero4();
#pragma unroll
            for (int g = 0; g < DG; g++) {
                const float4 kf = *reinterpret_cast<const float4*>(K + (kb * 16 + i16) * LD + 16 * g + 4 * g4);
#pragma unroll
                for (int st = 0; st < 4; st++) s[kb] = mfma4(comp(kf, st), comp(qreg[g], st), s[kb]);
            }
        }
        // lane holds raw scores of query tq against keys kt*64 + kb*16 + 4*g4 + v
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                if (DIAG && kt * TILE + kb * 16 + 4 * g4 + v > tq) s[kb][v] = -INFINITY;
                mx = fmaxf(mx, s[kb][v]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference max m (base 2) of each row moves only when the row's new max
        // exceeds it by more than 8, i.e. probabilities relative to m stay below 2^8; the
        // result is the same softmax, and O is rescaled only on the (rare, wave-wide)
        // occasions when some row's reference moves.
        const float mnew = fmaxf(m, mx * scale2);
        if (__any(mnew > m + 8.0f)) {
            const float alpha = exp2_hw(m - mnew);
            l *= alpha;
            m = mnew;
            // O rows are queries 4*g4 + v of the wave: rescale with their alpha.
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float a = __shfl(alpha, 4 * g4 + v, 64);
#pragma unroll
                for (int d = 0; d < DG; d++) o[d][v] *= a;
            }
        }
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float p = exp2_hw(fmaf(s[kb][v], scale2, -m));
                s[kb][v] = p;
                rs += p;
            }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        l += rs;
        // O += P V
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float* vrow = V + (kb * 16 + 4 * g4 + v) * LD + i16;
#pragma unroll
                for (int d = 0; d < DG; d++) o[d] = mfma4(s[kb][v], vrow[16 * d], o[d]);
            }
        if (kt + 1 < nkt) {
            tile_store<HS>(Ks[cur ^ 1], kreg);
            tile_store<HS>(Vs[cur ^ 1], vreg);
        }
        __syncthreads();
    };
    for (int kt = 0; kt < qt; kt++) step(kt, std::false_type{});
    step(qt, std::true_type{});
    const float linv = 1.0f / l;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int q = q0 + 4 * g4 + v;
        const float a = __shfl(linv, 4 * g4 + v, 64);
        if (q < T) {
            float* orow = out + ((long)b * T + q) * C + h * HS + i16;
#pragma unroll
            for (int d = 0; d < DG; d++) orow[16 * d] = o[d][v] * a;
        }
    }
    if (g4 == 0 && tq < T) lse[((long)b * NH + h) * T + tq] = (m + log2_hw(l)) * LN2;
}

// ---------------------------------------------------------------------------- dq (+ D)
template <int HS>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(float* __restrict__ dqkv, float* __restrict__ delta,
                                                          const float* __restrict__ dout, const float* __restrict__ qkv,
                                                          const float* __restrict__ out, const float* __restrict__ lse,
                                                          int B, int T, int C, int NH, float scale) {
    constexpr int DG = HS / 16, LD = HS + 4;
    __shared__ __attribute__((aligned(16))) float Ks[2][TILE * LD];
    __shared__ __attribute__((aligned(16))) float Vs[2][TILE * LD];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int qt = nqt - 1 - (int)(blockIdx.x / (B * NH));
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const long ld = 3L * C;
    const float* base = qkv + (long)b * T * ld;
    const int q0 = qt * TILE + wave * 16;
    const int tq = q0 + i16;
    const bool valid = tq < T;

    float4 qreg[DG], doreg[DG];
    float dd = 0.f;
#pragma unroll
    for (int g = 0; g < DG; g++) {
        const int col = h * HS + 16 * g + 4 * g4;
        if (valid) {
            qreg[g] = *reinterpret_cast<const float4*>(base + (long)tq * ld + col);
            doreg[g] = *reinterpret_cast<const float4*>(dout + ((long)b * T + tq) * C + col);
            const float4 ov = *reinterpret_cast<const float4*>(out + ((long)b * T + tq) * C + col);
            dd += doreg[g].x * ov.x + doreg[g].y * ov.y + doreg[g].z * ov.z + doreg[g].w * ov.w;
        } else {
            qreg[g] = doreg[g] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    dd += __shfl_xor(dd, 16, 64);
    dd += __shfl_xor(dd, 32, 64);
    const float D = dd;
    const float L = valid ? lse[((long)b * NH + h) * T + tq] : INFINITY;
    const float L2 = L * LOG2E, scale2 = scale * LOG2E;
    if (g4 == 0 && valid) delta[((long)b * NH + h) * T + tq] = D;

    f32x4 dq[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) dq[d] = zero4();
    float4 kreg[DG], vreg[DG];
    const int nkt = qt + 1;
    tile_load<HS>(kreg, base + C + h * HS, ld, 0, T);
    tile_load<HS>(vreg, base + 2 * C + h * HS, ld, 0, T);
    tile_store<HS>(Ks[0], kreg);
    tile_store<HS>(Vs[0], vreg);
    __syncthreads();
    // one key tile; only the diagonal tile (kt == qt) has keys after the query
    auto step = [&](int kt, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const int cur = kt & 1;
        if (kt + 1 < nkt) {
            tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
            tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
        }
        const float* K = Ks[cur];
        const float* V = Vs[cur];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            f32x4 s = zero4(), dp = zero4();
#pragma unroll
            for (int g = 0; g < DG; g++) {
                const float4 kf = *reinterpret_cast<const float4*>(K + (kb * 16 + i16) * LD + 16 * g + 4 * g4);
                const float4 vf = *reinterpret_cast<const float4*>(V + (kb * 16 + i16) * LD + 16 * g + 4 * g4);
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    s = mfma4(comp(kf, st), comp(qreg[g], st), s);
                    dp = mfma4(comp(vf, st), comp(doreg[g], st), dp);
                }
            }
            // lane: key kt*64 + kb*16 + 4*g4 + v, query tq
            float ds[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int key = kt * TILE + kb * 16 + 4 * g4 + v;
                const float p = (!DIAG || key <= tq) ? exp2_hw(fmaf(s[v], scale2, -L2)) : 0.f;
                ds[v] = p * (dp[v] - D);
            }
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float* krow = K + (kb * 16 + 4 * g4 + v) * LD + i16;
#pragma unroll
                for (int d = 0; d < DG; d++) dq[d] = mfma4(ds[v], krow[16 * d], dq[d]);
            }
        }
        if (kt + 1 < nkt) {
            tile_store<HS>(Ks[cur ^ 1], kreg);
            tile_store<HS>(Vs[cur ^ 1], vreg);
        }
        __syncthreads();
    };
    for (int kt = 0; kt < qt; kt++) step(kt, std::false_type{});
    step(qt, std::true_type{});
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int q = q0 + 4 * g4 + v;
        if (q < T) {
            float* drow = dqkv + ((long)b * T + q) * ld + h * HS + i16;
#pragma unroll
            for (int d = 0; d < DG; d++) drow[16 * d] = dq[d][v] * scale;
        }
    }
}

// ---------------------------------------------------------------------------- dk, dv
template <int HS>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(float* __restrict__ dqkv, const float* __restrict__ delta,
                                                            const float* __restrict__ dout, const float* __restrict__ qkv,
                                                            const float* __restrict__ lse, int B, int T, int C, int NH,
                                                            float scale) {
    constexpr int DG = HS / 16, LD = HS + 4;
    __shared__ __attribute__((aligned(16))) float Qs[2][TILE * LD];
    __shared__ __attribute__((aligned(16))) float Os[2][TILE * LD];
    __shared__ float Ls[2][TILE], Ds[2][TILE];  // base-2 log-sum-exp and D of the query tile
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int kt = (int)(blockIdx.x / (B * NH));  // key tile 0 sees the most queries: first
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const long ld = 3L * C;
    const float* base = qkv + (long)b * T * ld;
    const float* dbase = dout + (long)b * T * C;
    const float* lrow = lse + ((long)b * NH + h) * T;
    const float* drow_ = delta + ((long)b * NH + h) * T;
    const int u0 = kt * TILE + wave * 16;
    const int tu = u0 + i16;

    float4 kreg[DG], vreg[DG];
#pragma unroll
    for (int g = 0; g < DG; g++) {
        const int col = h * HS + 16 * g + 4 * g4;
        if (tu < T) {
            kreg[g] = *reinterpret_cast<const float4*>(base + (long)tu * ld + C + col);
            vreg[g] = *reinterpret_cast<const float4*>(base + (long)tu * ld + 2 * C + col);
        } else {
            kreg[g] = vreg[g] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    f32x4 dk[DG], dv[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) dk[d] = dv[d] = zero4();
    const float scale2 = scale * LOG2E;

    float4 qreg[DG], oreg[DG];
    float lv = 0.f, dv1 = 0.f;
    auto load_side = [&](int qt) {
        const int r = qt * TILE + (threadIdx.x & 63);
        if (threadIdx.x < 64) {
            lv = r < T ? lrow[r] * LOG2E : INFINITY;
            dv1 = r < T ? drow_[r] : 0.f;
        }
    };
    auto store_side = [&](int stage) {
        if (threadIdx.x < 64) {
            Ls[stage][threadIdx.x] = lv;
            Ds[stage][threadIdx.x] = dv1;
        }
    };
    tile_load<HS>(qreg, base + h * HS, ld, kt * TILE, T);
    tile_load<HS>(oreg, dbase + h * HS, C, kt * TILE, T);
    load_side(kt);
    tile_store<HS>(Qs[0], qreg);
    tile_store<HS>(Os[0], oreg);
    store_side(0);
    __syncthreads();
    // one query tile; only the diagonal tile (qt == kt) has queries before the key
    auto step = [&](int qt, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const int cur = (qt - kt) & 1;
        if (qt + 1 < nqt) {
            tile_load<HS>(qreg, base + h * HS, ld, (qt + 1) * TILE, T);
            tile_load<HS>(oreg, dbase + h * HS, C, (qt + 1) * TILE, T);
            load_side(qt + 1);
        }
        const float* Q = Qs[cur];
        const float* O = Os[cur];
#pragma unroll
        for (int qb = 0; qb < 4; qb++) {
            f32x4 s = zero4(), dp = zero4();
#pragma unroll
            for (int g = 0; g < DG; g++) {
                const float4 qf = *reinterpret_cast<const float4*>(Q + (qb * 16 + i16) * LD + 16 * g + 4 * g4);
                const float4 of = *reinterpret_cast<const float4*>(O + (qb * 16 + i16) * LD + 16 * g + 4 * g4);
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    s = mfma4(comp(qf, st), comp(kreg[g], st), s);
                    dp = mfma4(comp(of, st), comp(vreg[g], st), dp);
                }
            }
            // lane: query qt*64 + qb*16 + 4*g4 + v, key tu
            float p[4], ds[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int qi = qb * 16 + 4 * g4 + v;
                const int q = qt * TILE + qi;
                const float pv = (!DIAG || tu <= q) ? exp2_hw(fmaf(s[v], scale2, -Ls[cur][qi])) : 0.f;
                p[v] = pv;
                ds[v] = pv * (dp[v] - Ds[cur][qi]);
            }
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int qi = qb * 16 + 4 * g4 + v;
                const float* orow = O + qi * LD + i16;
                const float* qrow = Q + qi * LD + i16;
#pragma unroll
                for (int d = 0; d < DG; d++) {
                    dv[d] = mfma4(p[v], orow[16 * d], dv[d]);
                    dk[d] = mfma4(ds[v], qrow[16 * d], dk[d]);
                }
            }
        }
        if (qt + 1 < nqt) {
            tile_store<HS>(Qs[cur ^ 1], qreg);
            tile_store<HS>(Os[cur ^ 1], oreg);
            store_side(cur ^ 1);
        }
        __syncthreads();
    };
    step(kt, std::true_type{});
    for (int qt = kt + 1; qt < nqt; qt++) step(qt, std::false_type{});
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int u = u0 + 4 * g4 + v;
        if (u < T) {
            float* row = dqkv + ((long)b * T + u) * ld + h * HS + i16;
#pragma unroll
            for (int d = 0; d < DG; d++) {
                row[C + 16 * d] = dk[d][v] * scale;
                row[2 * C + 16 * d] = dv[d][v];
            }
        }
    }
}

template <int HS>
const char* fwd_name() {
    return HS == 16 ? "attn_fwd_kernel<16>" : HS == 32 ? "attn_fwd_kernel<32>" : "attn_fwd_kernel<64>";
}
template <int HS>
const char* dq_name() {
    return HS == 16 ? "attn_bwd_dq_kernel<16>" : HS == 32 ? "attn_bwd_dq_kernel<32>" : "attn_bwd_dq_kernel<64>";
}
template <int HS>
const char* dkdv_name() {
    return HS == 16 ? "attn_bwd_dkdv_kernel<16>" : HS == 32 ? "attn_bwd_dkdv_kernel<32>" : "attn_bwd_dkdv_kernel<64>";
}

template <int HS>
void launch_fwd(float* out, float* lse, const float* qkv, int B, int T, int C, int NH, hipStream_t st) {
    const int nqt = (T + TILE - 1) / TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    // causal half: T(T+1)/2 (query, key) pairs per (b, h), two products of HS MACs each
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    ProfScope ps(st, fwd_name<HS>(), pairs * HS * 2 * 2, 4.0 * B * T * (3.0 * C + C + NH));
    hipLaunchKernelGGL(attn_fwd_kernel<HS>, dim3(nqt * B * NH), dim3(256), 0, st, out, lse, qkv, B, T, C, NH, scale);
}

template <int HS>
void launch_bwd(float* dqkv, float* delta, const float* dout, const float* qkv, const float* out, const float* lse,
                int B, int T, int C, int NH, hipStream_t st) {
    const int nt = (T + TILE - 1) / TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    {
        // products formed: S (recomputed), dP, dQ
        ProfScope ps(st, dq_name<HS>(), pairs * HS * 2 * 3, 4.0 * B * T * (2.0 * C + 3.0 * C + 2 * NH));
        hipLaunchKernelGGL(attn_bwd_dq_kernel<HS>, dim3(nt * B * NH), dim3(256), 0, st, dqkv, delta, dout, qkv, out,
                           lse, B, T, C, NH, scale);
    }
    // products formed: S (recomputed), dP, dV, dK
    ProfScope ps(st, dkdv_name<HS>(), pairs * HS * 2 * 4, 4.0 * B * T * (3.0 * C + C + 2.0 * C + 2 * NH));
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<HS>, dim3(nt * B * NH), dim3(256), 0, st, dqkv, (const float*)delta, dout,
                       qkv, lse, B, T, C, NH, scale);
}

}  // namespace

hipError_t attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                             hipStream_t st) {
    if (C % NH || C % 4) return hipErrorInvalidValue;
    if ((long)B * T == 0) return hipSuccess;
    switch (C / NH) {
        case 16: launch_fwd<16>(out, lse, qkv, B, T, C, NH, st); break;
        case 32: launch_fwd<32>(out, lse, qkv, B, T, C, NH, st); break;
        case 64: launch_fwd<64>(out, lse, qkv, B, T, C, NH, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t attention_backward(float* dqkv, float* delta, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C, int NH,
                              hipStream_t st) {
    if (C % NH || C % 4) return hipErrorInvalidValue;
    if ((long)B * T == 0) return hipSuccess;
    switch (C / NH) {
        case 16: launch_bwd<16>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st); break;
        case 32: launch_bwd<32>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st); break;
        case 64: launch_bwd<64>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gpt2k
