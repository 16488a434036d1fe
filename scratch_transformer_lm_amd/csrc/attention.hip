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
// layout of the next product, so P never goes through LDS.  The next K/V (or Q/dO) tile
// is prefetched into registers while the current one is used.  dQ keeps one LDS copy of
// each tile (two barriers per tile) so that three blocks fit a CU: with the query tiles'
// very unequal lengths (1 to T/64 key tiles), 768 block slots schedule the 1536 blocks of
// the 124M shape almost evenly where 512 slots leave a 9% tail.  The forward and dK/dV
// double-buffer their tiles (one barrier per tile) at two blocks per CU, measured faster
// there (the forward 1.60 -> 1.58 ms per step at the 124M shape; dQ double-buffered is
// slower, 2.24 -> 2.25 ms).
//
// LDS rows are stored head-dimension interleaved: dimension d = 16j + i (i < 16,
// j < HS/16) sits at position (HS/16) i + j.  A tile is read two ways, and both become
// one LDS read of HS/16 consecutive floats per lane (16 bytes at HS = 64):
//  - as the operand of a dot product over d (S = Q K^T, dP = dO V^T): MFMA (a, j) takes
//    from lane group g the dimension 16j + 4a + g, so a lane's HS/16 values for fixed a
//    are the run at i = 4a + g (the dot product is summed in another order);
//  - as the B operand of a product into d (O += P V, dQ += dS K, dK, dV): output block j
//    holds dimensions 16j + i for lane i, i.e. the run at i.
// Rows are padded to HS + 4 floats so that 16 lanes reading 16 rows, or 16 runs of one
// row, hit 16 different bank groups.
// dq and dk/dv come from separate kernels (query-tile and key-tile ownership) so every
// output element has one writer: no atomics, bitwise reproducible.  With a score-gradient
// buffer (the default of the step), D comes from its own small kernel, the dK/dV kernel
// (the only one that recomputes S and dP) also stores ds for every causal tile pair, and
// dQ is the plain product ds K: one product per pair instead of three (at the 124M shape
// 0.89 against 2.25 ms per step for dQ, +0.22 ms of stores in dK/dV: the step 54.3 ->
// 53.35 ms).  Without the buffer, dQ recomputes S and dP itself.
#include <string>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 64;
// Build options: blocks per CU of the forward and dQ kernels (their registers are capped
// to fit), and whether the next LDS fragments are read while the current ones multiply
// (two register buffers) or just before use (one).
#ifndef ATTN_FWD_OCC
#define ATTN_FWD_OCC 2
#endif
#ifndef ATTN_AHEAD
#define ATTN_AHEAD 1
#endif
// forward and dQ: the next K/V tile is loaded into registers while the current one is used
// (1), or after the current one is done, straight before it is stored to LDS (0)
#ifndef ATTN_PREFETCH
#define ATTN_PREFETCH 1
#endif
// forward: K/V tiles double-buffered in LDS (one barrier per tile; the LDS then holds two
// blocks per CU, so ATTN_FWD_OCC is 2) instead of one copy and two barriers (then 3)
#ifndef ATTN_FWD_DB
#define ATTN_FWD_DB 1
#endif
// the same for the dQ kernel, and its own blocks per CU
#ifndef ATTN_DQ_DB
#define ATTN_DQ_DB 0
#endif
#ifndef ATTN_DQ_OCC
#define ATTN_DQ_OCC 3
#endif
constexpr int NFB = ATTN_AHEAD ? 2 : 1;
GPT2_DEV constexpr int fb(int a) { return ATTN_AHEAD ? (a & 1) : 0; }

GPT2_DEV f32x4 mfma4(float a, float b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

GPT2_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }


// Softmax arithmetic runs in base 2 on the hardware transcendental unit (v_exp_f32,
// v_log_f32): exp(x) = 2^(x log2 e), with log2 e folded into the score scale and the
// stored log-sum-exp converted back to natural log.
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
GPT2_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
GPT2_DEV float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// DG = HS/16 consecutive floats of an interleaved LDS row (aligned to 4*DG bytes).
template <int DG>
GPT2_DEV void lds_get(float (&v)[DG], const float* src) {
    if constexpr (DG == 4) {
        const float4 t = *reinterpret_cast<const float4*>(src);
        v[0] = t.x;
        v[1] = t.y;
        v[2] = t.z;
        v[3] = t.w;
    } else if constexpr (DG == 2) {
        const float2 t = *reinterpret_cast<const float2*>(src);
        v[0] = t.x;
        v[1] = t.y;
    } else {
        v[0] = src[0];
    }
}

template <int DG>
GPT2_DEV void lds_put(float* dst, const float (&v)[DG]) {
    if constexpr (DG == 4) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (DG == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    else dst[0] = v[0];
}

// A 64-row x HS tile of rows [r0, r0+64) (row stride ld floats, rows >= T are zero) in
// registers as 16-byte loads: thread t holds float4 column t % (HS/4) of rows
// t / (HS/4) + (256 / (HS/4)) p.
template <int HS>
GPT2_DEV void tile_load(float4 (&reg)[HS / 16], const float* src, long ld, int r0, int T) {
    constexpr int C4 = HS / 4, RPP = 256 / C4;
    static_assert(RPP * (HS / 16) == TILE, "one pass per 256 threads covers RPP rows");
    const int t = threadIdx.x;
    const float* s0 = src + (long)r0 * ld;  // the tile's first row (uniform)
    if (r0 + TILE <= T) {
        // whole tile inside the sequence: no per-row checks
#pragma unroll
        for (int p = 0; p < HS / 16; p++)
            reg[p] = *reinterpret_cast<const float4*>(s0 + (long)(t / C4 + RPP * p) * ld + (t % C4) * 4);
        return;
    }
#pragma unroll
    for (int p = 0; p < HS / 16; p++) {
        const int r = r0 + t / C4 + RPP * p;
        reg[p] = r < T ? *reinterpret_cast<const float4*>(src + (long)r * ld + (t % C4) * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Writes the tile into the interleaved layout: element e of float4 column c is dimension
// d = 4c + e at position (HS/16)(d % 16) + d / 16.  At HS = 64 a wave's four single-float
// writes per float4 each cover 64 distinct banks.
template <int HS>
GPT2_DEV void tile_store(float* S, const float4 (&reg)[HS / 16]) {
    constexpr int C4 = HS / 4, RPP = 256 / C4, LD = HS + 4, DG = HS / 16;
    const int t = threadIdx.x, c = t % C4;
#pragma unroll
    for (int p = 0; p < HS / 16; p++) {
        float* row = S + (t / C4 + RPP * p) * LD;
        if (DG == 1) {
            *reinterpret_cast<float4*>(row + 4 * c) = reg[p];
        } else {
            const float e4[4] = {reg[p].x, reg[p].y, reg[p].z, reg[p].w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int d = 4 * c + e;
                row[DG * (d % 16) + d / 16] = e4[e];
            }
        }
    }
}

// Keeps the compiler from moving instructions across this point: LDS reads issued before
// it stay ahead of the MFMAs after it, so their latency is covered.
GPT2_DEV void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// This lane's dimensions of one row for the dot-product operand: v[a][j] = row[16j + 4a + g].
template <int HS>
GPT2_DEV void dot_operand(float (&v)[4][HS / 16], const float* row, bool valid, int g) {
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int j = 0; j < HS / 16; j++) v[a][j] = valid ? row[16 * j + 4 * a + g] : 0.f;
}

// ---------------------------------------------------------------------------- forward
// SS: also store the raw scores q.k of every causal (query tile, key tile) pair, laid out
// as the score gradients are (64x64 row-major block per pair, see the dK/dV kernel), so
// that the backward need not form them again.
template <int HS, bool SS>
__global__ __launch_bounds__(256, ATTN_FWD_OCC) void attn_fwd_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                       const float* __restrict__ qkv, int B, int T, int C, int NH,
                                                       float scale, float* __restrict__ sout) {
    constexpr int DG = HS / 16, LD = HS + 4;
    constexpr int NBUF = ATTN_FWD_DB ? 2 : 1;
    __shared__ __attribute__((aligned(16))) float Ks[NBUF][TILE * LD];
    __shared__ __attribute__((aligned(16))) float Vs[NBUF][TILE * LD];
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

    float qreg[4][DG];
    dot_operand<HS>(qreg, base + (long)min(tq, T - 1) * ld + h * HS, tq < T, g4);
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
        if (ATTN_PREFETCH && kt + 1 < nkt) {
            tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
            tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
        }
        const int cur = ATTN_FWD_DB ? (kt & 1) : 0;
        const float* K = Ks[cur];
        const float* V = Vs[cur];
        // S^T[key][query] = K Q^T for 4 blocks of 16 keys, the four chains interleaved;
        // the K runs of step a+1 are read while step a multiplies
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) s[kb] = zero4();
        float kf[NFB][4][DG];
        auto read_k = [&](int a, float (&dst)[4][DG]) {
#pragma unroll
            for (int kb = 0; kb < 4; kb++) lds_get<DG>(dst[kb], K + (kb * 16 + i16) * LD + DG * (4 * a + g4));
        };
        read_k(0, kf[0]);
#pragma unroll
        for (int a = 0; a < 4; a++) {
            if (ATTN_AHEAD && a + 1 < 4) read_k(a + 1, kf[fb(a + 1)]);
            if (!ATTN_AHEAD && a > 0) read_k(a, kf[0]);
            sched_fence();
#pragma unroll
            for (int j = 0; j < DG; j++)
#pragma unroll
                for (int kb = 0; kb < 4; kb++) s[kb] = mfma4(kf[fb(a)][kb][j], qreg[a][j], s[kb]);
            sched_fence();
        }
        // the V runs of the first key block, read while the softmax runs
        float vf[NFB][4][DG];
        auto read_v = [&](int kb, float (&dst)[4][DG]) {
#pragma unroll
            for (int v = 0; v < 4; v++) lds_get<DG>(dst[v], V + (kb * 16 + 4 * g4 + v) * LD + DG * i16);
        };
        read_v(0, vf[0]);
        sched_fence();
        // lane holds raw scores of query tq against keys kt*64 + kb*16 + 4*g4 + v
        if (SS) {
            float* dst = sout + (((long)bh * ((long)nqt * (nqt + 1) / 2) + (long)qt * (qt + 1) / 2 + kt) << 12) +
                         (wave * 16 + i16) * TILE + 4 * g4;
#pragma unroll
            for (int kb = 0; kb < 4; kb++) *reinterpret_cast<f32x4*>(dst + 16 * kb) = s[kb];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                if (DIAG && kt * TILE + kb * 16 + 4 * g4 + v > tq) s[kb][v] = -INFINITY;
                mx = fmaxf(mx, s[kb][v]);
            }
        // The reference max m (base 2) of each row moves only when the row's new max
        // exceeds it by more than 8, i.e. probabilities relative to m stay below 2^8; the
        // result is the same softmax, and O is rescaled only on the (rare, wave-wide)
        // occasions when some row's reference moves.  A row's max exceeds m + 8 exactly
        // when one of its four lanes' partial maxima does, so the row max across the lanes
        // is only formed on those occasions.
        if (__any(mx * scale2 > m + 8.0f)) {
            const float mnew = fmaxf(m, rows4_max(mx) * scale2);
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
        l += rows4_sum(rs);
        // O += P V: for key kb*16 + 4*g4 + v this lane needs V[key][16d + i16], d < DG,
        // which is one interleaved run; block kb+1's runs are read while block kb multiplies
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            if (ATTN_AHEAD && kb + 1 < 4) read_v(kb + 1, vf[fb(kb + 1)]);
            if (!ATTN_AHEAD && kb > 0) read_v(kb, vf[0]);
            sched_fence();
#pragma unroll
            for (int v = 0; v < 4; v++)
#pragma unroll
                for (int d = 0; d < DG; d++) o[d] = mfma4(s[kb][v], vf[fb(kb)][v][d], o[d]);
            sched_fence();
        }
        if (kt + 1 < nkt) {
            if (!ATTN_PREFETCH) {
                tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
                tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
            }
            if (ATTN_FWD_DB) {
                // the other buffer was last read in the previous step, before its barrier
                tile_store<HS>(Ks[cur ^ 1], kreg);
                tile_store<HS>(Vs[cur ^ 1], vreg);
                __syncthreads();
            } else {
                // every wave is done with this tile before the next one overwrites it
                __syncthreads();
                tile_store<HS>(Ks[0], kreg);
                tile_store<HS>(Vs[0], vreg);
                __syncthreads();
            }
        }
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
__global__ __launch_bounds__(256, ATTN_DQ_OCC) void attn_bwd_dq_kernel(float* __restrict__ dqkv, float* __restrict__ delta,
                                                          const float* __restrict__ dout, const float* __restrict__ qkv,
                                                          const float* __restrict__ out, const float* __restrict__ lse,
                                                          int B, int T, int C, int NH, float scale) {
    constexpr int DG = HS / 16, LD = HS + 4;
    constexpr int NBUF = ATTN_DQ_DB ? 2 : 1;
    __shared__ __attribute__((aligned(16))) float Ks[NBUF][TILE * LD];
    __shared__ __attribute__((aligned(16))) float Vs[NBUF][TILE * LD];
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
    const long trow = (long)b * T + min(tq, T - 1);

    float qreg[4][DG], doreg[4][DG], oreg[4][DG];
    dot_operand<HS>(qreg, qkv + trow * ld + h * HS, valid, g4);
    dot_operand<HS>(doreg, dout + trow * C + h * HS, valid, g4);
    dot_operand<HS>(oreg, out + trow * C + h * HS, valid, g4);
    float dd = 0.f;
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int j = 0; j < DG; j++) dd = fmaf(doreg[a][j], oreg[a][j], dd);
    dd = rows4_sum(dd);
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
        if (ATTN_PREFETCH && kt + 1 < nkt) {
            tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
            tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
        }
        const int cur = ATTN_DQ_DB ? (kt & 1) : 0;
        const float* K = Ks[cur];
        const float* V = Vs[cur];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
            f32x4 s = zero4(), dp = zero4();
            // the K runs for dQ first (used last), then K and V fragments one step ahead
            float kr[4][DG];
#pragma unroll
            for (int v = 0; v < 4; v++) lds_get<DG>(kr[v], K + (kb * 16 + 4 * g4 + v) * LD + DG * i16);
            float kf[NFB][DG], vf[NFB][DG];
            auto read_kv = [&](int a, float (&k)[DG], float (&v)[DG]) {
                lds_get<DG>(k, K + (kb * 16 + i16) * LD + DG * (4 * a + g4));
                lds_get<DG>(v, V + (kb * 16 + i16) * LD + DG * (4 * a + g4));
            };
            read_kv(0, kf[0], vf[0]);
#pragma unroll
            for (int a = 0; a < 4; a++) {
                if (ATTN_AHEAD && a + 1 < 4) read_kv(a + 1, kf[fb(a + 1)], vf[fb(a + 1)]);
                if (!ATTN_AHEAD && a > 0) read_kv(a, kf[0], vf[0]);
                sched_fence();
#pragma unroll
                for (int j = 0; j < DG; j++) {
                    s = mfma4(kf[fb(a)][j], qreg[a][j], s);
                    dp = mfma4(vf[fb(a)][j], doreg[a][j], dp);
                }
                sched_fence();
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
            for (int v = 0; v < 4; v++)
#pragma unroll
                for (int d = 0; d < DG; d++) dq[d] = mfma4(ds[v], kr[v][d], dq[d]);
        }
        if (kt + 1 < nkt) {
            if (!ATTN_PREFETCH) {
                tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
                tile_load<HS>(vreg, base + 2 * C + h * HS, ld, (kt + 1) * TILE, T);
            }
            if (ATTN_DQ_DB) {
                // the other buffer was last read in the previous step, before its barrier
                tile_store<HS>(Ks[cur ^ 1], kreg);
                tile_store<HS>(Vs[cur ^ 1], vreg);
                __syncthreads();
            } else {
                // every wave is done with this tile before the next one overwrites it
                __syncthreads();
                tile_store<HS>(Ks[0], kreg);
                tile_store<HS>(Vs[0], vreg);
                __syncthreads();
            }
        }
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
// DS: also store dS (unscaled, p (dP - D)) of every causal (query tile, key tile) pair,
// for the dQ kernel that multiplies it by K instead of recomputing S and dP: tile pair
// (qt, kt <= qt) of (b, h) is the 64x64 row-major block at ((b NH + h) P + qt(qt+1)/2 +
// kt) 4096, P = nqt(nqt+1)/2; entries of masked or out-of-range pairs are 0.
// SL: the raw scores come from the forward's store (sin, same layout) instead of Q K^T.
template <int HS, bool DS, bool SL = false>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(float* __restrict__ dqkv, const float* __restrict__ delta,
                                                            const float* __restrict__ dout, const float* __restrict__ qkv,
                                                            const float* __restrict__ lse, int B, int T, int C, int NH,
                                                            float scale, float* __restrict__ dsout,
                                                            const float* __restrict__ sin = nullptr) {
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

    float kreg[4][DG], vreg[4][DG];
    dot_operand<HS>(kreg, base + (long)min(tu, T - 1) * ld + C + h * HS, tu < T, g4);
    dot_operand<HS>(vreg, base + (long)min(tu, T - 1) * ld + 2 * C + h * HS, tu < T, g4);
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
    // SL: this lane's 16 stored scores of a pair: queries qb*16 + 4*g4 + v (qb, v < 4),
    // key wave*16 + i16; the next pair's requested while this one is used
    float scur[16], snext[16];
    auto load_s = [&](float (&dst)[16], int qt) {
        const float* src = sin + (((long)bh * ((long)nqt * (nqt + 1) / 2) + (long)qt * (qt + 1) / 2 + kt) << 12) +
                           (4 * g4) * TILE + wave * 16 + i16;
#pragma unroll
        for (int qb = 0; qb < 4; qb++)
#pragma unroll
            for (int v = 0; v < 4; v++) dst[4 * qb + v] = src[(qb * 16 + v) * TILE];
    };
    if (SL) load_s(scur, kt);
    // one query tile; only the diagonal tile (qt == kt) has queries before the key
    auto step = [&](int qt, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const int cur = (qt - kt) & 1;
        if (qt + 1 < nqt) {
            tile_load<HS>(qreg, base + h * HS, ld, (qt + 1) * TILE, T);
            tile_load<HS>(oreg, dbase + h * HS, C, (qt + 1) * TILE, T);
            load_side(qt + 1);
            if (SL) load_s(snext, qt + 1);
        }
        const float* Q = Qs[cur];
        const float* O = Os[cur];
#pragma unroll
        for (int qb = 0; qb < 4; qb++) {
            f32x4 s = zero4(), dp = zero4();
            // dV += P^T dO, dK += dS^T Q: this lane needs dO and Q of query qb*16 + 4*g4 + v
            // at dimensions 16d + i16, one interleaved run each (read first, used last)
            float orun[4][DG], qrun[4][DG];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int qi = qb * 16 + 4 * g4 + v;
                lds_get<DG>(orun[v], O + qi * LD + DG * i16);
                lds_get<DG>(qrun[v], Q + qi * LD + DG * i16);
            }
            float qf[2][DG], of[2][DG];
            auto read_qo = [&](int a, float (&q)[DG], float (&o)[DG]) {
                if (!SL) lds_get<DG>(q, Q + (qb * 16 + i16) * LD + DG * (4 * a + g4));
                lds_get<DG>(o, O + (qb * 16 + i16) * LD + DG * (4 * a + g4));
            };
            read_qo(0, qf[0], of[0]);
#pragma unroll
            for (int a = 0; a < 4; a++) {
                if (a + 1 < 4) read_qo(a + 1, qf[(a + 1) & 1], of[(a + 1) & 1]);
                sched_fence();
#pragma unroll
                for (int j = 0; j < DG; j++) {
                    if (!SL) s = mfma4(qf[a & 1][j], kreg[a][j], s);
                    dp = mfma4(of[a & 1][j], vreg[a][j], dp);
                }
                sched_fence();
            }
            if (SL) {
#pragma unroll
                for (int v = 0; v < 4; v++) s[v] = scur[4 * qb + v];
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
            if (DS) {
                // this lane: queries qb*16 + 4*g4 + v of the tile, key wave*16 + i16
                float* dst = dsout + (((long)bh * ((long)nqt * (nqt + 1) / 2) + (long)qt * (qt + 1) / 2 + kt) << 12) +
                             (qb * 16 + 4 * g4) * TILE + wave * 16 + i16;
#pragma unroll
                for (int v = 0; v < 4; v++) dst[v * TILE] = ds[v];
            }
#pragma unroll
            for (int v = 0; v < 4; v++)
#pragma unroll
                for (int d = 0; d < DG; d++) {
                    dv[d] = mfma4(p[v], orun[v][d], dv[d]);
                    dk[d] = mfma4(ds[v], qrun[v][d], dk[d]);
                }
        }
        if (qt + 1 < nqt) {
            tile_store<HS>(Qs[cur ^ 1], qreg);
            tile_store<HS>(Os[cur ^ 1], oreg);
            store_side(cur ^ 1);
            if (SL) {
#pragma unroll
                for (int e = 0; e < 16; e++) scur[e] = snext[e];
            }
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

// D_t = dO_t . o_t of every (row, head): a wave per row, lane l holding float4 l of each
// 256-float pass (all passes requested first, up to four at a time); each lane's four
// products are added in order, then the HS/4 lanes of a head by DPP steps (within quads,
// then half rows, then rows).
template <int GL>
GPT2_DEV float group_sum(float x) {
    x += dpp_f<DPP_XOR1>(x);
    x += dpp_f<DPP_XOR2>(x);
    if (GL >= 8) x += dpp_f<DPP_HALF_MIRROR>(x);
    if (GL >= 16) x += dpp_f<DPP_MIRROR>(x);
    return x;
}
template <int HS>
__global__ __launch_bounds__(256) void attn_delta_kernel(float* __restrict__ delta, const float* __restrict__ dout,
                                                         const float* __restrict__ out, int B, int T, int C, int NH) {
    constexpr int GL = HS / 4;  // lanes per head
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (long)B * T) return;  // the whole wave: row is uniform over it
    const int C4 = C / 4;
    const float4* a = reinterpret_cast<const float4*>(dout + row * C);
    const float4* o = reinterpret_cast<const float4*>(out + row * C);
    const long b = row / T, t = row - b * T;
    for (int p0 = 0; p0 < C4; p0 += 256) {
        float4 x[4], y[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int i = p0 + 64 * q + lane;
            x[q] = i < C4 ? a[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            y[q] = i < C4 ? o[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int i = p0 + 64 * q + lane;
            if (p0 + 64 * q >= C4) break;  // uniform
            float s = x[q].x * y[q].x;
            s = fmaf(x[q].y, y[q].y, s);
            s = fmaf(x[q].z, y[q].z, s);
            s = fmaf(x[q].w, y[q].w, s);
            s = group_sum<GL>(s);
            if (i < C4 && lane % GL == 0) delta[(b * NH + i / GL) * T + t] = s;
        }
    }
}

// dQ = scale dS K from the dS blocks the dK/dV kernel stored: a block per 64-query tile
// (longest first), 4 waves x 16 queries.  Per key tile the K tile goes through LDS, stored
// plainly (row-major, one 16-byte write per float4: the interleaved layout's scalar writes
// would cost as much as the tile's reads here) and double-buffered (one barrier per tile),
// and each lane takes its query row's 16 dS values at keys 16 g4 .. 16 g4 + 15 straight
// from memory (the next tile's requested while this one multiplies).  MFMA step m (m < 16)
// has k slot g4 hold key 16 g4 + m, so a lane's A values are its 16 consecutive dS; output
// block db holds dimensions DG j + db in column j, so a lane's B values for all blocks are
// the DG consecutive floats of key row 16 g4 + m at DG i16 (one LDS read), and its
// results for query row v are DG consecutive floats (one store).  One product per pair
// instead of the three (S, dP, dS K) of recomputation.
template <int HS>
__global__ __launch_bounds__(256, 3) void attn_bwd_dq_ds_kernel(float* __restrict__ dqkv, const float* __restrict__ ds,
                                                                const float* __restrict__ qkv, int B, int T, int C,
                                                                int NH, float scale) {
    constexpr int DG = HS / 16, LD = HS + 4, C4 = HS / 4, RPP = 256 / C4;
    __shared__ __attribute__((aligned(16))) float Ks[2][TILE * LD];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int qt = nqt - 1 - (int)(blockIdx.x / (B * NH));  // longest rows first
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const long ld = 3L * C;
    const float* base = qkv + (long)b * T * ld;
    // this lane's dS row (query wave*16 + i16 of the tile), keys 16*g4 .. 16*g4 + 15, of pair (qt, kt)
    const float* arow = ds + (((long)bh * ((long)nqt * (nqt + 1) / 2) + (long)qt * (qt + 1) / 2) << 12) +
                        (wave * 16 + i16) * TILE + 16 * g4;
    // plain row-major K tile: thread t's float4 p sits at row t / C4 + RPP p, column 4 (t % C4)
    auto kstore = [&](float* S, const float4 (&reg)[HS / 16]) {
#pragma unroll
        for (int p = 0; p < HS / 16; p++)
            *reinterpret_cast<float4*>(S + (threadIdx.x / C4 + RPP * p) * LD + 4 * (threadIdx.x % C4)) = reg[p];
    };
    f32x4 dq[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) dq[d] = zero4();
    float4 acur[4], anxt[4];
#pragma unroll
    for (int j = 0; j < 4; j++) acur[j] = reinterpret_cast<const float4*>(arow)[j];
    float4 kreg[DG];
    tile_load<HS>(kreg, base + C + h * HS, ld, 0, T);
    kstore(Ks[0], kreg);
    __syncthreads();
    for (int kt = 0; kt <= qt; kt++) {
        const int cur = kt & 1;
        if (kt < qt) {
            tile_load<HS>(kreg, base + C + h * HS, ld, (kt + 1) * TILE, T);
            const float4* an = reinterpret_cast<const float4*>(arow + ((long)(kt + 1) << 12));
#pragma unroll
            for (int j = 0; j < 4; j++) anxt[j] = an[j];
        }
        const float* K = Ks[cur];
        const float av[16] = {acur[0].x, acur[0].y, acur[0].z, acur[0].w, acur[1].x, acur[1].y, acur[1].z, acur[1].w,
                              acur[2].x, acur[2].y, acur[2].z, acur[2].w, acur[3].x, acur[3].y, acur[3].z, acur[3].w};
        float kf[2][DG];
        lds_get<DG>(kf[0], K + (16 * g4) * LD + DG * i16);
#pragma unroll
        for (int m = 0; m < 16; m++) {
            if (m + 1 < 16) lds_get<DG>(kf[(m + 1) & 1], K + (16 * g4 + m + 1) * LD + DG * i16);
            sched_fence();
#pragma unroll
            for (int d = 0; d < DG; d++) dq[d] = mfma4(av[m], kf[m & 1][d], dq[d]);
            sched_fence();
        }
        if (kt < qt) {
            // the other buffer was last read in the previous step, before its barrier
            kstore(Ks[cur ^ 1], kreg);
#pragma unroll
            for (int j = 0; j < 4; j++) acur[j] = anxt[j];
            __syncthreads();
        }
    }
    const int q0 = qt * TILE + wave * 16;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int q = q0 + 4 * g4 + v;
        if (q < T) {
            float o[DG];
#pragma unroll
            for (int d = 0; d < DG; d++) o[d] = dq[d][v] * scale;
            lds_put<DG>(dqkv + ((long)b * T + q) * ld + h * HS + DG * i16, o);
        }
    }
}

template <int HS, bool SS>
const char* fwd_name() {
    static const std::string n = "attn_fwd_kernel<" + std::to_string(HS) + (SS ? ", true>" : ", false>");
    return n.c_str();
}
template <int HS>
const char* dq_name() {
    return HS == 16 ? "attn_bwd_dq_kernel<16>" : HS == 32 ? "attn_bwd_dq_kernel<32>" : "attn_bwd_dq_kernel<64>";
}
// as the profiler prints the instantiation
template <int HS, bool DS = false, bool SL = false>
const char* dkdv_name() {
    static const std::string n = "attn_bwd_dkdv_kernel<" + std::to_string(HS) + (DS ? ", true" : ", false") +
                                 (SL ? ", true>" : ", false>");
    return n.c_str();
}

template <int HS>
void launch_fwd(float* out, float* lse, const float* qkv, int B, int T, int C, int NH, hipStream_t st, float* sbuf) {
    const int nqt = (T + TILE - 1) / TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    // causal half: T(T+1)/2 (query, key) pairs per (b, h), two products of HS MACs each
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    if (sbuf) {
        ProfScope ps(st, fwd_name<HS, true>(), pairs * HS * 2 * 2,
                     4.0 * B * T * (3.0 * C + C + NH) + 4.0 * attn_ds_floats(B, T, NH));
        hipLaunchKernelGGL((attn_fwd_kernel<HS, true>), dim3(nqt * B * NH), dim3(256), 0, st, out, lse, qkv, B, T, C,
                           NH, scale, sbuf);
        return;
    }
    ProfScope ps(st, fwd_name<HS, false>(), pairs * HS * 2 * 2, 4.0 * B * T * (3.0 * C + C + NH));
    hipLaunchKernelGGL((attn_fwd_kernel<HS, false>), dim3(nqt * B * NH), dim3(256), 0, st, out, lse, qkv, B, T, C, NH,
                       scale, (float*)nullptr);
}

template <int HS>
const char* delta_name() {
    return HS == 16 ? "attn_delta_kernel<16>" : HS == 32 ? "attn_delta_kernel<32>" : "attn_delta_kernel<64>";
}
template <int HS>
const char* dqds_name() {
    return HS == 16 ? "attn_bwd_dq_ds_kernel<16>" : HS == 32 ? "attn_bwd_dq_ds_kernel<32>" : "attn_bwd_dq_ds_kernel<64>";
}

template <int HS>
void launch_bwd(float* dqkv, float* delta, const float* dout, const float* qkv, const float* out, const float* lse,
                int B, int T, int C, int NH, hipStream_t st, float* ds, const float* sbuf) {
    const int nt = (T + TILE - 1) / TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    if (ds) {
        const double rows = (double)B * T, dsbytes = 4.0 * attn_ds_floats(B, T, NH);
        {
            ProfScope ps(st, delta_name<HS>(), 0.0, 4.0 * (2.0 * rows * C + rows * NH));
            const long n = (long)B * T;
            hipLaunchKernelGGL(attn_delta_kernel<HS>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, delta, dout,
                               out, B, T, C, NH);
        }
        if (sbuf) {
            // products formed: dP, dV, dK (S from the forward's store); dS stored
            ProfScope ps(st, dkdv_name<HS, true, true>(), pairs * HS * 2 * 3,
                         4.0 * rows * (3.0 * C + C + 2.0 * C + 2 * NH) + 2.0 * dsbytes);
            hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HS, true, true>), dim3(nt * B * NH), dim3(256), 0, st, dqkv,
                               (const float*)delta, dout, qkv, lse, B, T, C, NH, scale, ds, sbuf);
        } else {
            // products formed: S (recomputed), dP, dV, dK; dS stored
            ProfScope ps(st, dkdv_name<HS, true>(), pairs * HS * 2 * 4,
                         4.0 * rows * (3.0 * C + C + 2.0 * C + 2 * NH) + dsbytes);
            hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HS, true>), dim3(nt * B * NH), dim3(256), 0, st, dqkv,
                               (const float*)delta, dout, qkv, lse, B, T, C, NH, scale, ds);
        }
        // products formed: dQ = dS K
        ProfScope ps(st, dqds_name<HS>(), pairs * HS * 2, 4.0 * rows * (C + C) + dsbytes);
        hipLaunchKernelGGL(attn_bwd_dq_ds_kernel<HS>, dim3(nt * B * NH), dim3(256), 0, st, dqkv, (const float*)ds, qkv,
                           B, T, C, NH, scale);
        return;
    }
    {
        // products formed: S (recomputed), dP, dQ
        ProfScope ps(st, dq_name<HS>(), pairs * HS * 2 * 3, 4.0 * B * T * (2.0 * C + 3.0 * C + 2 * NH));
        hipLaunchKernelGGL(attn_bwd_dq_kernel<HS>, dim3(nt * B * NH), dim3(256), 0, st, dqkv, delta, dout, qkv, out,
                           lse, B, T, C, NH, scale);
    }
    // products formed: S (recomputed), dP, dV, dK
    ProfScope ps(st, dkdv_name<HS>(), pairs * HS * 2 * 4, 4.0 * B * T * (3.0 * C + C + 2.0 * C + 2 * NH));
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HS, false>), dim3(nt * B * NH), dim3(256), 0, st, dqkv,
                       (const float*)delta, dout, qkv, lse, B, T, C, NH, scale, (float*)nullptr);
}

}  // namespace

hipError_t attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                             hipStream_t st, float* sbuf) {
    if (C % NH || C % 4) return hipErrorInvalidValue;
    if ((long)B * T == 0) return hipSuccess;
    switch (C / NH) {
        case 16: launch_fwd<16>(out, lse, qkv, B, T, C, NH, st, sbuf); break;
        case 32: launch_fwd<32>(out, lse, qkv, B, T, C, NH, st, sbuf); break;
        case 64: launch_fwd<64>(out, lse, qkv, B, T, C, NH, st, sbuf); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

size_t attn_ds_floats(int B, int T, int NH) {
    const size_t nqt = (size_t)(T + TILE - 1) / TILE;
    return (size_t)B * NH * (nqt * (nqt + 1) / 2) * TILE * TILE;
}

hipError_t attention_backward(float* dqkv, float* delta, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C, int NH,
                              hipStream_t st, float* ds, const float* sbuf) {
    if (C % NH || C % 4) return hipErrorInvalidValue;
    if ((long)B * T == 0) return hipSuccess;
    if ((ds && ((uintptr_t)ds & 15)) || (sbuf && ((uintptr_t)sbuf & 15))) return hipErrorInvalidValue;
    switch (C / NH) {
        case 16: launch_bwd<16>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st, ds, ds ? sbuf : nullptr); break;
        case 32: launch_bwd<32>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st, ds, ds ? sbuf : nullptr); break;
        case 64: launch_bwd<64>(dqkv, delta, dout, qkv, out, lse, B, T, C, NH, st, ds, ds ? sbuf : nullptr); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gpt2k
