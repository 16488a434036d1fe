// Causal multi-head attention of the mixed-precision variant on the bf16 matrix cores.
//
// Same layer as attention.hip (the pages' attention_forward / attention_backward: huxiu
// page "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1), with the
// mixed-precision reading: the products take bf16 roundings of q, k, v and of the output
// gradient dO, while the probabilities p and score gradients ds stay unrounded.  A
// product with p or ds as an operand is done as three bf16 MFMAs, of hi = bf16(x),
// mid = bf16(x - hi) and lo = bf16(x - hi - mid): each rounding leaves at most 2^-8 of
// what it rounds, so |x - hi - mid - lo| <= 2^-24 |x|, fp32's own precision.
//   forward:   s = bf16(q).bf16(k) scale, p = softmax(s), o = p . bf16(v)
//   backward:  dv = p^T bf16(dO);  dp = bf16(dO) . bf16(v);  D = bf16(dO) . o (which is
//              sum_u p_u dp_u exactly);  ds = p (dp - D);  dq = ds . bf16(k) scale;
//              dk = ds^T bf16(q) scale.
//
// Operand layouts.  v_mfma_f32_16x16x32_bf16 takes from lane i + 16g the 8 values of
// k-slots 8g..8g+7 of row i (A) or column i (B); its 16x16 fp32 result C[i][j] sits in
// lane j + 16(i/4), register i%4, as in every 16x16 MFMA.  A bf16 copy of each head is
// kept per (batch, head) in two layouts (attn_prep_kernel):
//   row-major (T, HS): a lane's 8 consecutive head dimensions are one 16-byte read (the
//     operands of products summed over the head dimension: s, dp);
//   transposed (HS, Tp): for each dimension, the tokens of every 64-token tile permuted so
//     that position 32P + 8g + 4h + v holds token 16(2P + h) + 4g + v.  A score block
//     computed transposed (keys as rows) leaves in lane j + 16g, for key blocks 2P and
//     2P+1, exactly the tokens 16(2P+h) + 4g + v: the 8 k-slots of the next product's A
//     operand, in registers; the permutation puts the matching B operand values (v, k, q
//     or dO of those tokens) in one 16-byte read.
// LDS rows are padded by 8 bf16 so that 16 lanes reading 16 rows hit 16 bank groups.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TILE = 64, NTH = 256;
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;

GPT2_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
GPT2_DEV float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
GPT2_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
GPT2_DEV f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
GPT2_DEV bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u)); }
GPT2_DEV bf16x8 ld8(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p)); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
GPT2_DEV float bf16_float(uint32_t b) { return __uint_as_float(b << 16); }

// x = hi + mid + lo + r, |r| <= 2^-24 |x|, with hi, mid, lo bf16 (see the header); each
// rounding of a pair is one v_cvt_pk_bf16_f32 (round to nearest, ties to even)
struct Split3 {
    bf16x8 p[3];
};
GPT2_DEV Split3 split8(const float (&x)[8]) {
    uint32_t w[3][4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        f32x2 r = {x[2 * e], x[2 * e + 1]};
#pragma unroll
        for (int k = 0; k < 3; k++) {
            const bf16x2 h = __builtin_convertvector(r, bf16x2);
            w[k][e] = __builtin_bit_cast(uint32_t, h);
            r -= __builtin_convertvector(h, f32x2);
        }
    }
    Split3 s;
#pragma unroll
    for (int k = 0; k < 3; k++) s.p[k] = __builtin_bit_cast(bf16x8, make_uint4(w[k][0], w[k][1], w[k][2], w[k][3]));
    return s;
}
// c += x . b with x split in three
GPT2_DEV f32x4 mfma3(const Split3& x, bf16x8 b, f32x4 c) {
    c = mfma(x.p[0], b, c);
    c = mfma(x.p[1], b, c);
    return mfma(x.p[2], b, c);
}

// the two key (or query) blocks 2P, 2P+1 of a lane's score registers as one operand
GPT2_DEV void pair8(float (&x)[8], const f32x4& a, const f32x4& b) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
        x[v] = a[v];
        x[4 + v] = b[v];
    }
}

// token position inside a 64-token tile of a transposed copy (an involution is not
// needed: the prep kernel maps positions back to tokens with tok_of_pos)
GPT2_DEV int tok_of_pos(int pos) {
    const int P = pos >> 5, g = (pos >> 3) & 3, hh = (pos >> 2) & 1, v = pos & 3;
    return 16 * (2 * P + hh) + 4 * g + v;
}

// ------------------------------------------------------------------- bf16 head copies
// Grid (Tp/64, B*NH, sources).  Source z is the fp32 (B, T, ld) tensor src + z*zoff, head
// h at columns h*HS; row-major copy rm[z] (B*NH, T, HS), transposed copy tr[z]
// (B*NH, HS, Tp) (either may be null), tokens >= T zero in the transposed copy.
struct PrepArgs {
    const float* src;
    long ld, zoff;
    uint16_t* rm[3];
    uint16_t* tr[3];
    int B, T, NH, HS, Tp;
};

__global__ __launch_bounds__(NTH) void attn_prep_kernel(PrepArgs a) {
    __shared__ float tile[TILE][64 + 1];
    const int t = threadIdx.x, z = blockIdx.z;
    const int bh = blockIdx.y, b = bh / a.NH, h = bh % a.NH;
    const int t0 = blockIdx.x * TILE, HS = a.HS, C4 = HS / 4;
    const float* src = a.src + (long)z * a.zoff + (long)b * a.T * a.ld + h * HS;
    uint16_t* rm = a.rm[z];
    uint16_t* tr = a.tr[z];
    for (int c = t; c < TILE * C4; c += NTH) {
        const int r = c / C4, d4 = (c % C4) * 4, tok = t0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok < a.T) {
            v = *reinterpret_cast<const float4*>(src + (long)tok * a.ld + d4);
            if (rm) {
                uint2 o;
                o.x = bf16_pack2(v.x, v.y);
                o.y = bf16_pack2(v.z, v.w);
                *reinterpret_cast<uint2*>(rm + ((long)bh * a.T + tok) * HS + d4) = o;
            }
        }
        tile[r][d4 + 0] = v.x;
        tile[r][d4 + 1] = v.y;
        tile[r][d4 + 2] = v.z;
        tile[r][d4 + 3] = v.w;
    }
    if (!tr) return;
    __syncthreads();
    // transposed: (dimension d, 8 consecutive positions) per 16-byte store
    for (int c = t; c < HS * 8; c += NTH) {
        const int d = c / 8, pos0 = (c % 8) * 8;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
            w[e] = bf16_pack2(tile[tok_of_pos(pos0 + 2 * e)][d], tile[tok_of_pos(pos0 + 2 * e + 1)][d]);
        *reinterpret_cast<uint4*>(tr + ((long)bh * HS + d) * a.Tp + t0 + pos0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ------------------------------------------------------------------- tile staging
// A 64-row slab of a row-major copy (rows >= T zero) or of a transposed copy, moved
// through registers (16-byte chunks) into a padded LDS tile.
template <int HS>
struct RowTile {
    static constexpr int CPR = HS / 8, CH = TILE * CPR, PER = (CH + NTH - 1) / NTH, RS = HS + 8;
    uint4 r[PER];
    GPT2_DEV void load(const uint16_t* src, int r0, int T) {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int c = threadIdx.x + NTH * p, row = c / CPR, col = (c % CPR) * 8;
            r[p] = (c < CH && r0 + row < T) ? *reinterpret_cast<const uint4*>(src + (long)(r0 + row) * HS + col)
                                            : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    GPT2_DEV void store(uint16_t* S) const {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int c = threadIdx.x + NTH * p, row = c / CPR, col = (c % CPR) * 8;
            if (c < CH) *reinterpret_cast<uint4*>(S + row * RS + col) = r[p];
        }
    }
};

template <int HS>
struct TrTile {
    static constexpr int CH = HS * 8, PER = (CH + NTH - 1) / NTH, TS = TILE + 8;
    uint4 r[PER];
    GPT2_DEV void load(const uint16_t* src, int t0, int Tp) {  // src: (HS, Tp) of one head
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int c = threadIdx.x + NTH * p, d = c / 8, col = (c % 8) * 8;
            r[p] = c < CH ? *reinterpret_cast<const uint4*>(src + (long)d * Tp + t0 + col) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    GPT2_DEV void store(uint16_t* S) const {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int c = threadIdx.x + NTH * p, d = c / 8, col = (c % 8) * 8;
            if (c < CH) *reinterpret_cast<uint4*>(S + d * TS + col) = r[p];
        }
    }
};

// operand of a product over the head dimension from a row-major LDS tile: row r, k-step
// ks, lane group g (zero past HS)
template <int HS>
GPT2_DEV bf16x8 dot_frag(const uint16_t* S, int r, int ks, int g) {
    return 32 * ks + 8 * g < HS ? ld8(S + r * (HS + 8) + 32 * ks + 8 * g) : zero8();
}
// B operand of a product over tokens from a transposed LDS tile: dimension d, token pair P
GPT2_DEV const uint16_t* tr_frag_ptr(const uint16_t* S, int d, int P, int g) { return S + d * (TILE + 8) + 32 * P + 8 * g; }

template <int HS>
GPT2_DEV void head_frags(bf16x8 (&f)[(HS + 31) / 32], const uint16_t* row, bool valid, int g) {
#pragma unroll
    for (int ks = 0; ks < (HS + 31) / 32; ks++)
        f[ks] = valid && 32 * ks + 8 * g < HS ? ld8(row + 32 * ks + 8 * g) : zero8();
}

// ---------------------------------------------------------------------------- forward
template <int HS>
__global__ __launch_bounds__(NTH, 2) void attn_fwd_bf16_kernel(float* __restrict__ out, uint16_t* __restrict__ outb,
                                                             float* __restrict__ lse,
                                                             const uint16_t* __restrict__ qb,
                                                             const uint16_t* __restrict__ kb,
                                                             const uint16_t* __restrict__ vt, int B, int T, int C,
                                                             int NH, int Tp, float scale) {
    constexpr int NKS = (HS + 31) / 32, DG = HS / 16, RS = HS + 8, TS = TILE + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[HS * TS];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int qt = nqt - 1 - (int)(blockIdx.x / (B * NH));  // longest rows first
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int q0 = qt * TILE + wave * 16, tq = q0 + i16;
    const uint16_t* Kh = kb + (long)bh * T * HS;
    const uint16_t* Vh = vt + (long)bh * HS * Tp;

    bf16x8 qf[NKS];
    head_frags<HS>(qf, qb + ((long)bh * T + min(tq, T - 1)) * HS, tq < T, g4);
    f32x4 o[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) o[d] = zero4();
    float m = -INFINITY, l = 0.f;  // running max (base 2) and sum of this lane's query row
    const float scale2 = scale * LOG2E;

    RowTile<HS> kr;
    TrTile<HS> vr;
    const int nkt = qt + 1;
    kr.load(Kh, 0, T);
    vr.load(Vh, 0, Tp);
    kr.store(Ks);
    vr.store(Vt);
    __syncthreads();
    auto step = [&](int kt, auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if (kt + 1 < nkt) {
            kr.load(Kh, (kt + 1) * TILE, T);
            vr.load(Vh, (kt + 1) * TILE, Tp);
        }
        // S^T[key][query] for 4 blocks of 16 keys
        f32x4 s[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++) s[k4] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ks++)
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) s[k4] = mfma(dot_frag<HS>(Ks, k4 * 16 + i16, ks, g4), qf[ks], s[k4]);
        // lane holds raw scores of query tq against keys kt*64 + k4*16 + 4*g4 + v
        float mx = -INFINITY;
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                if (DIAG && kt * TILE + k4 * 16 + 4 * g4 + v > tq) s[k4][v] = -INFINITY;
                mx = fmaxf(mx, s[k4][v]);
            }
        // the reference max moves only when a row's max exceeds it by more than 8 (base 2);
        // the softmax is the same, and O is rescaled only then.  A row's max does so exactly
        // when one of its four lanes' partial maxima does, so the row max is formed only then.
        if (__any(mx * scale2 > m + 8.0f)) {
            const float mnew = fmaxf(m, rows4_max(mx) * scale2);
            const float alpha = exp2_hw(m - mnew);
            l *= alpha;
            m = mnew;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float a = __shfl(alpha, 4 * g4 + v, 64);
#pragma unroll
                for (int d = 0; d < DG; d++) o[d][v] *= a;
            }
        }
        float rs = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float p = exp2_hw(fmaf(s[k4][v], scale2, -m));
                s[k4][v] = p;
                rs += p;
            }
        l += rows4_sum(rs);
        // O += P V over key pairs (2P, 2P+1): P as hi + lo
#pragma unroll
        for (int P = 0; P < 2; P++) {
            float x[8];
            pair8(x, s[2 * P], s[2 * P + 1]);
            const Split3 ps = split8(x);
#pragma unroll
            for (int d = 0; d < DG; d++) o[d] = mfma3(ps, ld8(tr_frag_ptr(Vt, d * 16 + i16, P, g4)), o[d]);
        }
        if (kt + 1 < nkt) {
            __syncthreads();
            kr.store(Ks);
            vr.store(Vt);
            __syncthreads();
        }
    };
    for (int kt = 0; kt < qt; kt++) step(kt, std::false_type{});
    step(qt, std::true_type{});
    const float linv = 1.0f / l;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const float a = __shfl(linv, 4 * g4 + v, 64);
#pragma unroll
        for (int d = 0; d < DG; d++) o[d][v] *= a;
    }
    const long orow0 = ((long)b * T + q0 + 4 * g4) * C + h * HS + i16;
#pragma unroll
    for (int v = 0; v < 4; v++)
        if (q0 + 4 * g4 + v < T) {
#pragma unroll
            for (int d = 0; d < DG; d++) out[orow0 + v * (long)C + 16 * d] = o[d][v];
        }
    if (outb) {
        // the bf16 copy of the output, the next GEMM's operand
#pragma unroll
        for (int v = 0; v < 4; v += 2)
#pragma unroll
            for (int d = 0; d < DG; d++) {
                uint16_t* p0 = outb + orow0 + v * (long)C + 16 * d;
                bf16_store_rows2(p0, p0 + C, o[d][v], o[d][v + 1], q0 + 4 * g4 + v < T, q0 + 4 * g4 + v + 1 < T);
            }
    }
    if (g4 == 0 && tq < T) lse[((long)b * NH + h) * T + tq] = (m + log2_hw(l)) * LN2;
}

// Output of a backward kernel: each wave holds 16 rows (row0 + 4 g4 + v) x 16 DG columns
// (i16 + 16 d) of the block's 64 x HS tile.  Stores the fp32 values, optionally their bf16
// rounding (pairs of rows through bf16_store_rows2), and optionally the tile's column sums
// over the rows inside the sequence (the bias gradient's partial row), added in a fixed
// order: v, then the four lane groups, then the four waves.  red is LDS scratch of
// 64 DG floats that no wave reads any more.
template <int DG>
GPT2_DEV void write_grad(const f32x4 (&x)[DG], float* out, uint16_t* outb, long ld, int row0, int T, float* csum,
                         float* red, int wave, int i16, int g4) {
#pragma unroll
    for (int v = 0; v < 4; v++)
        if (row0 + 4 * g4 + v < T) {
#pragma unroll
            for (int d = 0; d < DG; d++) out[(long)(4 * g4 + v) * ld + 16 * d] = x[d][v];
        }
    if (outb) {
#pragma unroll
        for (int v = 0; v < 4; v += 2)
#pragma unroll
            for (int d = 0; d < DG; d++) {
                uint16_t* p0 = outb + (long)(4 * g4 + v) * ld + 16 * d;
                bf16_store_rows2(p0, p0 + ld, x[d][v], x[d][v + 1], row0 + 4 * g4 + v < T, row0 + 4 * g4 + v + 1 < T);
            }
    }
    if (csum) {
        __syncthreads();
#pragma unroll
        for (int d = 0; d < DG; d++) {
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; v++)
                if (row0 + 4 * g4 + v < T) sum += x[d][v];
            sum = rows4_sum(sum);
            if (g4 == 0) red[wave * 16 * DG + 16 * d + i16] = sum;
        }
        __syncthreads();
        const int t = threadIdx.x;
        if (t < 16 * DG) csum[t] = ((red[t] + red[16 * DG + t]) + red[32 * DG + t]) + red[48 * DG + t];
    }
}

// ---------------------------------------------------------------------------- dq (+ D)
template <int HS>
__global__ __launch_bounds__(NTH, 2) void attn_bwd_dq_bf16_kernel(
    float* __restrict__ dqkv, uint16_t* __restrict__ dqkvb, float* __restrict__ bsum, float* __restrict__ delta,
    const uint16_t* __restrict__ dob, const float* __restrict__ out, const uint16_t* __restrict__ qb, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ kt_, const float* __restrict__ lse, int B, int T,
    int C, int NH, int Tp, float scale) {
    constexpr int NKS = (HS + 31) / 32, DG = HS / 16, RS = HS + 8, TS = TILE + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[TILE * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Kt[HS * TS];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int qt = nqt - 1 - (int)(blockIdx.x / (B * NH));
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int q0 = qt * TILE + wave * 16, tq = q0 + i16;
    const bool valid = tq < T;
    const int tqc = min(tq, T - 1);
    const uint16_t* Kh = kb + (long)bh * T * HS;
    const uint16_t* Vh = vb + (long)bh * T * HS;
    const uint16_t* KTh = kt_ + (long)bh * HS * Tp;

    bf16x8 qf[NKS], df[NKS];
    head_frags<HS>(qf, qb + ((long)bh * T + tqc) * HS, valid, g4);
    head_frags<HS>(df, dob + ((long)bh * T + tqc) * HS, valid, g4);
    // D = bf16(dO) . o over this row: each lane its 8 dimensions per k-step
    float dd = 0.f;
    const float* orow = out + ((long)b * T + tqc) * C + h * HS;
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
        if (32 * ks + 8 * g4 < HS) {
            const uint4 u = __builtin_bit_cast(uint4, df[ks]);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                dd = fmaf(bf16_float((w[e / 2] >> (16 * (e & 1))) & 0xffffu), orow[32 * ks + 8 * g4 + e], dd);
        }
    }
    dd = rows4_sum(dd);
    const float D = valid ? dd : 0.f;
    const float L2 = (valid ? lse[((long)b * NH + h) * T + tq] : INFINITY) * LOG2E, scale2 = scale * LOG2E;
    if (g4 == 0 && valid) delta[((long)b * NH + h) * T + tq] = D;

    f32x4 dq[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) dq[d] = zero4();
    RowTile<HS> kr, vr;
    TrTile<HS> ktr;
    const int nkt = qt + 1;
    kr.load(Kh, 0, T);
    vr.load(Vh, 0, T);
    ktr.load(KTh, 0, Tp);
    kr.store(Ks);
    vr.store(Vs);
    ktr.store(Kt);
    __syncthreads();
    auto step = [&](int kt, auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if (kt + 1 < nkt) {
            kr.load(Kh, (kt + 1) * TILE, T);
            vr.load(Vh, (kt + 1) * TILE, T);
            ktr.load(KTh, (kt + 1) * TILE, Tp);
        }
        f32x4 s[4], dp[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++) {
            s[k4] = zero4();
            dp[k4] = zero4();
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ks++)
#pragma unroll
            for (int k4 = 0; k4 < 4; k4++) {
                s[k4] = mfma(dot_frag<HS>(Ks, k4 * 16 + i16, ks, g4), qf[ks], s[k4]);
                dp[k4] = mfma(dot_frag<HS>(Vs, k4 * 16 + i16, ks, g4), df[ks], dp[k4]);
            }
        // lane: query tq, keys kt*64 + k4*16 + 4*g4 + v
#pragma unroll
        for (int k4 = 0; k4 < 4; k4++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int key = kt * TILE + k4 * 16 + 4 * g4 + v;
                const float p = (!DIAG || key <= tq) ? exp2_hw(fmaf(s[k4][v], scale2, -L2)) : 0.f;
                s[k4][v] = p * (dp[k4][v] - D);
            }
#pragma unroll
        for (int P = 0; P < 2; P++) {
            float x[8];
            pair8(x, s[2 * P], s[2 * P + 1]);
            const Split3 ds = split8(x);
#pragma unroll
            for (int d = 0; d < DG; d++) dq[d] = mfma3(ds, ld8(tr_frag_ptr(Kt, d * 16 + i16, P, g4)), dq[d]);
        }
        if (kt + 1 < nkt) {
            __syncthreads();
            kr.store(Ks);
            vr.store(Vs);
            ktr.store(Kt);
            __syncthreads();
        }
    };
    for (int kt = 0; kt < qt; kt++) step(kt, std::false_type{});
    step(qt, std::true_type{});
    const long ld = 3L * C;
#pragma unroll
    for (int d = 0; d < DG; d++) dq[d] *= scale;
    const long o = ((long)b * T + q0) * ld + h * HS + i16;
    write_grad<DG>(dq, dqkv + o, dqkvb ? dqkvb + o : nullptr, ld, q0, T,
                   bsum ? bsum + ((long)b * nqt + qt) * ld + h * HS : nullptr, reinterpret_cast<float*>(Ks), wave, i16,
                   g4);
}

// ---------------------------------------------------------------------------- dk, dv
// One block per (b, h, 64-key tile), each wave 16 keys; query tiles from the diagonal on.
template <int HS>
__global__ __launch_bounds__(NTH, 2) void attn_bwd_dkdv_bf16_kernel(
    float* __restrict__ dqkv, uint16_t* __restrict__ dqkvb, float* __restrict__ bsum,
    const uint16_t* __restrict__ dob, const uint16_t* __restrict__ dot_,
    const uint16_t* __restrict__ qb, const uint16_t* __restrict__ qt_, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const float* __restrict__ lse, const float* __restrict__ delta, int B, int T,
    int C, int NH, int Tp, float scale) {
    constexpr int NKS = (HS + 31) / 32, DG = HS / 16, RS = HS + 8, TS = TILE + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Qs[TILE * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Ds_[TILE * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Qt[HS * TS];
    __shared__ __attribute__((aligned(16))) uint16_t Dt[HS * TS];
    __shared__ float Ls[TILE], Dl[TILE];
    const int nqt = (T + TILE - 1) / TILE;
    const int bh = blockIdx.x % (B * NH);
    const int kt = (int)(blockIdx.x / (B * NH));  // key tile 0 (the most query tiles) first
    const int b = bh / NH, h = bh % NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int k0 = kt * TILE + wave * 16, tk = k0 + i16;
    const int tkc = min(tk, T - 1);
    const uint16_t* Qh = qb + (long)bh * T * HS;
    const uint16_t* QTh = qt_ + (long)bh * HS * Tp;
    const uint16_t* Dh = dob + (long)bh * T * HS;
    const uint16_t* DTh = dot_ + (long)bh * HS * Tp;
    const float* Lh = lse + (long)bh * T;
    const float* Dlh = delta + (long)bh * T;

    bf16x8 kf[NKS], vf[NKS];
    head_frags<HS>(kf, kb + ((long)bh * T + tkc) * HS, tk < T, g4);
    head_frags<HS>(vf, vb + ((long)bh * T + tkc) * HS, tk < T, g4);
    const float scale2 = scale * LOG2E;
    f32x4 dk[DG], dv[DG];
#pragma unroll
    for (int d = 0; d < DG; d++) {
        dk[d] = zero4();
        dv[d] = zero4();
    }
    RowTile<HS> qr, dr;
    TrTile<HS> qtr, dtr;
    float lreg = 0.f, dreg = 0.f;  // thread t < 64: lse and D of query t of the tile
    auto load_tiles = [&](int qtile) __attribute__((always_inline)) {
        const int t0 = qtile * TILE;
        qr.load(Qh, t0, T);
        dr.load(Dh, t0, T);
        qtr.load(QTh, t0, Tp);
        dtr.load(DTh, t0, Tp);
        if (threadIdx.x < TILE) {
            const int q = t0 + threadIdx.x;
            lreg = q < T ? Lh[q] * LOG2E : INFINITY;
            dreg = q < T ? Dlh[q] : 0.f;
        }
    };
    auto store_tiles = [&]() __attribute__((always_inline)) {
        qr.store(Qs);
        dr.store(Ds_);
        qtr.store(Qt);
        dtr.store(Dt);
        if (threadIdx.x < TILE) {
            Ls[threadIdx.x] = lreg;
            Dl[threadIdx.x] = dreg;
        }
    };
    load_tiles(kt);
    store_tiles();
    __syncthreads();
    auto step = [&](int qtile, auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if (qtile + 1 < nqt) load_tiles(qtile + 1);
        // S[query][key] and dP[query][key] for 4 blocks of 16 queries; lane: key tk,
        // queries qtile*64 + q4*16 + 4*g4 + v
        f32x4 s[4], dp[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            s[q4] = zero4();
            dp[q4] = zero4();
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ks++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                s[q4] = mfma(dot_frag<HS>(Qs, q4 * 16 + i16, ks, g4), kf[ks], s[q4]);
                dp[q4] = mfma(dot_frag<HS>(Ds_, q4 * 16 + i16, ks, g4), vf[ks], dp[q4]);
            }
        f32x4 ds[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int qi = q4 * 16 + 4 * g4 + v, query = qtile * TILE + qi;
                const float p = (!DIAG || query >= tk) ? exp2_hw(fmaf(s[q4][v], scale2, -Ls[qi])) : 0.f;
                ds[q4][v] = p * (dp[q4][v] - Dl[qi]);
                s[q4][v] = p;
            }
#pragma unroll
        for (int P = 0; P < 2; P++) {
            float x[8], y[8];
            pair8(x, s[2 * P], s[2 * P + 1]);
            pair8(y, ds[2 * P], ds[2 * P + 1]);
            const Split3 ps = split8(x), ss = split8(y);
#pragma unroll
            for (int d = 0; d < DG; d++) {
                dv[d] = mfma3(ps, ld8(tr_frag_ptr(Dt, d * 16 + i16, P, g4)), dv[d]);
                dk[d] = mfma3(ss, ld8(tr_frag_ptr(Qt, d * 16 + i16, P, g4)), dk[d]);
            }
        }
        if (qtile + 1 < nqt) {
            __syncthreads();
            store_tiles();
            __syncthreads();
        }
    };
    step(kt, std::true_type{});
    for (int qtile = kt + 1; qtile < nqt; qtile++) step(qtile, std::false_type{});
    const long ld = 3L * C;
#pragma unroll
    for (int d = 0; d < DG; d++) dk[d] *= scale;
    const long o = ((long)b * T + k0) * ld + h * HS + i16;
    float* cs = bsum ? bsum + ((long)b * nqt + kt) * ld + h * HS : nullptr;
    float* red = reinterpret_cast<float*>(Qs);
    write_grad<DG>(dk, dqkv + o + C, dqkvb ? dqkvb + o + C : nullptr, ld, k0, T, cs ? cs + C : nullptr, red, wave, i16,
                   g4);
    write_grad<DG>(dv, dqkv + o + 2 * C, dqkvb ? dqkvb + o + 2 * C : nullptr, ld, k0, T, cs ? cs + 2 * C : nullptr, red,
                   wave, i16, g4);
}

template <int HS>
hipError_t fwd_hs(const AttnBf16& a, float* out, uint16_t* outb, float* lse, int B, int T, int C, int NH,
                  hipStream_t st) {
    const int nqt = (T + TILE - 1) / TILE, Tp = nqt * TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    const double flops = 4.0 * B * NH * ((double)T * (T + 1) / 2) * HS;
    ProfScope ps(st, "attn_fwd_bf16_kernel", flops, (double)B * T * C * (3.0 * 2 + 4.0 + (outb ? 2.0 : 0.0)));
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<HS>), dim3(B * NH * nqt), dim3(NTH), 0, st, out, outb, lse, a.q, a.k,
                       a.vt, B, T, C, NH, Tp, scale);
    return hipGetLastError();
}

template <int HS>
hipError_t bwd_hs(const AttnBf16& a, float* dqkv, uint16_t* dqkvb, float* bsum, float* delta, const uint16_t* dob,
                  const uint16_t* dot, const float* out, const float* lse, int B, int T, int C, int NH, hipStream_t st) {
    const int nqt = (T + TILE - 1) / TILE, Tp = nqt * TILE;
    const float scale = 1.0f / sqrtf((float)HS);
    const double tri = B * NH * ((double)T * (T + 1) / 2) * HS;
    {
        ProfScope ps(st, "attn_bwd_dq_bf16_kernel", 6.0 * tri, (double)B * T * C * (2.0 * 5 + 4.0 * 2));
        hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<HS>), dim3(B * NH * nqt), dim3(NTH), 0, st, dqkv, dqkvb, bsum,
                           delta, dob, out, a.q, a.k, a.v, a.kt, lse, B, T, C, NH, Tp, scale);
    }
    {
        ProfScope ps(st, "attn_bwd_dkdv_bf16_kernel", 8.0 * tri, (double)B * T * C * (2.0 * 6 + 4.0 * 2));
        hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<HS>), dim3(B * NH * nqt), dim3(NTH), 0, st, dqkv, dqkvb, bsum,
                           dob, dot, a.q, a.qt, a.k, a.v, lse, delta, B, T, C, NH, Tp, scale);
    }
    return hipGetLastError();
}

bool ok16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

size_t attn_bf16_head_elems(int B, int T, int C) { return (size_t)B * (size_t)((T + TILE - 1) / TILE * TILE) * C; }

hipError_t attn_prep_bf16(const float* src, long ld, long zoff, int nsrc, uint16_t* const* rm, uint16_t* const* tr,
                          int B, int T, int C, int NH, hipStream_t st) {
    const int HS = C / NH;
    if (nsrc < 1 || nsrc > 3 || HS % 16 || HS > 64 || ld % 4 || !ok16(src)) return hipErrorInvalidValue;
    PrepArgs a{};
    a.src = src;
    a.ld = ld;
    a.zoff = zoff;
    for (int z = 0; z < 3; z++) {
        a.rm[z] = z < nsrc ? rm[z] : nullptr;
        a.tr[z] = z < nsrc ? tr[z] : nullptr;
        if ((a.rm[z] && !ok16(a.rm[z])) || (a.tr[z] && !ok16(a.tr[z]))) return hipErrorInvalidValue;
    }
    a.B = B;
    a.T = T;
    a.NH = NH;
    a.HS = HS;
    a.Tp = (T + TILE - 1) / TILE * TILE;
    if (B <= 0 || T <= 0) return hipSuccess;
    ProfScope ps(st, "attn_prep_kernel", 0.0, (double)nsrc * B * T * C * (4.0 + 2.0 + 2.0));
    hipLaunchKernelGGL(attn_prep_kernel, dim3(a.Tp / TILE, B * NH, nsrc), dim3(NTH), 0, st, a);
    return hipGetLastError();
}

hipError_t attention_forward_bf16(float* out, uint16_t* outb, float* lse, const AttnBf16& a, int B, int T, int C,
                                  int NH, hipStream_t st) {
    if (outb && ((uintptr_t)outb & 3)) return hipErrorInvalidValue;
    if (B <= 0 || T <= 0) return hipSuccess;
    switch (C / NH) {
        case 16: return fwd_hs<16>(a, out, outb, lse, B, T, C, NH, st);
        case 32: return fwd_hs<32>(a, out, outb, lse, B, T, C, NH, st);
        case 64: return fwd_hs<64>(a, out, outb, lse, B, T, C, NH, st);
        default: return hipErrorInvalidValue;
    }
}

size_t attn_bias_partial_floats(int B, int T, int C) { return (size_t)B * ((T + TILE - 1) / TILE) * 3 * (size_t)C; }
int attn_bias_partial_rows(int B, int T) { return B * ((T + TILE - 1) / TILE); }

hipError_t attention_backward_bf16(float* dqkv, uint16_t* dqkvb, float* bsum, float* delta, const uint16_t* dob,
                                   const uint16_t* dot, const float* out, const float* lse, const AttnBf16& a, int B,
                                   int T, int C, int NH, hipStream_t st) {
    if (dqkvb && ((uintptr_t)dqkvb & 3)) return hipErrorInvalidValue;
    if (B <= 0 || T <= 0) return hipSuccess;
    switch (C / NH) {
        case 16: return bwd_hs<16>(a, dqkv, dqkvb, bsum, delta, dob, dot, out, lse, B, T, C, NH, st);
        case 32: return bwd_hs<32>(a, dqkv, dqkvb, bsum, delta, dob, dot, out, lse, B, T, C, NH, st);
        case 64: return bwd_hs<64>(a, dqkv, dqkvb, bsum, delta, dob, dot, out, lse, B, T, C, NH, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gpt2k
