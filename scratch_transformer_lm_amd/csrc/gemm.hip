// fp32 GEMMs of the linear layers on gfx950 matrix cores.
//
// Every matmul of the step (the pages' matmul_forward / matmul_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1) is C[M,N] = A[M,K] . B[K,N]
// with one of three operand layouts:
//   forward  Y = X W^T (+ bias ...):  A = X  (k contiguous),  B = W  (k contiguous)
//   dgrad    dX = dY W:               A = dY (k contiguous),  B = W  (n contiguous)
//   wgrad    dW += dY^T X:            A = dY (m contiguous),  B = X  (n contiguous)
//
// Design for CDNA4: 256 threads = 4 wave64s, block tile 128x128, k-tile 32, each wave a
// 64x64 sub-tile made of 2x2 v_mfma_f32_32x32x2f32 blocks (64 accumulators per lane).
// Global tiles are prefetched into registers one k-tile ahead and written to one of two
// LDS buffers, so each k-tile costs one barrier.  LDS keeps the operand's own
// contiguity (k-contiguous rows padded to 36 floats, m/n-contiguous rows padded to
// 136), which keeps both the float4 stores and the fragment reads free of bank
// conflicts.  Inside a group of 8 k values each lane takes 4 consecutive k for its
// half-wave (k = 8g + 4h + s for MFMA step s), so a k-contiguous fragment is one
// 16-byte LDS read; the sum over k is the same sum in another order.
// Blocks are renumbered so that each XCD (blocks are dealt round-robin to the 8 XCDs)
// gets a contiguous range of tiles, grouped 8 tile-rows at a time for L2 reuse.
// Split-K writes per-split partial tiles that a second kernel adds in split order, so
// results never depend on timing.
#include "common.h"
#include "kernels.h"

namespace gpt2k {

namespace {

constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
constexpr int LDK = BK + 4;   // row stride of a k-contiguous LDS tile [row][k]
constexpr int LDR = BM + 8;   // row stride of a row-contiguous LDS tile [k][row]
constexpr int GROUP_M = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Epi { EPI_STORE = 0, EPI_BIAS, EPI_BIAS_RESID, EPI_BIAS_GELU, EPI_ACCUM, EPI_GELU_BWD, EPI_PARTIAL };

struct Params {
    int M, N, K;
    const float* A;
    long lda;
    const float* B;
    long ldb;
    float* C;
    long ldc;
    const float* bias;
    const float* aux;   // residual input (EPI_BIAS_RESID) or pre-GELU values (EPI_GELU_BWD)
    long ldaux;
    float* pre;         // pre-GELU output (EPI_BIAS_GELU)
    long ldpre;
    float* partial;     // split-K partial tiles, [split][M][N]
    int k_split;        // k extent of one split (multiple of BK)
    int tiles_m, tiles_n, splits;
};

// Loads the 128 x 32 slab of an operand whose rows (m or n index) have k contiguous:
// element (r, k) at X[r*ld + k].  Thread t covers rows t/8 + 32j, k = 4*(t%8)..+3.
GPT2_DEV void load_kcontig(float4 (&reg)[4], const float* X, long ld, int r0, int nrows, int k0,
                           int K) {
    const int t = threadIdx.x;
    const int kk = k0 + (t & 7) * 4;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int r = r0 + (t >> 3) + 32 * j;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nrows) {
            const float* p = X + (long)r * ld + kk;
            if (kk + 3 < K) {
                v = *reinterpret_cast<const float4*>(p);
            } else {
                if (kk + 0 < K) v.x = p[0];
                if (kk + 1 < K) v.y = p[1];
                if (kk + 2 < K) v.z = p[2];
            }
        }
        reg[j] = v;
    }
}

GPT2_DEV void store_kcontig(float* S, const float4 (&reg)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; j++)
        *reinterpret_cast<float4*>(S + ((t >> 3) + 32 * j) * LDK + (t & 7) * 4) = reg[j];
}

// Loads the 32 x 128 slab of an operand whose rows are k and whose row index (m or n)
// is contiguous: element (r, k) at X[k*ld + r].  Thread t covers k = t/32 + 8j and
// r = 4*(t%32)..+3.
GPT2_DEV void load_rcontig(float4 (&reg)[4], const float* X, long ld, int r0, int nrows, int k0,
                           int K) {
    const int t = threadIdx.x;
    const int r = r0 + (t & 31) * 4;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int kk = k0 + (t >> 5) + 8 * j;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kk < K) {
            const float* p = X + (long)kk * ld + r;
            if (r + 3 < nrows) {
                v = *reinterpret_cast<const float4*>(p);
            } else {
                if (r + 0 < nrows) v.x = p[0];
                if (r + 1 < nrows) v.y = p[1];
                if (r + 2 < nrows) v.z = p[2];
            }
        }
        reg[j] = v;
    }
}

GPT2_DEV void store_rcontig(float* S, const float4 (&reg)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; j++)
        *reinterpret_cast<float4*>(S + ((t >> 5) + 8 * j) * LDR + (t & 31) * 4) = reg[j];
}

// Fragment for k group g: the 4 values lane (i = lane%32, h = lane/32) feeds to the
// four MFMA steps, rows rb + i, k = 8g + 4h + s.
template <bool KCONTIG>
GPT2_DEV void read_frag(float (&f)[4], const float* S, int rb, int g) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 31, h = lane >> 5;
    if (KCONTIG) {
        float4 v = *reinterpret_cast<const float4*>(S + (rb + i) * LDK + 8 * g + 4 * h);
        f[0] = v.x;
        f[1] = v.y;
        f[2] = v.z;
        f[3] = v.w;
    } else {
#pragma unroll
        for (int s = 0; s < 4; s++) f[s] = S[(8 * g + 4 * h + s) * LDR + rb + i];
    }
}

template <bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(Params p) {
    constexpr int A_STAGE = A_K ? BM * LDK : BK * LDR;
    constexpr int B_STAGE = B_K ? BN * LDK : BK * LDR;
    __shared__ __attribute__((aligned(16))) float smem[2 * (A_STAGE + B_STAGE)];
    float* As = smem;
    float* Bs = smem + 2 * A_STAGE;

    // XCD-aware renumbering, then grouped tile order.
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int q = nb >> 3, r = nb & 7;
    const int lin = xcd * q + min(xcd, r) + local;
    const int per_split = p.tiles_m * p.tiles_n;
    const int split = lin / per_split;
    const int tile = lin - split * per_split;
    const int group_size = GROUP_M * p.tiles_n;
    const int group = tile / group_size;
    const int first_m = group * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int in_group = tile - group * group_size;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int k_begin = split * p.k_split;
    const int k_end = min(p.K, k_begin + p.k_split);
    const int nk = (k_end - k_begin + BK - 1) / BK;

    const int wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[a][b][e] = 0.f;

    float4 ra[4], rb[4];
    auto load = [&](int k0) {
        if (A_K) load_kcontig(ra, p.A, p.lda, m0, p.M, k0, k_end);
        else load_rcontig(ra, p.A, p.lda, m0, p.M, k0, k_end);
        if (B_K) load_kcontig(rb, p.B, p.ldb, n0, p.N, k0, k_end);
        else load_rcontig(rb, p.B, p.ldb, n0, p.N, k0, k_end);
    };
    auto store = [&](int stage) {
        if (A_K) store_kcontig(As + stage * A_STAGE, ra);
        else store_rcontig(As + stage * A_STAGE, ra);
        if (B_K) store_kcontig(Bs + stage * B_STAGE, rb);
        else store_rcontig(Bs + stage * B_STAGE, rb);
    };

    if (nk > 0) {
        load(k_begin);
        store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load(k_begin + (kt + 1) * BK);
        const float* Acur = As + cur * A_STAGE;
        const float* Bcur = Bs + cur * B_STAGE;
#pragma unroll
        for (int g = 0; g < BK / 8; g++) {
            float fa[2][4], fb[2][4];
            read_frag<A_K>(fa[0], Acur, wm, g);
            read_frag<A_K>(fa[1], Acur, wm + 32, g);
            read_frag<B_K>(fb[0], Bcur, wn, g);
            read_frag<B_K>(fb[1], Bcur, wn + 32, g);
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int a = 0; a < 2; a++)
#pragma unroll
                    for (int b = 0; b < 2; b++)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a][s], fb[b][s], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) store(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane holds column lane%32 and, in register
    // v, row 8*(v/4) + 4*(lane/32) + v%4.
    const int lane = threadIdx.x & 63;
    const int col_in = lane & 31, half = lane >> 5;
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) {
            const int col = n0 + wn + 32 * b + col_in;
            if (col >= p.N) continue;
            float bias_v = 0.f;
            if (EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU)
                bias_v = p.bias ? p.bias[col] : 0.f;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int row = m0 + wm + 32 * a + 8 * (v >> 2) + 4 * half + (v & 3);
                if (row >= p.M) continue;
                const float x = acc[a][b][v];
                if (EPI == EPI_STORE) {
                    p.C[(long)row * p.ldc + col] = x;
                } else if (EPI == EPI_BIAS) {
                    p.C[(long)row * p.ldc + col] = x + bias_v;
                } else if (EPI == EPI_BIAS_RESID) {
                    p.C[(long)row * p.ldc + col] = p.aux[(long)row * p.ldaux + col] + (x + bias_v);
                } else if (EPI == EPI_BIAS_GELU) {
                    const float u = x + bias_v;
                    p.pre[(long)row * p.ldpre + col] = u;
                    p.C[(long)row * p.ldc + col] = gelu_f(u);
                } else if (EPI == EPI_ACCUM) {
                    p.C[(long)row * p.ldc + col] += x;
                } else if (EPI == EPI_GELU_BWD) {
                    p.C[(long)row * p.ldc + col] = x * gelu_grad_f(p.aux[(long)row * p.ldaux + col]);
                } else {  // EPI_PARTIAL
                    p.partial[((long)split * p.M + row) * p.N + col] = x;
                }
            }
        }
}

// C (+)= sum over splits of partial[s], splits added in order.  N % 4 == 0.
__global__ void splitk_reduce_kernel(float* C, long ldc, const float* partial, int M, int N,
                                     int splits, int accumulate) {
    const long n4 = (long)M * N / 4;
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
        const long e = i * 4;
        const int row = (int)(e / N), col = (int)(e - (long)row * N);
        float4 s = *reinterpret_cast<const float4*>(partial + e);
        for (int k = 1; k < splits; k++) {
            const float4 t = *reinterpret_cast<const float4*>(partial + (long)k * M * N + e);
            s.x += t.x;
            s.y += t.y;
            s.z += t.z;
            s.w += t.w;
        }
        float4* c = reinterpret_cast<float4*>(C + (long)row * ldc + col);
        if (accumulate) {
            const float4 o = *c;
            s.x += o.x;
            s.y += o.y;
            s.z += o.z;
            s.w += o.w;
        }
        *c = s;
    }
}

template <bool A_K, bool B_K, int EPI>
hipError_t launch(Params& p, hipStream_t st) {
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    if (p.splits < 1) p.splits = 1;
    if (p.splits == 1) {
        p.k_split = p.K;
    } else {
        int ks = (p.K + p.splits - 1) / p.splits;
        p.k_split = (ks + BK - 1) / BK * BK;
        p.splits = (p.K + p.k_split - 1) / p.k_split;
    }
    const long blocks = (long)p.tiles_m * p.tiles_n * p.splits;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<A_K, B_K, EPI>), dim3((unsigned)blocks), dim3(NT), 0, st, p);
    return hipGetLastError();
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

}  // namespace

hipError_t linear_forward(float* out, long ldo, const float* inp, const float* w,
                          const float* bias, const float* resid, float* pre, int M, int N, int K,
                          hipStream_t st) {
    if (K % 4 || !aligned16(inp) || !aligned16(w)) return hipErrorInvalidValue;
    Params p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = inp;
    p.lda = K;
    p.B = w;
    p.ldb = K;
    p.C = out;
    p.ldc = ldo;
    p.bias = bias;
    p.splits = 1;
    if (pre) {
        p.pre = pre;
        p.ldpre = ldo;
        return launch<true, true, EPI_BIAS_GELU>(p, st);
    }
    if (resid) {
        p.aux = resid;
        p.ldaux = ldo;
        return launch<true, true, EPI_BIAS_RESID>(p, st);
    }
    if (bias) return launch<true, true, EPI_BIAS>(p, st);
    return launch<true, true, EPI_STORE>(p, st);
}

hipError_t linear_dgrad(float* din, const float* dout, long ld_dout, const float* w,
                        const float* gelu_pre, int M, int N, int K, int splits, float* partial,
                        hipStream_t st) {
    if (ld_dout % 4 || N % 4 || !aligned16(dout) || !aligned16(w)) return hipErrorInvalidValue;
    Params p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = dout;
    p.lda = ld_dout;
    p.B = w;
    p.ldb = N;
    p.C = din;
    p.ldc = N;
    if (gelu_pre) {
        p.aux = gelu_pre;
        p.ldaux = N;
        p.splits = 1;
        return launch<true, false, EPI_GELU_BWD>(p, st);
    }
    if (splits > 1 && partial) {
        p.partial = partial;
        p.splits = splits;
        hipError_t e = launch<true, false, EPI_PARTIAL>(p, st);
        if (e != hipSuccess) return e;
        const long n4 = (long)M * N / 4;
        const int grid = (int)std::min<long>((n4 + 255) / 256, 4096);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, st, din, (long)N, partial, M, N, p.splits, 0);
        return hipGetLastError();
    }
    p.splits = 1;
    return launch<true, false, EPI_STORE>(p, st);
}

hipError_t linear_wgrad(float* dw, const float* dout, long ld_dout, const float* inp, int M, int N,
                        int K, int splits, float* partial, hipStream_t st) {
    if (ld_dout % 4 || N % 4 || !aligned16(dout) || !aligned16(inp)) return hipErrorInvalidValue;
    Params p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = dout;
    p.lda = ld_dout;
    p.B = inp;
    p.ldb = N;
    p.C = dw;
    p.ldc = N;
    if (splits > 1 && partial) {
        p.partial = partial;
        p.splits = splits;
        hipError_t e = launch<false, false, EPI_PARTIAL>(p, st);
        if (e != hipSuccess) return e;
        const long n4 = (long)M * N / 4;
        const int grid = (int)std::min<long>((n4 + 255) / 256, 4096);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, st, dw, (long)N, partial, M, N, p.splits, 1);
        return hipGetLastError();
    }
    p.splits = 1;
    return launch<false, false, EPI_ACCUM>(p, st);
}

int splitk_effective(int K, int splits) {
    if (splits <= 1) return 1;
    int ks = (K + splits - 1) / splits;
    ks = (ks + BK - 1) / BK * BK;
    return (K + ks - 1) / ks;
}

}  // namespace gpt2k
