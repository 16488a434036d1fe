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
// 64x64 sub-tile made of 4x4 v_mfma_f32_16x16x4f32 blocks (64 accumulators per lane).
// The 16x16x4 form is used because it sustains the full fp32 matrix rate on gfx950,
// where the 32x32x2 form measures about 12% lower.  Global tiles are prefetched into
// registers one k-tile ahead and written to one of two LDS buffers, so each k-tile
// costs one barrier.  LDS keeps the operand's own contiguity: k-contiguous rows are 32
// floats with their 16-byte chunks XOR-swizzled by row, m/n-contiguous rows are padded
// to 132 floats, which keeps both the float4 stores and the fragment reads free of bank
// conflicts.  Inside a group of 16 k values each
// lane takes 4 consecutive k for its lane group (k = 16g + 4(lane/16) + s for MFMA step
// s), so a k-contiguous fragment is one 16-byte LDS read; the sum over k is the same
// sum in another order.
//
// Work distribution is stream-K: with two 74 KB blocks resident per CU the chip holds
// 512 blocks, and the many shapes here with a few hundred 128x128 tiles would leave
// most of a second round idle.  So a persistent grid of up to 512 blocks splits the
// (tile, k-tile) iteration space into equal contiguous ranges.  A block finishes whole
// tiles with the fused epilogue; a tile shared by several blocks is left as partial
// accumulators (in fragment order, fully coalesced) that a fix-up kernel adds in k order
// before running the same epilogue, so the result never depends on timing.  Logical
// block ids are laid out so that each XCD (blocks are dealt round-robin to the 8 XCDs)
// owns a contiguous iteration range, and tiles are ordered 8 tile-rows at a time, which
// keeps neighbouring blocks on the same operand panels in one L2.  Shapes with many
// tiles use the same kernel with one tile per block.
#include <string>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
constexpr int LDK = BK;       // row stride of a k-contiguous LDS tile [row][k] (16-byte chunks XOR-swizzled)
constexpr int LDR = BM + 4;   // row stride of a row-contiguous LDS tile [k][row]
constexpr int GROUP_M = 8;
constexpr int RESIDENT = 512;              // blocks the chip holds at once (2 per CU)
constexpr int SLOT_FLOATS = BM * BN + BM;  // one partial tile + its bias-gradient row sums

typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_STORE = 0, EPI_BIAS, EPI_BIAS_RESID, EPI_BIAS_GELU, EPI_ACCUM, EPI_GELU_BWD };

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
    float* partial;     // 2 partial slots per block
    float* dbias;       // wgrad: db[m] += sum over k of A(m, k), by the tiles with n0 == 0
    const float* lse;   // dlogits operand: per-row log-sum-exp of the logits
    const int32_t* tgt; // dlogits operand: per-row target id
    float xscale;       // dlogits operand: d loss / d loss_row (1 / rows)
    int tiles_m, tiles_n, nk;
    long total;         // tiles * nk iterations
    int G;              // persistent blocks
};

GPT2_DEV long range_start(long total, int G, int lb) { return (long)lb * total / G; }

// Block (logical id) whose iteration range contains iteration x.
GPT2_DEV int owner(long total, int G, long x) {
    int lb = (int)(x * G / total);
    while (lb + 1 < G && range_start(total, G, lb + 1) <= x) lb++;
    while (lb > 0 && range_start(total, G, lb) > x) lb--;
    return lb;
}

GPT2_DEV void tile_coords(const Params& p, int tile, int& m0, int& n0) {
    const int group_size = GROUP_M * p.tiles_n;
    const int group = tile / group_size;
    const int first_m = group * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int in_group = tile - group * group_size;
    m0 = (first_m + in_group % gm) * BM;
    n0 = (in_group / gm) * BN;
}

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
            const float* q = X + (long)r * ld + kk;
            if (kk + 3 < K) {
                v = *reinterpret_cast<const float4*>(q);
            } else {
                if (kk + 0 < K) v.x = q[0];
                if (kk + 1 < K) v.y = q[1];
                if (kk + 2 < K) v.z = q[2];
            }
        }
        reg[j] = v;
    }
}

GPT2_DEV void store_kcontig(float* S, const float4 (&reg)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; j++)
    {
        const int row = (t >> 3) + 32 * j;
        *reinterpret_cast<float4*>(S + row * LDK + (((t & 7) ^ ((row >> 1) & 7)) * 4)) = reg[j];
    }
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
            const float* q = X + (long)kk * ld + r;
            if (r + 3 < nrows) {
                v = *reinterpret_cast<const float4*>(q);
            } else {
                if (r + 0 < nrows) v.x = q[0];
                if (r + 1 < nrows) v.y = q[1];
                if (r + 2 < nrows) v.z = q[2];
            }
        }
        reg[j] = v;
    }
}

// The logits operand of the LM-head backward: each logit z of row `row` in vocabulary
// column c becomes d loss / d z = (exp(z - lse[row]) - [c == target[row]]) * scale.
// Applied to the prefetched registers just before they go to LDS (so the global loads
// keep their full k-tile of latency hiding); out-of-range elements stay zero.
GPT2_DEV float dlogit(float z, float lse, int tgt, int c, float scale) {
    return (__expf(z - lse) - (c == tgt ? 1.0f : 0.0f)) * scale;
}

// k-contiguous slab (LM-head dgrad): row r = r0 + t/8 + 32j is a logits row; its lse and
// target are `rl[j]`, `rt[j]`; columns kk.. are vocabulary ids.
GPT2_DEV void dlogit_kcontig(float4 (&reg)[4], const float (&rl)[4], const int (&rt)[4], int r0, int nrows,
                             int k0, int K, float scale) {
    const int t = threadIdx.x;
    const int kk = k0 + (t & 7) * 4;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (r0 + (t >> 3) + 32 * j >= nrows) continue;
        float4& v = reg[j];
        if (kk + 0 < K) v.x = dlogit(v.x, rl[j], rt[j], kk + 0, scale);
        if (kk + 1 < K) v.y = dlogit(v.y, rl[j], rt[j], kk + 1, scale);
        if (kk + 2 < K) v.z = dlogit(v.z, rl[j], rt[j], kk + 2, scale);
        if (kk + 3 < K) v.w = dlogit(v.w, rl[j], rt[j], kk + 3, scale);
    }
}

// row-contiguous slab (LM-head wgrad): k = k0 + t/32 + 8j is a logits row (lse rl[j],
// target rt[j]); the row index r.. is the vocabulary id.
GPT2_DEV void dlogit_rcontig(float4 (&reg)[4], const float (&rl)[4], const int (&rt)[4], int r0, int nrows,
                             int k0, int K, float scale) {
    const int t = threadIdx.x;
    const int r = r0 + (t & 31) * 4;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (k0 + (t >> 5) + 8 * j >= K) continue;
        float4& v = reg[j];
        if (r + 0 < nrows) v.x = dlogit(v.x, rl[j], rt[j], r + 0, scale);
        if (r + 1 < nrows) v.y = dlogit(v.y, rl[j], rt[j], r + 1, scale);
        if (r + 2 < nrows) v.z = dlogit(v.z, rl[j], rt[j], r + 2, scale);
        if (r + 3 < nrows) v.w = dlogit(v.w, rl[j], rt[j], r + 3, scale);
    }
}

GPT2_DEV void store_rcontig(float* S, const float4 (&reg)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; j++)
        *reinterpret_cast<float4*>(S + ((t >> 5) + 8 * j) * LDR + (t & 31) * 4) = reg[j];
}

// Fragment for k group g: the 4 values lane (i = lane%16, grp = lane/16) feeds to the
// four MFMA steps, rows rb + i, k = 16g + 4grp + s.
template <bool KCONTIG>
GPT2_DEV void read_frag(float (&f)[4], const float* S, int rb, int g) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, grp = lane >> 4;
    if (KCONTIG) {
        const int row = rb + i;
        float4 v = *reinterpret_cast<const float4*>(S + row * LDK + (((4 * g + grp) ^ ((row >> 1) & 7)) * 4));
        f[0] = v.x;
        f[1] = v.y;
        f[2] = v.z;
        f[3] = v.w;
    } else {
#pragma unroll
        for (int s = 0; s < 4; s++) f[s] = S[(16 * g + 4 * grp + s) * LDR + rb + i];
    }
}

// Fused epilogue on one finished 16x16 block (a, b) of this thread's wave.  16x16
// accumulator layout: lane holds column lane%16 and, in register v, row 4*(lane/16) + v.
template <int EPI>
GPT2_DEV void epilogue_block(const Params& p, const f32x4& acc, int m0, int n0, int a, int b) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int col = n0 + wn + 16 * b + (lane & 15), grp = lane >> 4;
    if (col >= p.N) return;
    float bias_v = 0.f;
    if (EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU) bias_v = p.bias ? p.bias[col] : 0.f;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int row = m0 + wm + 16 * a + 4 * grp + v;
        if (row >= p.M) continue;
        const float x = acc[v];
        float* c = p.C + (long)row * p.ldc + col;
        if (EPI == EPI_STORE) {
            *c = x;
        } else if (EPI == EPI_BIAS) {
            *c = x + bias_v;
        } else if (EPI == EPI_BIAS_RESID) {
            *c = p.aux[(long)row * p.ldaux + col] + (x + bias_v);
        } else if (EPI == EPI_BIAS_GELU) {
            const float u = x + bias_v;
            p.pre[(long)row * p.ldpre + col] = u;
            *c = gelu_f(u);
        } else if (EPI == EPI_ACCUM) {
            *c += x;
        } else {  // EPI_GELU_BWD
            *c = x * gelu_grad_f(p.aux[(long)row * p.ldaux + col]);
        }
    }
}

template <int EPI>
GPT2_DEV void epilogue(const Params& p, const f32x4 (&acc)[4][4], int m0, int n0) {
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) epilogue_block<EPI>(p, acc[a][b], m0, n0, a, b);
}

// Partial tile in fragment order: thread t's 64 accumulators at slot[(j*256 + t)],
// j = (a*4 + b)*4 + v.
GPT2_DEV void store_partial(float* slot, const f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) slot[((a * 4 + b) * 4 + v) * NT + threadIdx.x] = acc[a][b][v];
}


template <bool A_K, bool B_K, int EPI, bool XF>
__global__ __launch_bounds__(NT) void gemm_kernel(Params p) {
    constexpr int A_STAGE = A_K ? BM * LDK : BK * LDR;
    constexpr int B_STAGE = B_K ? BN * LDK : BK * LDR;
    __shared__ __attribute__((aligned(16))) float smem[2 * (A_STAGE + B_STAGE)];
    float* As = smem;
    float* Bs = smem + 2 * A_STAGE;

    // XCD-aware logical block id: XCD x (= blockIdx % 8) gets a contiguous id range.
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int lb = xcd * (nb >> 3) + min(xcd, nb & 7) + local;
    const long it_begin = range_start(p.total, p.G, lb);
    const long it_end = range_start(p.total, p.G, lb + 1);

    const int wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    float4 ra[4], rb[4];

    for (long it = it_begin; it < it_end;) {
        const int tile = (int)(it / p.nk);
        const int ks = (int)(it - (long)tile * p.nk);
        const int ke = (int)min((long)p.nk, ks + (it_end - it));
        int m0, n0;
        tile_coords(p, tile, m0, n0);
        const int k_end = min(p.K, ke * BK);

        f32x4 acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b < 4; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        // wgrad with bias: row sums of A over this segment's k, 4 rows per thread
        const bool bias_rows = !A_K && p.dbias != nullptr && n0 == 0;
        float bsum[4] = {0.f, 0.f, 0.f, 0.f};

        // dlogits operand: lse / target of the logits rows this thread's A slab covers
        float xl[4];
        int xt[4];
        int ra_k0 = 0;
        if (XF && A_K) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int r = m0 + (threadIdx.x >> 3) + 32 * j;
                xl[j] = r < p.M ? p.lse[r] : 0.f;
                xt[j] = r < p.M ? p.tgt[r] : -1;
            }
        }

        auto load = [&](int k0) {
            if (A_K) load_kcontig(ra, p.A, p.lda, m0, p.M, k0, k_end);
            else load_rcontig(ra, p.A, p.lda, m0, p.M, k0, k_end);
            if (B_K) load_kcontig(rb, p.B, p.ldb, n0, p.N, k0, k_end);
            else load_rcontig(rb, p.B, p.ldb, n0, p.N, k0, k_end);
            if (XF && !A_K) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int kk = k0 + (threadIdx.x >> 5) + 8 * j;
                    xl[j] = kk < k_end ? p.lse[kk] : 0.f;
                    xt[j] = kk < k_end ? p.tgt[kk] : -1;
                }
            }
            ra_k0 = k0;
        };
        auto store = [&](int stage) {
            if (XF) {
                if (A_K) dlogit_kcontig(ra, xl, xt, m0, p.M, ra_k0, k_end, p.xscale);
                else dlogit_rcontig(ra, xl, xt, m0, p.M, ra_k0, k_end, p.xscale);
            }
            if (!A_K && bias_rows) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    bsum[0] += ra[j].x;
                    bsum[1] += ra[j].y;
                    bsum[2] += ra[j].z;
                    bsum[3] += ra[j].w;
                }
            }
            if (A_K) store_kcontig(As + stage * A_STAGE, ra);
            else store_rcontig(As + stage * A_STAGE, ra);
            if (B_K) store_kcontig(Bs + stage * B_STAGE, rb);
            else store_rcontig(Bs + stage * B_STAGE, rb);
        };

        load(ks * BK);
        store(0);
        __syncthreads();
        const int n = ke - ks;
        for (int kt = 0; kt < n; kt++) {
            const int cur = kt & 1;
            if (kt + 1 < n) load((ks + kt + 1) * BK);
            const float* Acur = As + cur * A_STAGE;
            const float* Bcur = Bs + cur * B_STAGE;
            // both 16-k groups' fragments are read before the first MFMA
            float fa[BK / 16][4][4], fb[BK / 16][4][4];
#pragma unroll
            for (int g = 0; g < BK / 16; g++) {
#pragma unroll
                for (int a = 0; a < 4; a++) read_frag<A_K>(fa[g][a], Acur, wm + 16 * a, g);
#pragma unroll
                for (int b = 0; b < 4; b++) read_frag<B_K>(fb[g][b], Bcur, wn + 16 * b, g);
            }
#pragma unroll
            for (int g = 0; g < BK / 16; g++)
#pragma unroll
                for (int s = 0; s < 4; s++)
#pragma unroll
                    for (int a = 0; a < 4; a++)
#pragma unroll
                        for (int b = 0; b < 4; b++)
                            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[g][a][s], fb[g][b][s], acc[a][b], 0, 0, 0);
            if (kt + 1 < n) store(cur ^ 1);
            __syncthreads();
        }

        const bool full = ks == 0 && ke == p.nk;
        // first segment of the range -> slot 0, the range's last (shared) tile -> slot 1
        float* slot = p.partial + ((long)lb * 2 + (it == it_begin ? 0 : 1)) * SLOT_FLOATS;
        if (bias_rows) {
            // combine the 8 threads that share rows (t%32), in k-group order; the LDS
            // operand buffers are free after the loop's final barrier
            float* red = As;
#pragma unroll
            for (int e = 0; e < 4; e++) red[threadIdx.x * 4 + e] = bsum[e];
            __syncthreads();
            if (threadIdx.x < 32) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    float s = 0.f;
                    for (int g8 = 0; g8 < 8; g8++) s += red[(g8 * 32 + threadIdx.x) * 4 + e];
                    const int m = m0 + 4 * threadIdx.x + e;
                    if (full) {
                        if (m < p.M) p.dbias[m] += s;
                    } else {
                        slot[BM * BN + 4 * threadIdx.x + e] = s;
                    }
                }
            }
            __syncthreads();
        }
        if (full) {
            epilogue<EPI>(p, acc, m0, n0);
        } else {
            store_partial(slot, acc);
        }
        it += ke - ks;
    }
}

// Four blocks per range boundary that falls strictly inside a tile, one per row of
// 16x16 blocks (a) of the waves' sub-tiles; for the lowest such boundary of a tile they
// add that tile's partials in k order and run the epilogue.
template <int EPI>
__global__ __launch_bounds__(NT) void gemm_fixup_kernel(Params p) {
    const int quarter = blockIdx.x & 3;
    const int lbb = (blockIdx.x >> 2) + 1;  // boundary between blocks lbb-1 and lbb
    const long x = range_start(p.total, p.G, lbb);
    if (x % p.nk == 0) return;
    const int tile = (int)(x / p.nk);
    if (lbb >= 2) {
        const long xp = range_start(p.total, p.G, lbb - 1);
        if (xp / p.nk == tile && xp % p.nk != 0) return;
    }
    const long t0 = (long)tile * p.nk;
    const int first = owner(p.total, p.G, t0);
    const int last = owner(p.total, p.G, t0 + p.nk - 1);
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; b++) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int l = first; l <= last; l++) {
        const int which = range_start(p.total, p.G, l) / p.nk == tile ? 0 : 1;
        const float* slot = p.partial + ((long)l * 2 + which) * SLOT_FLOATS + quarter * 16 * NT + threadIdx.x;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; e++) v[e] = slot[e * NT];
#pragma unroll
        for (int e = 0; e < 16; e++) acc[e >> 2][e & 3] += v[e];
    }
    int m0, n0;
    tile_coords(p, tile, m0, n0);
#pragma unroll
    for (int b = 0; b < 4; b++) epilogue_block<EPI>(p, acc[b], m0, n0, quarter, b);
    if (p.dbias && n0 == 0 && quarter == 0 && threadIdx.x < BM && m0 + (int)threadIdx.x < p.M) {
        float s = 0.f;
        for (int l = first; l <= last; l++) {
            const int which = range_start(p.total, p.G, l) / p.nk == tile ? 0 : 1;
            s += p.partial[((long)l * 2 + which) * SLOT_FLOATS + BM * BN + threadIdx.x];
        }
        p.dbias[m0 + threadIdx.x] += s;
    }
}

// Kernel name as profilers print the instantiation.
template <bool A_K, bool B_K, int EPI, bool XF>
const char* gemm_name() {
    static const std::string s = std::string("gemm_kernel<") + (A_K ? "true" : "false") + ", " +
                                 (B_K ? "true" : "false") + ", " + std::to_string(EPI) + ", " +
                                 (XF ? "true" : "false") + ">";
    return s.c_str();
}

template <int EPI>
const char* fixup_name() {
    static const std::string s = "gemm_fixup_kernel<" + std::to_string(EPI) + ">";
    return s.c_str();
}

template <bool A_K, bool B_K, int EPI, bool XF = false>
hipError_t launch(Params& p, hipStream_t st) {
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.nk = (p.K + BK - 1) / BK;
    const long tiles = (long)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    if (p.nk == 0) {
        // empty reduction: every output is the epilogue of 0
        p.nk = 1;
    }
    p.total = tiles * p.nk;
    // Many tiles: one tile per block.  Otherwise stream-K over the resident blocks.
    const bool sk = tiles < 8L * RESIDENT && p.partial != nullptr;
    p.G = sk ? (int)std::min<long>(RESIDENT, p.total) : (int)tiles;
    const double mn = (double)p.M * p.N;
    const double extra = (EPI == EPI_BIAS_RESID || EPI == EPI_ACCUM || EPI == EPI_GELU_BWD || EPI == EPI_BIAS_GELU) ? mn : 0.0;
    {
        // algorithmic work: 2MNK flops; operands read once, C written (and read for += / aux)
        ProfScope ps(st, gemm_name<A_K, B_K, EPI, XF>(), 2.0 * mn * p.K,
                     4.0 * ((double)p.M * p.K + (double)p.N * p.K + mn + extra));
        hipLaunchKernelGGL((gemm_kernel<A_K, B_K, EPI, XF>), dim3(p.G), dim3(NT), 0, st, p);
    }
    const bool aligned_ranges = p.total % p.G == 0 && (p.total / p.G) % p.nk == 0;
    if (sk && !aligned_ranges && p.G > 1) {
        ProfScope ps(st, fixup_name<EPI>(), 0.0, 4.0 * (2.0 * p.G * SLOT_FLOATS + extra));
        hipLaunchKernelGGL((gemm_fixup_kernel<EPI>), dim3(4 * (p.G - 1)), dim3(NT), 0, st, p);
    }
    return hipGetLastError();
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

}  // namespace

size_t gemm_partial_floats() { return (size_t)RESIDENT * 2 * SLOT_FLOATS; }

hipError_t linear_forward(float* out, long ldo, const float* inp, const float* w,
                          const float* bias, const float* resid, float* pre, int M, int N, int K,
                          float* partial, hipStream_t st) {
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
    p.partial = partial;
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
                        const float* gelu_pre, int M, int N, int K, float* partial, hipStream_t st,
                        const XentOperand* xent) {
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
    p.partial = partial;
    if (gelu_pre) {
        p.aux = gelu_pre;
        p.ldaux = N;
        return launch<true, false, EPI_GELU_BWD>(p, st);
    }
    if (xent) {
        p.lse = xent->lse;
        p.tgt = xent->targets;
        p.xscale = xent->scale;
        return launch<true, false, EPI_STORE, true>(p, st);
    }
    return launch<true, false, EPI_STORE>(p, st);
}

hipError_t linear_wgrad(float* dw, float* dbias, const float* dout, long ld_dout, const float* inp, int M,
                        int N, int K, float* partial, hipStream_t st, const XentOperand* xent) {
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
    p.partial = partial;
    p.dbias = dbias;
    if (xent) {
        p.lse = xent->lse;
        p.tgt = xent->targets;
        p.xscale = xent->scale;
        return launch<false, false, EPI_ACCUM, true>(p, st);
    }
    return launch<false, false, EPI_ACCUM>(p, st);
}

}  // namespace gpt2k
