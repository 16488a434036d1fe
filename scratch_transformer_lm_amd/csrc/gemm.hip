// fp32 GEMMs of the linear layers on gfx950 matrix cores.
//
// Every matmul of the step (the pages' matmul_forward / matmul_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1) is C[M,N] = A[M,K] . B[K,N]
// with one of three operand layouts:
//   forward  Y = X W^T (+ bias ...):  A = X  (k contiguous),  B = W  (k contiguous)
//   dgrad    dX = dY W:               A = dY (k contiguous),  B = W  (n contiguous)
//   wgrad    dW += dY^T X:            A = dY (m contiguous),  B = X  (n contiguous)
// (the bfloat16 variant multiplies bf16 copies: forward and dgrad with both operands
// k-contiguous, W transposed for the dgrad; wgrad as above, see gemm_body)
//
// Design for CDNA4: 256 threads = 4 wave64s, block tile 128x128 (or 128x96 where that
// count of tiles fills whole rounds of the grid and 128x128 does not), each wave a
// 64x64 (64x48) sub-tile made of 4x4 (4x3) v_mfma_f32_16x16x4f32 blocks.  The
// 16x16x4 form is used because it sustains the full fp32 matrix rate on gfx950, where
// the 32x32x2 form measures about 12% lower.  Operand k-tiles go from global memory
// straight into LDS (global_load_lds_dwordx4, no register staging) through a ring of LDS
// buffers: 32-wide k-tiles in 2 buffers when A is k-contiguous, 16-wide k-tiles in 4
// buffers (3 in flight while one is consumed) for the wgrad; each k-tile costs one
// barrier.  LDS tiles are unpadded (a wave's transfer is 1 KB of consecutive LDS) and bank
// conflicts are avoided by swizzling 16-byte chunks (layouts at rpos below).  Each lane takes 4
// consecutive k for its lane group (k = 16g + 4(lane/16) + s for MFMA step s), so a
// k-contiguous fragment is one 16-byte LDS read; the sum over k is the same sum in
// another order.
//
// Work distribution: a persistent grid of up to 512 blocks (two 64 KB blocks per CU).
// Shapes with at least 512 tiles are first run in whole-tile rounds, block lb taking tile
// r*512 + lb in round r, so that the 64 blocks of an XCD work on 64 neighbouring tiles at
// the same k and share operand panels in that XCD's L2.  The remaining tiles (all tiles of
// the many shapes here with only a few hundred) are split stream-K style: their
// (tile, k-tile) iteration space is cut into equal contiguous ranges, one per block.  A
// block finishes whole tiles with the fused epilogue; a tile shared by several blocks is
// left as partial accumulators (in fragment order, fully coalesced) that a fix-up kernel
// adds in k order before running the same epilogue, so the result never depends on
// timing.  Logical block ids are laid out so that each XCD (blocks are dealt round-robin
// to the 8 XCDs) owns a contiguous id range, and tiles are ordered 8 tile-rows at a time.
#include <algorithm>
#include <cmath>
#include <string>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

// Block tile BM x BN, BN = 128 or (A k-contiguous only) 96, a template parameter; wave w
// holds the 64 x BN/2 sub-tile at (64 (w/2), BN/2 (w%2)) as 4 x NB blocks of 16x16,
// NB = BN/32.
constexpr int BM = 128, NT = 256;
// k-tile width and LDS ring depth (k-tiles in flight + 1) per operand layout: 32 and 2
// when A is k-contiguous (forward, dgrad), 16 and 4 for the wgrad, whose row-contiguous
// fragments and fused bias sums need more registers than a second wave per SIMD leaves
// with 32-wide k-tiles.  Both rings take 64 KB.
// Waves raise their issue priority for the k loop and drop it for the epilogue (build
// option).
#ifndef GEMM_SETPRIO
#define GEMM_SETPRIO 0
#endif
#ifndef GEMM_WG_BK
#define GEMM_WG_BK 16
#endif
#ifndef GEMM_WG_STAGES
#define GEMM_WG_STAGES 4
#endif
template <bool A_K>
struct KTile {
    static constexpr int BK = A_K ? 32 : GEMM_WG_BK;
    static constexpr int STAGES = A_K ? 2 : GEMM_WG_STAGES;
};
// bf16 operands (k-tile width in float pairs): a k-tile takes an eighth of the fp32 MFMA
// time, so more of them must be in flight to cover the global -> LDS latency.
#ifndef GEMM_BF_BK
#define GEMM_BF_BK 32
#endif
#ifndef GEMM_BF_STAGES
#define GEMM_BF_STAGES 2
#endif
// 256-wide bf16 tiles (64 x 128 per wave) take half-width k-tiles in 3 buffers, so that
// two blocks still fit a CU.
#ifndef GEMM_BF256_BK
#define GEMM_BF256_BK 16
#endif
#ifndef GEMM_BF256_STAGES
#define GEMM_BF256_STAGES 3
#endif
template <bool A_K, bool BF, int BN = 128>
struct KTileOf : KTile<A_K> {};
template <int BN>
struct KTileOf<true, true, BN> {
    static constexpr int BK = BN == 256 ? GEMM_BF256_BK : GEMM_BF_BK;
    static constexpr int STAGES = BN == 256 ? GEMM_BF256_STAGES : GEMM_BF_STAGES;
};
// bf16 operands stored row-contiguous, [k][rows] (the weight gradient's dY and X as the
// forward and backward write them): k-tiles of GEMM_BFT_BK k rows, a 128-row tile row
// being 256 bytes, so a k-tile takes as much LDS as the k-contiguous bf16 one.
#ifndef GEMM_BFT_BK
#define GEMM_BFT_BK 64
#endif
#ifndef GEMM_BFT_STAGES
#define GEMM_BFT_STAGES 2
#endif
template <int BN>
struct KTileOf<false, true, BN> {
    static constexpr int BK = GEMM_BFT_BK;
    static constexpr int STAGES = GEMM_BFT_STAGES;
};
constexpr int XF_FLOATS = 4 * 64;                // dlogits wgrad: per-wave lse slots
#ifndef GEMM_GROUP_M
#define GEMM_GROUP_M 8
#endif
constexpr int GROUP_M = GEMM_GROUP_M;  // tile rows per group of the tile order
constexpr int RESIDENT = 512;                    // blocks the chip holds at once (2 per CU)
constexpr int MAX_UNITS = 1536;                  // split-K units the partial region holds
// partial slot of a BM x BN tile: the tile (at least BM x 128), then its bias-gradient row sums
template <int BN>
constexpr int slot_bias() { return BM * (BN > 128 ? BN : 128); }
template <int BN>
constexpr int slot_floats() { return slot_bias<BN>() + BM; }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr float LOG2E_EPI = 1.4426950408889634f;

// EPI_DLOGITS: LM-head dgrad whose A held s * softmax only; the one-hot part of dlogits,
// s * onehot(target) . W = s * W[target], is subtracted here.
// EPI_STORE_LSE: the LM-head forward; stores the logits and, per row, the base-2
// (max, sum of 2^(x log2 e - max)) of each wave's half of the tile's columns.
enum Epi { EPI_STORE = 0, EPI_BIAS, EPI_BIAS_RESID, EPI_BIAS_GELU, EPI_ACCUM, EPI_GELU_BWD, EPI_DLOGITS, EPI_STORE_LSE };

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
    float* partial;     // partial-tile slots
    float* dbias;       // wgrad: db[m] += sum over k of A(m, k), by the tiles with n0 == 0
    const float* lse;   // dlogits operand: per-row log-sum-exp of the logits
    const int32_t* tgt; // dlogits operand: per-row target id
    float xscale;       // dlogits operand: d loss / d loss_row (1 / rows)
    float xlog2s;       // log2(xscale)
    float* lsep;        // EPI_STORE_LSE: partial (max, sum) pairs, [2 * tiles_n][M] float2
    uint16_t* cb;       // EPI_BIAS_GELU, EPI_GELU_BWD: bf16 rounding of C (nullable)
    long ldcb;
    float* csum;        // EPI_GELU_BWD: column sums of C per 16-row slice, [M/16][N] (nullable)
    int tiles_m, tiles_n, nk;
    int G;              // persistent blocks
    int R;              // whole-tile rounds: block lb takes tiles r*G + lb, r < R
    int tile0;          // first tile of the split region (R * G)
    int skt;            // tiles in the split region
    long total;         // skt * nk iterations of the split region
    int nr;             // ranges the split region is cut into (<= G), range lb for block lb
    int S;              // > 1: split-K rounds instead (units = tiles * S, see schedule)
    int units;
};

GPT2_DEV long range_start(long total, int G, int lb) { return (long)lb * total / G; }

// Block (logical id) whose iteration range contains iteration x.
GPT2_DEV int owner(long total, int G, long x) {
    int lb = (int)(x * G / total);
    while (lb + 1 < G && range_start(total, G, lb + 1) <= x) lb++;
    while (lb > 0 && range_start(total, G, lb) > x) lb--;
    return lb;
}

template <int BN>
GPT2_DEV void tile_coords(const Params& p, int tile, int& m0, int& n0) {
    const int group_size = GROUP_M * p.tiles_n;
    const int group = tile / group_size;
    const int first_m = group * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int in_group = tile - group * group_size;
    m0 = (first_m + in_group % gm) * BM;
    n0 = (in_group / gm) * BN;
}

// Fused epilogue, one row of this wave's 16x16 blocks (a, b = 0..NB-1) at a time.
// 16x16 accumulator layout: lane holds column lane%16 and, in register v, row
// 4*(lane/16) + v.  epi_load requests the values the row's epilogue reads (residual,
// pre-activation, old C, target rows of W); epi_store forms the outputs and stores them
// back to back.  CHECK: the tile crosses the edge of C, so rows and columns are
// bounds-checked.
template <int EPI>
constexpr bool epi_reads() {
    return EPI == EPI_BIAS_RESID || EPI == EPI_ACCUM || EPI == EPI_GELU_BWD || EPI == EPI_DLOGITS;
}

template <int EPI, bool CHECK, int NB>
GPT2_DEV void epi_load(const Params& p, int m0, int n0, int a, float (&in)[NB][4]) {
    if (!epi_reads<EPI>()) return;
    constexpr int WN = 16 * NB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = m0 + (wave >> 1) * 64 + 16 * a + 4 * (lane >> 4), c0 = n0 + (wave & 1) * WN + (lane & 15);
    const float* src = EPI == EPI_ACCUM ? p.C : p.aux;
    const long lds = EPI == EPI_ACCUM ? p.ldc : p.ldaux;
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int row = r0 + v;
        const float* q = src + (long)row * lds + c0;
        // EPI_DLOGITS reads row target[row] of W (B, k = vocabulary id) instead
        if (EPI == EPI_DLOGITS) q = p.B + (long)(!CHECK || row < p.M ? p.tgt[row] : 0) * p.ldb + c0;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            in[b][v] = 0.f;
            if (!CHECK || (row < p.M && c0 + 16 * b < p.N)) in[b][v] = q[16 * b];
        }
    }
}

template <int EPI, bool CHECK, int NB>
GPT2_DEV void epi_store(const Params& p, const f32x4 (&acc)[NB], int m0, int n0, int a, float (&in)[NB][4]) {
    constexpr int WN = 16 * NB;
    constexpr bool HAS_BIAS = EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = m0 + (wave >> 1) * 64 + 16 * a + 4 * (lane >> 4), c0 = n0 + (wave & 1) * WN + (lane & 15);
    auto inside = [&](int b, int v) { return !CHECK || (r0 + v < p.M && c0 + 16 * b < p.N); };
    float bias_v[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) {
        bias_v[b] = 0.f;
        if (HAS_BIAS && p.bias && (!CHECK || c0 + 16 * b < p.N)) bias_v[b] = p.bias[c0 + 16 * b];
    }
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float x = acc[b][v];
            float& o = in[b][v];
            if (EPI == EPI_STORE || EPI == EPI_STORE_LSE) o = x;
            else if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) o = x + bias_v[b];
            else if (EPI == EPI_BIAS_RESID) o = o + (x + bias_v[b]);
            else if (EPI == EPI_ACCUM) o = o + x;
            else if (EPI == EPI_DLOGITS) o = x - p.xscale * o;
            else o = x * gelu_grad_f(o);  // EPI_GELU_BWD
        }
    auto store_row = [&](float* dst, long ld) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float* q = dst + (long)(r0 + v) * ld + c0;
#pragma unroll
            for (int b = 0; b < NB; b++)
                if (inside(b, v)) q[16 * b] = in[b][v];
        }
    };
    if constexpr (EPI == EPI_STORE_LSE) {
        // this wave's 16*NB columns of each of its 4 rows: 16 lanes x NB values
        const int part = (n0 / (32 * NB)) * 2 + (wave & 1);
        float pm = -INFINITY, ps = 0.f;  // lanes 0..3 of each group keep row r0 + (lane & 15)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float m = -INFINITY;
#pragma unroll
            for (int b = 0; b < NB; b++)
                if (inside(b, v)) m = fmaxf(m, in[b][v] * LOG2E_EPI);
            m = row16_max(m);
            float sum = 0.f;
            if (m > -INFINITY) {
#pragma unroll
                for (int b = 0; b < NB; b++)
                    if (inside(b, v)) sum += __builtin_amdgcn_exp2f(fmaf(in[b][v], LOG2E_EPI, -m));
            }
            sum = row16_sum(sum);
            if ((lane & 15) == v) {
                pm = m;
                ps = sum;
            }
        }
        // one store of 16 consecutive rows (lanes 0..3 of the four groups)
        const int row = r0 + (lane & 15);
        if ((lane & 15) < 4 && row < p.M) reinterpret_cast<float2*>(p.lsep)[(long)part * p.M + row] = make_float2(pm, ps);
    }
    if (EPI == EPI_BIAS_GELU) {
        store_row(p.pre, p.ldpre);  // the pre-activation, then its GELU
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) in[b][v] = gelu_f(in[b][v]);
    }
    store_row(p.C, p.ldc);
    if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_GELU_BWD) {
        // the bf16 copy the next GEMM multiplies (and the weight gradient reads)
        if (p.cb) {
#pragma unroll
            for (int b = 0; b < NB; b++)
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    uint16_t* q = p.cb + (long)(r0 + v) * p.ldcb + c0 + 16 * b;
                    bf16_store_rows2(q, q + p.ldcb, in[b][v], in[b][v + 1], inside(b, v), inside(b, v + 1));
                }
        }
    }
    if constexpr (EPI == EPI_GELU_BWD) {
        // the bias gradient of the layer whose output gradient C is: this row slice's 16
        // rows added per column (v, then the four lane groups), one partial row per slice
        if (p.csum) {
            const int slice = (m0 + (wave >> 1) * 64 + 16 * a) >> 4;
#pragma unroll
            for (int b = 0; b < NB; b++) {
                float t = 0.f;
#pragma unroll
                for (int v = 0; v < 4; v++)
                    if (inside(b, v)) t += in[b][v];
                t = rows4_sum(t);
                if ((lane >> 4) == 0 && 16 * slice < p.M && (!CHECK || c0 + 16 * b < p.N))
                    p.csum[(long)slice * p.N + c0 + 16 * b] = t;
            }
        }
    }
}

// NA rows (a0 ..) of blocks: the next row's inputs are requested before this row's
// outputs are stored, so the memory operations overlap.  `pre` runs once the first row's
// inputs are requested (the fix-up sums its partials there).
template <int EPI, int NA, bool CHECK, int NB, class Pre>
GPT2_DEV void epilogue_rows_(const Params& p, const f32x4 (&acc)[NA][NB], int m0, int n0, int a0, Pre&& pre) {
    float in0[NB][4], in1[NB][4];
    epi_load<EPI, CHECK>(p, m0, n0, a0, in0);
    pre();
#pragma unroll
    for (int i = 0; i < NA; i++) {
        if (i + 1 < NA) epi_load<EPI, CHECK>(p, m0, n0, a0 + i + 1, (i & 1) ? in0 : in1);
        epi_store<EPI, CHECK>(p, acc[i], m0, n0, a0 + i, (i & 1) ? in1 : in0);
    }
}

template <int EPI, int NA, int NB, class Pre>
GPT2_DEV void epilogue_rows(const Params& p, const f32x4 (&acc)[NA][NB], int m0, int n0, int a0, Pre&& pre) {
    if (m0 + BM <= p.M && n0 + 32 * NB <= p.N) epilogue_rows_<EPI, NA, false>(p, acc, m0, n0, a0, pre);
    else epilogue_rows_<EPI, NA, true>(p, acc, m0, n0, a0, pre);
}

// Partial tile in fragment order: thread t's 16*NB accumulators at slot[(j*256 + t)],
// j = (a*NB + b)*4 + v.
template <int NB>
GPT2_DEV void store_partial(float* slot, const f32x4 (&acc)[4][NB]) {
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int v = 0; v < 4; v++) slot[((a * NB + b) * 4 + v) * NT + threadIdx.x] = acc[a][b][v];
}



typedef __attribute__((address_space(3))) float lds_float;

// LDS offset of a pointer into shared memory.
GPT2_DEV unsigned lds_offset(const float* p) { return (unsigned)(uintptr_t)(const lds_float*)p; }

// Global -> LDS transfers (16 or 4 bytes per lane): lane l's bytes land at lds + l*size,
// lds being uniform over the wave.  Written as inline asm so that the compiler, which
// cannot tell these LDS writes apart from the k-tiles being read, does not wait for all
// of them before every LDS read; the kernel waits for them itself (wait_vm).  M0 holds the
// LDS base; nothing else in these kernels uses M0.
GPT2_DEV void dma16(const float* g, float* lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds_offset(lds))), "v"(g) : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte offset, so
// that moving to the next k-tile is a scalar add.
GPT2_DEV void dma16s(const char* base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
GPT2_DEV void dma4(const void* g, float* lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds_offset(lds))), "v"(g) : "memory", "m0");
}

// LDS layouts of one k-tile (BK k values of ROWS rows), without padding so that a wave's
// 1 KB transfer is contiguous:
//  k-contiguous [row][BK]: 16-byte chunk c of row r sits at chunk position c ^ ((r>>1) % (BK/4))
//  row-contiguous, 128 rows, [k][128]: chunk c (rows 4c..4c+3) of k row kr sits at
//  c ^ rswz(kr)
//  row-contiguous, 96 rows, [row/16][kperm(kr)][16]: a 96-float k row cannot be swizzled
//  within itself (its six 16-float blocks cannot take four distinct bank groups for four k
//  rows), so each 16-row block is stored as a column of BK k rows with k row kr at
//  kperm(kr) = kr ^ ((kr>>2) & 3).
// A fragment read takes, for MFMA step s, k rows 16g + 4q + s (q = lane group) and 16
// consecutive rows: the swizzles put the four lane groups in four different 16-bank groups.
template <int BK>
GPT2_DEV int kswz(int r) { return (r >> 1) & (BK / 4 - 1); }
GPT2_DEV int rswz(int kr) { return ((kr >> 2) & 3) << 2; }
GPT2_DEV int kperm(int kr) { return kr ^ ((kr >> 2) & 3); }  // an involution
// float position of (k row kr, row r) in a row-contiguous tile of ROWS rows
template <int ROWS, int BK>
GPT2_DEV int rpos(int kr, int r) {
    static_assert(ROWS == 128 || ROWS == 96, "row-contiguous tiles are 128 or 96 rows");
    if (ROWS == 128) return kr * 128 + ((((r >> 2) ^ rswz(kr)) << 2) | (r & 3));
    return (((r >> 4) * BK + kperm(kr)) << 4) | (r & 15);
}

// Per-lane byte offsets of a tile's transfers from the tile's base, the operand element
// (row r0, k 0) for a k-contiguous operand X[r*ld + k] or (k 0, row r0) for a
// row-contiguous one X[k*ld + r].  A k-tile is then base + kstep * (its k stride), and
// wave transfer j of wave w fills LDS chunk q = 4j + w (1 KB).
//  k-contiguous: transfer q covers 16 rows (BK = 16: 64/KC rows); rows past rmax are
//  clamped to it (they only feed outputs that are never stored).
template <int ROWS, int BK>
GPT2_DEV void kcontig_offsets(unsigned (&off)[ROWS * BK / 1024], long ld, int r0, int rmax) {
    constexpr int KC = BK / 4;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < ROWS * BK / 1024; j++) {
        const int q = j * 4 + w;
        const int R = q * (64 / KC) + l / KC;
        const int c = (l % KC) ^ kswz<BK>(R);
        const int r = min(r0 + R, rmax);
        off[j] = (unsigned)(((long)(r - r0) * ld + 4 * c) * 4);
    }
}

//  row-contiguous: LDS chunk 64q + l holds 4 rows of one k row (the inverse of rpos);
//  float4 row groups are clamped to rmax4 (a multiple of 4 inside the row).
template <int ROWS, int BK>
GPT2_DEV void rcontig_offsets(unsigned (&off)[ROWS * BK / 1024], long ld, int r0, int rmax4) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < ROWS * BK / 1024; j++) {
        const int ch = (j * 4 + w) * 64 + l;
        int kr, rr;
        if (ROWS == 128) {
            kr = ch >> 5;
            rr = ((ch & 31) ^ rswz(kr)) << 2;
        } else {
            const int blk = ch >> 2;  // 16-float block: 16-row group blk / BK, k row kperm(blk % BK)
            kr = kperm(blk % BK);
            rr = (blk / BK) * 16 + 4 * (ch & 3);
        }
        const int r = min(r0 + rr, rmax4);
        off[j] = (unsigned)(((long)kr * ld + (r - r0)) * 4);
    }
}

// Bounds-checked k-tile through registers (the last k-tile when K is not a multiple of
// 16): zero outside the operand, written in the same swizzled layouts.
template <int ROWS, int BK>
GPT2_DEV void fill_kcontig(float* S, const float* X, long ld, int r0, int nrows, int k0, int K) {
    constexpr int KC = BK / 4, RPP = NT / KC;  // chunks per row, rows per pass
    const int t = threadIdx.x;
    const int c = t % KC, kk = k0 + 4 * c;
    float4 v[ROWS / RPP];
#pragma unroll
    for (int j = 0; j < ROWS / RPP; j++) {
        const int R = t / KC + RPP * j, r = r0 + R;
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nrows) {
            const float* q = X + (long)r * ld + kk;
            if (kk + 0 < K) v[j].x = q[0];
            if (kk + 1 < K) v[j].y = q[1];
            if (kk + 2 < K) v[j].z = q[2];
            if (kk + 3 < K) v[j].w = q[3];
        }
    }
#pragma unroll
    for (int j = 0; j < ROWS / RPP; j++) {
        const int R = t / KC + RPP * j;
        *reinterpret_cast<float4*>(S + R * BK + ((c ^ kswz<BK>(R)) << 2)) = v[j];
    }
}

template <int ROWS, int BK>
GPT2_DEV void fill_rcontig(float* S, const float* X, long ld, int r0, int nrows, int k0, int K) {
    constexpr int CH = ROWS / 4, PASSES = BK * CH / NT;  // chunks per k row, chunks per thread
    static_assert(BK * CH % NT == 0, "whole passes");
    const int t = threadIdx.x;
    float4 v[PASSES];
#pragma unroll
    for (int j = 0; j < PASSES; j++) {
        const int kr = (t + NT * j) / CH, k = k0 + kr, r = r0 + 4 * ((t + NT * j) % CH);
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k < K) {
            const float* q = X + (long)k * ld + r;
            if (r + 0 < nrows) v[j].x = q[0];
            if (r + 1 < nrows) v[j].y = q[1];
            if (r + 2 < nrows) v[j].z = q[2];
            if (r + 3 < nrows) v[j].w = q[3];
        }
    }
#pragma unroll
    for (int j = 0; j < PASSES; j++) {
        const int kr = (t + NT * j) / CH, c = (t + NT * j) % CH;
        *reinterpret_cast<float4*>(S + rpos<ROWS, BK>(kr, 4 * c)) = v[j];
    }
}

// bf16 row-contiguous tiles, [k][128] bf16 (256 bytes a k row, sixteen 16-byte chunks):
// chunk c of k row kr sits at chunk position c ^ trswz(kr).  A fragment is read with
// ds_read_b64_tr_b16, which hands lane i of a 16-lane group the i-th 16-bit value of each
// of the four 8-byte pieces that lanes 4e..4e+3 of the group loaded: lanes 4e + h load
// k row kb + e, rows 4h..4h+3 of the fragment, so lane i gets rows i of k rows kb..kb+3,
// the A (or B) operand layout of v_mfma_f32_16x16x32_bf16 (a second read gives k rows
// kb+4..kb+7).  One read instruction covers 16 k rows (kb = 8g for lane group g), 32 bytes
// of each; the swizzle puts them in the 8 32-byte bank windows of a 256-byte LDS row, two
// each: window (r/16) ^ ((kr & 3) | (kr & 8) >> 1).
GPT2_DEV int trswz(int kr) { return ((kr & 3) | ((kr >> 1) & 4)) << 1; }

// Per-lane byte offsets of a bf16 row-contiguous tile's transfers from the element (k 0,
// row r0) of X[k*ld + r] (ld in bf16 elements, a multiple of 8): LDS chunk 64q + l (q =
// 4j + wave) holds chunk (ch % 16) ^ trswz(ch / 16) of k row ch / 16.  Chunks past the
// end of a row are clamped to its last chunk (they only feed outputs never stored).
template <int BK>
GPT2_DEV void tr_offsets(unsigned (&off)[BK / 16], long ld, int r0) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < BK / 16; j++) {
        const int ch = (j * 4 + w) * 64 + l;
        const int kr = ch >> 4, c = (ch & 15) ^ trswz(ch >> 4);
        const long r = (long)r0 + 8 * c < ld - 8 ? (long)r0 + 8 * c : ld - 8;
        off[j] = (unsigned)(((long)kr * ld + (r - r0)) * 2);
    }
}

// The same tile through registers, zero for k >= K (the last k-tile when K is not a
// multiple of BK).
template <int BK>
GPT2_DEV void fill_tr(float* S, const float* Xf, long ld, int r0, int k0, int K) {
    const uint16_t* X = reinterpret_cast<const uint16_t*>(Xf);
    uint4 v[BK * 16 / NT];
#pragma unroll
    for (int j = 0; j < BK * 16 / NT; j++) {
        const int ch = (int)threadIdx.x + NT * j, kr = ch >> 4, c = (ch & 15) ^ trswz(ch >> 4);
        const long r = (long)r0 + 8 * c < ld - 8 ? (long)r0 + 8 * c : ld - 8;
        v[j] = make_uint4(0u, 0u, 0u, 0u);
        if (k0 + kr < K) v[j] = *reinterpret_cast<const uint4*>(X + (long)(k0 + kr) * ld + r);
    }
#pragma unroll
    for (int j = 0; j < BK * 16 / NT; j++) reinterpret_cast<uint4*>(S)[threadIdx.x + NT * j] = v[j];
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// 8 consecutive k of one fragment row: two transposing reads 4 k rows (1 KB) apart
GPT2_DEV bf16x8 tr_frag(const lds_char* p) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 1024));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, (v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}));
}

// The logits operand of the LM-head backward: each logit z of row r in vocabulary column
// c becomes d loss / d z = s * (exp(z - lse_r) - [c == target_r]), s = 1/rows.  The
// first term is formed as 2^(z log2 e - (lse_r log2 e - log2 s)) on v_exp_f32 with the
// row constant precomputed; the dgrad leaves the one-hot term to its epilogue and the
// wgrad to its caller.
constexpr float LOG2E = 1.4426950408889634f;
GPT2_DEV float softmax_s(float z, float c2) { return __builtin_amdgcn_exp2f(fmaf(z, LOG2E, -c2)); }

template <int N>
GPT2_DEV void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// BF: both operands are bfloat16 (mixed-precision variant).  k-contiguous (forward,
// dgrad), they are addressed as float pairs: a row of K bf16 values is a row of K/2
// floats, so the k-tiles, their LDS layout and the transfers are exactly those of the
// fp32 k-contiguous case, and each 16-float fragment group (16 bytes per lane = 8 bf16)
// feeds one v_mfma_f32_16x16x32_bf16 per block instead of four fp32 steps.
// Row-contiguous (the weight gradients, TR below), the k-tiles are 64 k rows of 128 bf16
// in the swizzled layout of trswz, and each fragment is two transposing LDS reads.
template <bool A_K, bool B_K, int EPI, bool XF, int BN, bool BF>
GPT2_DEV void gemm_body(const Params& p) {
    static_assert(BN == 128 || (BN == 96 && A_K) || (BN == 256 && BF), "tile widths: 128; 96 (A k-contiguous); 256 (bf16)");
    constexpr int SLOT_BIAS = slot_bias<BN>(), SLOT_FLOATS = slot_floats<BN>();
    static_assert(!BF || (A_K == B_K && !XF), "bf16 operands are both k-contiguous or both row-contiguous");
    // TR: bf16 row-contiguous operands, fragments by transposing LDS reads; p.K counts k
    // rows and p.lda, p.ldb bf16 elements
    constexpr bool TR = BF && !A_K;
    static_assert(!TR || BN == 128, "row-contiguous bf16 tiles are 128 x 128");
    constexpr int WN = BN / 2, NB = BN / 32;
    constexpr bool XR = XF && !A_K;  // dlogits as the row-contiguous operand (LM-head wgrad)
    constexpr int BK = KTileOf<A_K, BF, BN>::BK, STAGES = KTileOf<A_K, BF, BN>::STAGES;
    // the operands' k-tiles in LDS (floats)
    constexpr int A_FLOATS = TR ? BM * BK / 2 : BM * BK, B_FLOATS = TR ? BN * BK / 2 : BN * BK;
    constexpr int STAGE_FLOATS = A_FLOATS + B_FLOATS + (XR ? XF_FLOATS : 0);
    constexpr int LPS = (A_FLOATS + B_FLOATS) / 1024 + (XR ? 1 : 0);  // transfers per thread per k-tile
    __shared__ __attribute__((aligned(1024))) float smem[STAGES * STAGE_FLOATS];

    // XCD-aware logical block id: XCD x (= blockIdx % 8) gets a contiguous id range.
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int lb = xcd * (nb >> 3) + min(xcd, nb & 7) + local;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * WN;
    const int li = lane & 15, grp = lane >> 4;
    // 96-row row-contiguous B fragments: element (k row 16g + 4grp + s, row wn + 16b + li)
    // sits at rpos<96> = boff96[s] + (b BK + 16g) 16, since wn is a multiple of 16 and
    // kperm(16g + 4grp + s) = 16g + 4grp + (s ^ grp); the lane-dependent part stays in
    // four registers and the rest folds into the LDS reads' immediate offsets.
    int boff96[4];
#pragma unroll
    for (int s = 0; s < 4; s++) boff96[s] = (((wn >> 4) * BK + 4 * grp + (s ^ grp)) << 4) + li;
    const int kfull = p.K / BK;  // k-tiles that need no bounds check
    // row clamps: k-contiguous rows to the last row; row-contiguous float4 groups to the
    // last whole group inside the row (for the logits operand, inside the padded row)
    const int rmaxA = A_K ? p.M - 1 : (XF ? (int)p.lda - 4 : p.M - 4);
    const int rmaxB = B_K ? p.N - 1 : p.N - 4;

    // Work items: R whole tiles, then this block's range of the split region.
    long it = 0, it_begin = 0, it_end = 0;
    if (lb < p.nr) {
        it_begin = range_start(p.total, p.nr, lb);
        it_end = range_start(p.total, p.nr, lb + 1);
    }
    it = it_begin;
    int r = 0;
    struct Item {
        int tile, ks, ke, m0, n0;
        float* slot;  // partial-tile slot (split tiles only)
    };
    auto next_item = [&](Item& w) -> bool {
        w.slot = nullptr;
        if (p.S > 1) {
            // split-K rounds: unit u = r*G + lb is k-segment u / tiles of tile u % tiles
            const int u = r * p.G + lb;
            if (u >= p.units) return false;
            const int tiles = p.tiles_m * p.tiles_n;
            const int sg = u / tiles;
            w.tile = u - sg * tiles;
            w.ks = (int)((long)sg * p.nk / p.S);
            w.ke = (int)((long)(sg + 1) * p.nk / p.S);
            w.slot = p.partial + (long)u * SLOT_FLOATS;
            r++;
        } else if (r < p.R) {
            w.tile = r * p.G + lb;
            w.ks = 0;
            w.ke = p.nk;
            r++;
        } else if (it < it_end) {
            const int t = (int)(it / p.nk);
            w.ks = (int)(it - (long)t * p.nk);
            w.ke = (int)min((long)p.nk, w.ks + (it_end - it));
            // first segment of the range -> slot 0, the range's last (shared) tile -> slot 1
            w.slot = p.partial + ((long)lb * 2 + (it == it_begin ? 0 : 1)) * SLOT_FLOATS;
            w.tile = p.tile0 + t;
            it += w.ke - w.ks;
        } else {
            return false;
        }
        tile_coords<BN>(p, w.tile, w.m0, w.n0);
        return true;
    };

    // per-lane transfer offsets of the current item's tile (set by prologue)
    unsigned offA[A_FLOATS / 1024], offB[B_FLOATS / 1024];
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int buf, int kstep, int m0, int n0) {
        float* Sa = smem + buf * STAGE_FLOATS;
        float* Sb = Sa + A_FLOATS;
        const int k0 = kstep * BK;
        if constexpr (TR) {
            if (kstep < kfull) {
                const char* ba = reinterpret_cast<const char*>(p.A) + ((long)k0 * p.lda + m0) * 2;
                const char* bb = reinterpret_cast<const char*>(p.B) + ((long)k0 * p.ldb + n0) * 2;
                const unsigned la = lds0 + (unsigned)(buf * STAGE_FLOATS) * 4 + (unsigned)wave_u * 1024;
                const unsigned lb_ = la + A_FLOATS * 4;
#pragma unroll
                for (int j = 0; j < A_FLOATS / 1024; j++) dma16s(ba, offA[j], la + j * 4096);
#pragma unroll
                for (int j = 0; j < B_FLOATS / 1024; j++) dma16s(bb, offB[j], lb_ + j * 4096);
            } else {
                fill_tr<BK>(Sa, p.A, p.lda, m0, k0, p.K);
                fill_tr<BK>(Sb, p.B, p.ldb, n0, k0, p.K);
            }
        } else if (kstep < kfull) {
            const char* ba = reinterpret_cast<const char*>(p.A) +
                             (A_K ? (long)m0 * p.lda + k0 : (long)k0 * p.lda + m0) * 4;
            const char* bb = reinterpret_cast<const char*>(p.B) +
                             (B_K ? (long)n0 * p.ldb + k0 : (long)k0 * p.ldb + n0) * 4;
            const unsigned la = lds0 + (unsigned)(buf * STAGE_FLOATS) * 4 + (unsigned)wave_u * 1024;
            const unsigned lb_ = la + A_FLOATS * 4;
#pragma unroll
            for (int j = 0; j < BM * BK / 1024; j++) dma16s(ba, offA[j], la + j * 4096);
#pragma unroll
            for (int j = 0; j < BN * BK / 1024; j++) dma16s(bb, offB[j], lb_ + j * 4096);
        } else {
            if constexpr (A_K) fill_kcontig<BM, BK>(Sa, p.A, p.lda, m0, p.M, k0, p.K);
            else fill_rcontig<BM, BK>(Sa, p.A, p.lda, m0, XF ? (int)p.lda : p.M, k0, p.K);
            if constexpr (B_K) fill_kcontig<BN, BK>(Sb, p.B, p.ldb, n0, p.N, k0, p.K);
            else fill_rcontig<BN, BK>(Sb, p.B, p.ldb, n0, p.N, k0, p.K);
        }
        if (XR) {
            // lanes 0..BK-1: lse of k rows k0.. (further lanes repeat them)
            dma4(p.lse + min(k0 + lane % BK, p.K - 1), Sb + B_FLOATS + wave * 64);
        }
    };
    // the first STAGES-1 k-tiles of an item
    auto prologue = [&](const Item& w) {
        if constexpr (TR) {
            tr_offsets<BK>(offA, p.lda, w.m0);
            tr_offsets<BK>(offB, p.ldb, w.n0);
        } else {
            if constexpr (A_K) kcontig_offsets<BM, BK>(offA, p.lda, w.m0, rmaxA);
            else rcontig_offsets<BM, BK>(offA, p.lda, w.m0, rmaxA);
            if constexpr (B_K) kcontig_offsets<BN, BK>(offB, p.ldb, w.n0, rmaxB);
            else rcontig_offsets<BN, BK>(offB, p.ldb, w.n0, rmaxB);
        }
#pragma unroll
        for (int s = 0; s < STAGES - 1; s++)
            if (s < w.ke - w.ks) issue(s, w.ks + s, w.m0, w.n0);
    };

    Item cur;
    bool have = next_item(cur);
    if (have) prologue(cur);
    while (have) {
        const int m0 = cur.m0, n0 = cur.n0, ks = cur.ks, ke = cur.ke;
        f32x4 acc[4][NB];
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b < NB; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        // wgrad with bias: the waves of sub-tile column 0 sum their A fragments
        const bool bias_rows = !A_K && p.dbias != nullptr && n0 == 0 && wn == 0;
        float bsum[4] = {0.f, 0.f, 0.f, 0.f};

        // dlogits as the k-contiguous operand (LM-head dgrad): the exponent offset
        // lse log2 e - log2 s of this lane's four fragment rows
        float xl[4];
        if (XF && A_K) {
#pragma unroll
            for (int a = 0; a < 4; a++) {
                const int row = m0 + wm + 16 * a + li;
                xl[a] = row < p.M ? fmaf(p.lse[row], LOG2E, -p.xlog2s) : 0.f;
            }
        }

        // bf16 k-tile: BK/16 groups of 32 bf16, one MFMA per block and group
        auto compute_bf16 = [&](int buf) {
            const float* Sa = smem + buf * STAGE_FLOATS;
            const float* Sb = Sa + A_FLOATS;
#pragma unroll
            for (int g = 0; g < BK / 16; g++) {
                bf16x8 fa[4], fb[NB];
#pragma unroll
                for (int a = 0; a < 4; a++) {
                    const int row = wm + 16 * a + li;
                    fa[a] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const float4*>(
                                                           Sa + row * BK + (((4 * g + grp) ^ kswz<BK>(row)) << 2)));
                }
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    const int row = wn + 16 * b + li;
                    fb[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const float4*>(
                                                           Sb + row * BK + (((4 * g + grp) ^ kswz<BK>(row)) << 2)));
                }
#pragma unroll
                for (int a = 0; a < 4; a++)
#pragma unroll
                    for (int b = 0; b < NB; b++)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
            }
        };

        // one k-tile: BK/16 groups of 16 k, each 4 MFMA steps over this wave's blocks
        // (a generic lambda: instantiated only on the fp32 path)
        auto compute_f32 = [&](int buf, auto kstep) {
            const float* Sa = smem + buf * STAGE_FLOATS;
            const float* Sb = Sa + A_FLOATS;
            const int k0 = kstep * BK;
#pragma unroll
            for (int g = 0; g < BK / 16; g++) {
                float fa[4][4], fb[NB][4];
#pragma unroll
                for (int a = 0; a < 4; a++) {
                    const int row = wm + 16 * a + li;
                    if (A_K) {
                        const float4 v = *reinterpret_cast<const float4*>(Sa + row * BK + (((4 * g + grp) ^ kswz<BK>(row)) << 2));
                        fa[a][0] = v.x;
                        fa[a][1] = v.y;
                        fa[a][2] = v.z;
                        fa[a][3] = v.w;
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; s++) {
                            const int kr = 16 * g + 4 * grp + s;
                            fa[a][s] = Sa[rpos<BM, BK>(kr, row)];
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    const int row = wn + 16 * b + li;
                    if (B_K) {
                        const float4 v = *reinterpret_cast<const float4*>(Sb + row * BK + (((4 * g + grp) ^ kswz<BK>(row)) << 2));
                        fb[b][0] = v.x;
                        fb[b][1] = v.y;
                        fb[b][2] = v.z;
                        fb[b][3] = v.w;
                    } else if (BN == 96) {
                        // rpos<96> split into a per-lane part and an immediate offset
#pragma unroll
                        for (int s = 0; s < 4; s++) fb[b][s] = Sb[boff96[s] + (b * BK + 16 * g) * 16];
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; s++) {
                            const int kr = 16 * g + 4 * grp + s;
                            fb[b][s] = Sb[rpos<BN, BK>(kr, row)];
                        }
                    }
                }
                // dlogits: no bounds checks needed, since B is zero for k >= K (the
                // bounds-checked k-tile) and rows m >= M only feed outputs never stored
                if (XF && A_K) {
#pragma unroll
                    for (int a = 0; a < 4; a++)
#pragma unroll
                        for (int s = 0; s < 4; s++) fa[a][s] = softmax_s(fa[a][s], xl[a]);
                }
                if (XR) {
                    const float* xs = Sb + B_FLOATS + wave * 64 + 16 * g + 4 * grp;
                    const float4 l4 = *reinterpret_cast<const float4*>(xs);
                    // softmax term only: the caller subtracts the one-hot term
                    const float ls[4] = {fmaf(l4.x, LOG2E, -p.xlog2s), fmaf(l4.y, LOG2E, -p.xlog2s),
                                         fmaf(l4.z, LOG2E, -p.xlog2s), fmaf(l4.w, LOG2E, -p.xlog2s)};
#pragma unroll
                    for (int a = 0; a < 4; a++)
#pragma unroll
                        for (int s = 0; s < 4; s++) fa[a][s] = softmax_s(fa[a][s], ls[s]);
                }
                if (!A_K && bias_rows) {
#pragma unroll
                    for (int a = 0; a < 4; a++) bsum[a] += (fa[a][0] + fa[a][1]) + (fa[a][2] + fa[a][3]);
                }
#pragma unroll
                for (int s = 0; s < 4; s++)
#pragma unroll
                    for (int a = 0; a < 4; a++)
#pragma unroll
                        for (int b = 0; b < NB; b++)
                            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[a][s], fb[b][s], acc[a][b], 0, 0, 0);
            }
        };
        // bf16 row-contiguous k-tile: BK/32 groups of 32 k rows; lane (i, g) reads k rows
        // 32 kg + 8g + (i / 4) (+4) at fragment rows 4 (i % 4) .. +3
        auto compute_tr = [&](int buf) {
            const lds_char* Sa = (const lds_char*)(smem + buf * STAGE_FLOATS);
            const lds_char* Sb = Sa + A_FLOATS * 4;
            const int kr = 8 * grp + (li >> 2), sw = trswz(kr);
            auto frag_off = [&](int r) { return kr * 256 + ((((r >> 3) ^ sw)) << 4) + ((r & 7) << 1); };
#pragma unroll
            for (int kg = 0; kg < BK / 32; kg++) {
                bf16x8 fa[4], fb[NB];
#pragma unroll
                for (int a = 0; a < 4; a++) fa[a] = tr_frag(Sa + kg * 8192 + frag_off(wm + 16 * a + 4 * (li & 3)));
#pragma unroll
                for (int b = 0; b < NB; b++) fb[b] = tr_frag(Sb + kg * 8192 + frag_off(wn + 16 * b + 4 * (li & 3)));
#pragma unroll
                for (int a = 0; a < 4; a++)
#pragma unroll
                    for (int b = 0; b < NB; b++)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
            }
        };
        auto compute = [&](int buf, int kstep) {
            if constexpr (TR) compute_tr(buf);
            else if constexpr (BF) compute_bf16(buf);
            else compute_f32(buf, kstep);
        };

        // LDS ring: k-tile kt lives in buffer kt % STAGES; STAGES-1 tiles are in flight
        // while one is consumed.  Each thread waits for its own transfers of the next
        // k-tile, and the barrier then makes every thread's transfers visible (and retires
        // all reads of the buffer the next transfer overwrites).  Before k-tile 0 the
        // previous item's epilogue loads and stores may still be outstanding, and stores
        // can complete out of order with loads, so that wait is for everything.
        const int n = ke - ks;
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (GEMM_SETPRIO) __builtin_amdgcn_s_setprio(1);
        for (int kt = 0; kt < n; kt++) {
            if (kt + STAGES - 1 < n) issue((kt + STAGES - 1) % STAGES, ks + kt + STAGES - 1, m0, n0);
            compute(kt % STAGES, ks + kt);
            // k-tile kt+1 must have landed: STAGES-2 later ones may still be in flight
            if (kt + STAGES - 1 < n) wait_vm<(STAGES - 2) * LPS>();
            else wait_vm<0>();
            __builtin_amdgcn_s_barrier();
        }

        if (GEMM_SETPRIO) __builtin_amdgcn_s_setprio(0);
        // start the next item's transfers, then finish this one while they fly
        float* slot = cur.slot;
        have = next_item(cur);
        if (have) prologue(cur);

        const bool full = ks == 0 && ke == p.nk;
        if (bias_rows) {
            // add the four lane groups (k offsets) of each row
#pragma unroll
            for (int a = 0; a < 4; a++) {
                float s = bsum[a];
                s = rows4_sum(s);
                const int row = wm + 16 * a + li;
                if (grp == 0) {
                    if (full) {
                        if (m0 + row < p.M) p.dbias[m0 + row] += s;
                    } else {
                        slot[SLOT_BIAS + row] = s;
                    }
                }
            }
        }
        if (full) {
            epilogue_rows<EPI, 4>(p, acc, m0, n0, 0, [] {});
        } else {
            store_partial(slot, acc);
        }
    }
}

template <bool A_K, bool B_K, int EPI, bool XF, int BN>
__global__ __launch_bounds__(NT, 2) void gemm_kernel(Params p) {
    gemm_body<A_K, B_K, EPI, XF, BN, false>(p);
}

#ifndef GEMM_BF_OCC
#define GEMM_BF_OCC 2
#endif
template <int EPI, int BN>
__global__ __launch_bounds__(NT, GEMM_BF_OCC) void gemm_bf16_kernel(Params p) {
    gemm_body<true, true, EPI, false, BN, true>(p);
}

// bf16 operands row-contiguous (the weight gradients)
template <int EPI, int BN>
__global__ __launch_bounds__(NT, GEMM_BF_OCC) void gemm_bf16_tr_kernel(Params p) {
    gemm_body<false, false, EPI, false, BN, true>(p);
}

// Four blocks per range boundary that falls strictly inside a tile, one per row of
// 16x16 blocks (a) of the waves' sub-tiles; for the lowest such boundary of a tile they
// add that tile's partials in k order and run the epilogue.
template <int EPI, int BN>
__global__ __launch_bounds__(NT) void gemm_fixup_kernel(Params p) {
    constexpr int NB = BN / 32, SLOT_BIAS = slot_bias<BN>(), SLOT_FLOATS = slot_floats<BN>();
    const int quarter = blockIdx.x & 3;
    const int lbb = (blockIdx.x >> 2) + 1;  // boundary between blocks lbb-1 and lbb
    const long x = range_start(p.total, p.nr, lbb);
    if (x % p.nk == 0) return;
    const int tile = (int)(x / p.nk);
    if (lbb >= 2) {
        const long xp = range_start(p.total, p.nr, lbb - 1);
        if (xp / p.nk == tile && xp % p.nk != 0) return;
    }
    const long t0 = (long)tile * p.nk;
    const int first = owner(p.total, p.nr, t0);
    const int last = owner(p.total, p.nr, t0 + p.nk - 1);
    f32x4 acc[1][NB];
#pragma unroll
    for (int b = 0; b < NB; b++) acc[0][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    int m0, n0;
    tile_coords<BN>(p, p.tile0 + tile, m0, n0);
    // the partials are summed after the epilogue has requested its own inputs
    auto slot_of = [&](int l) {
        const int which = range_start(p.total, p.nr, l) / p.nk == tile ? 0 : 1;
        return p.partial + ((long)l * 2 + which) * SLOT_FLOATS + quarter * (4 * NB) * NT + threadIdx.x;
    };
    epilogue_rows<EPI, 1>(p, acc, m0, n0, quarter, [&] {
        // four partials at a time in flight, added in k order
        constexpr int F = 4;
        for (int l = first; l <= last; l += F) {
            float v[F][4 * NB];
#pragma unroll
            for (int f = 0; f < F; f++) {
                if (l + f <= last) {
                    const float* sf = slot_of(l + f);
#pragma unroll
                    for (int e = 0; e < 4 * NB; e++) v[f][e] = sf[e * NT];
                }
            }
#pragma unroll
            for (int f = 0; f < F; f++) {
                if (l + f <= last) {
#pragma unroll
                    for (int e = 0; e < 4 * NB; e++) acc[0][e >> 2][e & 3] += v[f][e];
                }
            }
        }
    });
    if (p.dbias && n0 == 0 && quarter == 0 && threadIdx.x < BM && m0 + (int)threadIdx.x < p.M) {
        float s = 0.f;
        for (int l = first; l <= last; l++) {
            const int which = range_start(p.total, p.nr, l) / p.nk == tile ? 0 : 1;
            s += p.partial[((long)l * 2 + which) * SLOT_FLOATS + SLOT_BIAS + threadIdx.x];
        }
        p.dbias[m0 + threadIdx.x] += s;
    }
}

// Split-K rounds: four blocks per tile, one per row of 16x16 blocks (a) of the waves'
// sub-tiles, add the tile's S partials in k order and run the epilogue.  Partials in
// flight per step: 4 (8 measured slower on the 124M weight gradients: 22.4 against 18.2 us
// per launch).
#ifndef GEMM_FIXUP_F
#define GEMM_FIXUP_F 4
#endif
template <int EPI, int BN>
__global__ __launch_bounds__(NT) void gemm_splitk_fixup_kernel(Params p) {
    constexpr int NB = BN / 32, SLOT_BIAS = slot_bias<BN>(), SLOT_FLOATS = slot_floats<BN>();
    const int tiles = p.tiles_m * p.tiles_n;
    const int tile = blockIdx.x >> 2, quarter = blockIdx.x & 3;
    f32x4 acc[1][NB];
#pragma unroll
    for (int b = 0; b < NB; b++) acc[0][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    int m0, n0;
    tile_coords<BN>(p, tile, m0, n0);
    epilogue_rows<EPI, 1>(p, acc, m0, n0, quarter, [&] {
        // GEMM_FIXUP_F partials at a time in flight, added in segment order
        constexpr int F = GEMM_FIXUP_F;
        for (int sg = 0; sg < p.S; sg += F) {
            float v[F][4 * NB];
#pragma unroll
            for (int f = 0; f < F; f++) {
                if (sg + f < p.S) {
                    const float* slot = p.partial + ((long)(sg + f) * tiles + tile) * SLOT_FLOATS +
                                        quarter * (4 * NB) * NT + threadIdx.x;
#pragma unroll
                    for (int e = 0; e < 4 * NB; e++) v[f][e] = slot[e * NT];
                }
            }
#pragma unroll
            for (int f = 0; f < F; f++) {
                if (sg + f < p.S) {
#pragma unroll
                    for (int e = 0; e < 4 * NB; e++) acc[0][e >> 2][e & 3] += v[f][e];
                }
            }
        }
    });
    if (p.dbias && n0 == 0 && quarter == 0 && threadIdx.x < BM && m0 + (int)threadIdx.x < p.M) {
        float sum = 0.f;
        for (int sg = 0; sg < p.S; sg++) sum += p.partial[((long)sg * tiles + tile) * SLOT_FLOATS + SLOT_BIAS + threadIdx.x];
        p.dbias[m0 + threadIdx.x] += sum;
    }
}

// Kernel name as profilers print the instantiation.
template <bool A_K, bool B_K, int EPI, bool XF, int BN>
const char* gemm_name() {
    static const std::string s = std::string("gemm_kernel<") + (A_K ? "true" : "false") + ", " +
                                 (B_K ? "true" : "false") + ", " + std::to_string(EPI) + ", " +
                                 (XF ? "true" : "false") + ", " + std::to_string(BN) + ">";
    return s.c_str();
}

template <int EPI, int BN>
const char* bf16_name(bool tr = false) {
    static const std::string s = "gemm_bf16_kernel<" + std::to_string(EPI) + ", " + std::to_string(BN) + ">";
    static const std::string t = "gemm_bf16_tr_kernel<" + std::to_string(EPI) + ", " + std::to_string(BN) + ">";
    if (tr) return t.c_str();
    return s.c_str();
}

template <int EPI, int BN>
const char* fixup_name() {
    static const std::string s = "gemm_fixup_kernel<" + std::to_string(EPI) + ", " + std::to_string(BN) + ">";
    return s.c_str();
}

template <int EPI, int BN>
const char* splitk_fixup_name() {
    static const std::string s = "gemm_splitk_fixup_kernel<" + std::to_string(EPI) + ", " + std::to_string(BN) + ">";
    return s.c_str();
}

// Work distribution over a persistent grid of up to RESIDENT blocks: whole-tile rounds
// while at least RESIDENT tiles remain, then equal ranges of the rest.
// The fp32 weight gradients run on their own stream next to the main backward chain; a
// persistent grid of fewer blocks than the chip holds leaves CU slots to that chain
// (measured slower: 448, 384 and 256 blocks give 55.6, 56.5 and 57.0 ms per step against
// 55.0 at 512).
#ifndef GEMM_WGRAD_RESIDENT
#define GEMM_WGRAD_RESIDENT RESIDENT
#endif
// fp32 weight gradients as split-K rounds ordered k-segment first (as the bf16 ones)
// instead of stream-K ranges: the 64 blocks of an XCD then work on neighbouring tiles at
// the same k and share operand panels in that XCD's L2.  Same time (54.90 against
// 54.84 ms per step), but the kernel's memory-side reads fall from 435 to 80 MB per
// launch (114.8 MB algorithmic), which leaves the fabric to the concurrent main chain.
#ifndef GEMM_F32_WGRAD_SPLITK
#define GEMM_F32_WGRAD_SPLITK 1
#endif
// ... launched as one block per split-K unit rather than a persistent grid, so that blocks
// retire (and free CU slots for the main chain's kernels) every unit (measured slower:
// 56.15 against 55.06 ms per step).
#ifndef GEMM_WGRAD_NONPERSISTENT
#define GEMM_WGRAD_NONPERSISTENT 0
#endif
void schedule(Params& p, long tiles, int split, int resident = RESIDENT) {
    p.R = 0;
    p.tile0 = 0;
    p.S = 0;
    p.units = 0;
    if (split > 1 && p.partial != nullptr && tiles * split <= MAX_UNITS && split <= p.nk) {
        p.S = split;
        p.units = (int)tiles * split;
        // resident < 0: one block per unit instead of a persistent grid
        p.G = resident < 0 ? p.units : std::min(resident, p.units);
        p.nr = 0;
        p.skt = 0;
        p.total = 0;
        return;
    }
    if (resident < 0) resident = RESIDENT;
    if (p.partial == nullptr) {  // nowhere to put partial tiles: one tile per block
        p.G = (int)tiles;
        p.R = 1;
        p.tile0 = (int)tiles;
        p.skt = 0;
        p.total = 0;
        p.nr = 0;
        return;
    }
    if (tiles >= resident) {
        p.G = resident;
        p.R = (int)(tiles / resident);
        p.tile0 = p.R * resident;
    }
    p.skt = (int)(tiles - p.tile0);
    p.total = (long)p.skt * p.nk;
    p.nr = (int)std::min<long>(resident, p.total);
    if (p.R == 0) p.G = p.nr;
}

template <bool A_K, bool B_K, int EPI, bool XF, int BN, bool BF = false>
hipError_t launch(Params& p, hipStream_t st, int split, int resident = RESIDENT) {
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.nk = (p.K + KTileOf<A_K, BF, BN>::BK - 1) / KTileOf<A_K, BF, BN>::BK;
    const long tiles = (long)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    if (p.nk == 0) {
        // empty reduction: every output is the epilogue of 0
        p.nk = 1;
    }
    schedule(p, tiles, split, resident);
    const double mn = (double)p.M * p.N;
    const double extra = (EPI == EPI_BIAS_RESID || EPI == EPI_ACCUM || EPI == EPI_GELU_BWD || EPI == EPI_BIAS_GELU ||
                          EPI == EPI_DLOGITS) ? mn : 0.0;
    {
        // algorithmic work: 2MNK flops; operands read once, C written (and read for += / aux)
        // (bf16 k-contiguous: p.K counts float pairs, so the flops double and the operand
        // bytes match; bf16 row-contiguous: p.K counts k rows of 2-byte elements)
        constexpr bool TR = BF && !A_K;
        ProfScope ps(st, BF ? bf16_name<EPI, BN>(TR) : gemm_name<A_K, B_K, EPI, XF, BN>(),
                     (BF && !TR ? 4.0 : 2.0) * mn * p.K,
                     (TR ? 2.0 : 4.0) * ((double)p.M * p.K + (double)p.N * p.K) + 4.0 * (mn + extra));
        if constexpr (TR) hipLaunchKernelGGL((gemm_bf16_tr_kernel<EPI, BN>), dim3(p.G), dim3(NT), 0, st, p);
        else if constexpr (BF) hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BN>), dim3(p.G), dim3(NT), 0, st, p);
        else hipLaunchKernelGGL((gemm_kernel<A_K, B_K, EPI, XF, BN>), dim3(p.G), dim3(NT), 0, st, p);
    }
    // fix-up algorithmic bytes: the partial tiles it reads, and for each tile it finishes
    // the output written (and read too where the epilogue reads C or an aux tensor)
    const double slot = (double)BM * BN + BM;
    const double per_tile = (double)BM * BN * (extra > 0 ? 2.0 : 1.0);
    if (p.S > 1) {
        const double split_tiles = (double)(p.units / p.S);
        ProfScope ps(st, splitk_fixup_name<EPI, BN>(), 0.0, 4.0 * ((double)p.units * slot + split_tiles * per_tile));
        hipLaunchKernelGGL((gemm_splitk_fixup_kernel<EPI, BN>), dim3(4 * (p.units / p.S)), dim3(NT), 0, st, p);
    } else if (p.nr > 1 && !(p.total % p.nr == 0 && (p.total / p.nr) % p.nk == 0)) {
        // the (range, tile) pieces that are not whole tiles, and the tiles they split
        long pieces = 0, split_tiles = 0, last_split = -1;
        for (int l = 0; l < p.nr; l++) {
            const long s0 = (long)l * p.total / p.nr, s1 = (long)(l + 1) * p.total / p.nr;
            for (long t = s0 / p.nk; s1 > s0 && t <= (s1 - 1) / p.nk; t++) {
                const long a = std::max(s0, t * p.nk), b = std::min(s1, (t + 1) * p.nk);
                if (b - a < p.nk) {
                    pieces++;
                    if (t != last_split) split_tiles++, last_split = t;
                }
            }
        }
        ProfScope ps(st, fixup_name<EPI, BN>(), 0.0, 4.0 * ((double)pieces * slot + (double)split_tiles * per_tile));
        hipLaunchKernelGGL((gemm_fixup_kernel<EPI, BN>), dim3(4 * (p.nr - 1)), dim3(NT), 0, st, p);
    }
    return hipGetLastError();
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

// k-split factor that turns a shape with fewer tiles than resident blocks and a long k
// extent into whole rounds of split-K units (e.g. 384 tiles -> 4 segments, 3 rounds); 0
// when there is none (stream-K then).
template <bool A_K, int BN, bool BF = false>
int pick_split(int M, int N, int K) {
    const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int nk = (K + KTileOf<A_K, BF, BN>::BK - 1) / KTileOf<A_K, BF, BN>::BK;
    if (tiles == 0 || tiles >= RESIDENT) return 0;
    for (int s = 2; s <= 8; s++)
        if ((tiles * s) % RESIDENT == 0 && tiles * s <= MAX_UNITS && nk >= 16 * s) return s;
    return 0;
}

// Tile width of the kernels whose A is k-contiguous (forward, dgrad): 96 when that gives
// whole rounds of resident blocks and 128 does not, else 128.  For 8192 rows, N = 768 is
// 512 tiles of 128x96 (one round, no split tiles) against 384 of 128x128, and N = 2304 is
// 1536 (three rounds) against 1152.  gemm_set_tile_policy can force either width.
int g_tile_policy = GEMM_TILES_AUTO;

int tile_n(int M, int N) {
    if (g_tile_policy == GEMM_TILES_128) return 128;
    if (g_tile_policy == GEMM_TILES_96) return 96;
    const long tm = (M + BM - 1) / BM;
    const long t128 = tm * ((N + 127) / 128), t96 = tm * ((N + 95) / 96);
    return (t96 > 0 && t96 % RESIDENT == 0 && t128 % RESIDENT != 0) ? 96 : 128;
}

// bf16 shapes with fewer tiles than resident blocks (the weight gradients: few output
// tiles, k = B*T long) run as split-K rounds ordered k-segment first, so the 64 blocks of
// an XCD work on 64 neighbouring tiles at the same k and share their operand panels in
// that XCD's L2 (stream-K gives each block its own k offset, and every panel comes from
// HBM again).  S is the split that fills rounds best (at least 90%), each unit at least
// 8 k-tiles long.
#ifndef GEMM_BF_SPLITK
#define GEMM_BF_SPLITK 1
#endif
template <bool A_K, bool BF, int BN>
int pick_split_rounds(int M, int N, int K, int resident = RESIDENT, int max_rounds = 3, double min_util = 0.9) {
    const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int nk = (K + KTileOf<A_K, BF, BN>::BK - 1) / KTileOf<A_K, BF, BN>::BK;
    if (tiles == 0 || tiles >= resident) return 0;
    int best = 0;
    double best_util = min_util;
    for (int s = 2; s <= 16; s++) {
        const long units = tiles * s;
        if (units > MAX_UNITS || units > (long)max_rounds * resident || nk < 8 * s) break;
        const double util = (double)units / (double)(((units + resident - 1) / resident) * resident);
        if (util > best_util + 1e-9) {
            best_util = util;
            best = s;
        }
    }
    return best;
}

// the bf16 weight gradients' split-K: at most this many rounds of resident blocks, filled
// at least this well.  One round at >= 0.5 gives 4 k-segments instead of 14 for 108 tiles
// and 3 instead of 7 for 144: at bf16 speed the partial tiles' traffic costs more than the
// idle blocks (measured at the 124M shapes: 55.8 against 61.3 us per launch, fix-ups 11.9
// against 16.9 us, bf16 step 15.84 against 16.15 ms).
#ifndef GEMM_BF_WGRAD_MAX_ROUNDS
#define GEMM_BF_WGRAD_MAX_ROUNDS 1
#endif
#ifndef GEMM_BF_WGRAD_MIN_UTIL
#define GEMM_BF_WGRAD_MIN_UTIL 0.5
#endif
template <int BN>
int split_bf16(int M, int N, int K) {
    return GEMM_BF_SPLITK ? pick_split_rounds<true, true, BN>(M, N, K) : 0;
}

// Tile width of the bf16 GEMMs: 256 (a 64 x 128 sub-tile per wave: a quarter less LDS and
// L2 traffic per MFMA than 64 x 64) where N allows, else as the fp32 forward GEMMs.
// Measured slower at the 124M shapes (fewer tiles: more and larger stream-K partials,
// with no faster main loop), so off unless built with -DGEMM_BF_WIDE=1.
#ifndef GEMM_BF_WIDE
#define GEMM_BF_WIDE 0
#endif
int bf16_tile_n(int M, int N) {
    if (GEMM_BF_WIDE && N >= 256) return 256;
    return tile_n(M, N);
}

template <bool B_K, int EPI, bool XF = false>
hipError_t launch_ak(Params& p, hipStream_t st) {
    // The dlogits dgrad keeps 128-wide tiles unless forced: its exponentials are spread
    // over 16 instead of 12 MFMAs per fragment row, and its long k extent over few tiles
    // runs as split-K rounds (measured: 128 x 128 with 4 k-segments beats one round of
    // 128 x 96 tiles over the whole vocabulary).
    const int bn = (XF && g_tile_policy == GEMM_TILES_AUTO) ? 128 : tile_n(p.M, p.N);
    if (bn == 96) return launch<true, B_K, EPI, XF, 96>(p, st, XF ? pick_split<true, 96>(p.M, p.N, p.K) : 0);
    return launch<true, B_K, EPI, XF, 128>(p, st, XF ? pick_split<true, 128>(p.M, p.N, p.K) : 0);
}

}  // namespace

size_t lse_partial_floats(int M, int N) { return (size_t)M * 2 * 2 * (size_t)((N + 95) / 96); }

// (max, sum) pairs per row that an LSE-fused forward of this shape writes: two per tile
// column, at the tile width its launcher picks
int lse_partial_count(int M, int N, bool bf16) {
    const int bn = bf16 ? bf16_tile_n(M, N) : tile_n(M, N);
    return 2 * ((N + bn - 1) / bn);
}

size_t gemm_partial_floats() { return (size_t)std::max(RESIDENT * 2, MAX_UNITS) * slot_floats<GEMM_BF_WIDE ? 256 : 128>(); }

bool gemm_set_tile_policy(int policy) {
    if (policy != GEMM_TILES_AUTO && policy != GEMM_TILES_128 && policy != GEMM_TILES_96) return false;
    g_tile_policy = policy;
    return true;
}

hipError_t linear_forward(float* out, long ldo, const float* inp, const float* w,
                          const float* bias, const float* resid, float* pre, int M, int N, int K,
                          float* partial, hipStream_t st, float* lse_part) {
    if (K % 4 || !aligned16(inp) || !aligned16(w)) return hipErrorInvalidValue;
    if (lse_part && (bias || resid || pre)) return hipErrorInvalidValue;
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
        return launch_ak<true, EPI_BIAS_GELU>(p, st);
    }
    if (resid) {
        p.aux = resid;
        p.ldaux = ldo;
        return launch_ak<true, EPI_BIAS_RESID>(p, st);
    }
    if (bias) return launch_ak<true, EPI_BIAS>(p, st);
    if (lse_part) {
        p.lsep = lse_part;
        return launch_ak<true, EPI_STORE_LSE>(p, st);
    }
    return launch_ak<true, EPI_STORE>(p, st);
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
        return launch_ak<false, EPI_GELU_BWD>(p, st);
    }
    if (xent) {
        p.lse = xent->lse;
        p.tgt = xent->targets;
        if (!(xent->scale > 0.f)) return hipErrorInvalidValue;
        p.xscale = xent->scale;
        p.xlog2s = (float)std::log2((double)xent->scale);
        return launch_ak<false, EPI_DLOGITS, true>(p, st);
    }
    return launch_ak<false, EPI_STORE>(p, st);
}

hipError_t linear_wgrad(float* dw, float* dbias, const float* dout, long ld_dout, const float* inp, int M,
                        int N, int K, float* partial, hipStream_t st, const XentOperand* xent) {
    // row-contiguous operands move in 16-byte groups: dout's row groups must stay inside
    // its M columns (or, for the logits operand, inside its padded row)
    if (ld_dout % 4 || N % 4 || ld_dout < M || (!xent && M % 4) || !aligned16(dout) || !aligned16(inp))
        return hipErrorInvalidValue;
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
        if (!(xent->scale > 0.f)) return hipErrorInvalidValue;
        p.xscale = xent->scale;
        p.xlog2s = (float)std::log2((double)xent->scale);
        return launch<false, false, EPI_ACCUM, true, 128>(p, st, 0);
    }
    const int split = GEMM_F32_WGRAD_SPLITK ? pick_split_rounds<false, false, 128>(M, N, K, GEMM_WGRAD_RESIDENT) : 0;
    return launch<false, false, EPI_ACCUM, false, 128>(
        p, st, split, (GEMM_WGRAD_NONPERSISTENT && split > 1) ? -1 : GEMM_WGRAD_RESIDENT);
}

hipError_t gemm_bf16(int epi, float* c, long ldc, const uint16_t* a, long lda, const uint16_t* b, long ldb, int M,
                     int N, int K, const float* bias, const float* aux, long ldaux, float* pre, float* partial,
                     hipStream_t st, float* lse_part, uint16_t* cb, long ldcb, float* csum) {
    if (K % 2 || lda % 8 || ldb % 8 || lda < K || ldb < K || !aligned16(a) || !aligned16(b)) return hipErrorInvalidValue;
    if (cb && ((epi != BF16_BIAS_GELU && epi != BF16_GELU_BWD) || N % 2 || ldcb % 2 || ldcb < N || ((uintptr_t)cb & 3)))
        return hipErrorInvalidValue;
    if (csum && epi != BF16_GELU_BWD) return hipErrorInvalidValue;
    Params p{};
    p.M = M;
    p.N = N;
    p.K = K / 2;  // float pairs
    p.A = reinterpret_cast<const float*>(a);
    p.lda = lda / 2;
    p.B = reinterpret_cast<const float*>(b);
    p.ldb = ldb / 2;
    p.C = c;
    p.ldc = ldc;
    p.bias = bias;
    p.aux = aux;
    p.ldaux = ldaux;
    p.pre = pre;
    p.ldpre = ldc;
    p.partial = partial;
    p.cb = cb;
    p.ldcb = ldcb;
    p.csum = csum;
    const int bn = bf16_tile_n(M, N);
    auto go = [&](auto epi_c) -> hipError_t {
        constexpr int E = decltype(epi_c)::value;
        if constexpr (GEMM_BF_WIDE != 0)
            if (bn == 256) return launch<true, true, E, false, 256, true>(p, st, split_bf16<256>(p.M, p.N, p.K));
        if (bn == 96) return launch<true, true, E, false, 96, true>(p, st, split_bf16<96>(p.M, p.N, p.K));
        return launch<true, true, E, false, 128, true>(p, st, split_bf16<128>(p.M, p.N, p.K));
    };
    switch (epi) {
        case BF16_STORE:
            if (lse_part) {
                p.lsep = lse_part;
                return go(std::integral_constant<int, EPI_STORE_LSE>{});
            }
            return go(std::integral_constant<int, EPI_STORE>{});
        case BF16_BIAS: return go(std::integral_constant<int, EPI_BIAS>{});
        case BF16_BIAS_RESID: return aux ? go(std::integral_constant<int, EPI_BIAS_RESID>{}) : hipErrorInvalidValue;
        case BF16_BIAS_GELU: return pre ? go(std::integral_constant<int, EPI_BIAS_GELU>{}) : hipErrorInvalidValue;
        case BF16_ACCUM: return go(std::integral_constant<int, EPI_ACCUM>{});
        case BF16_GELU_BWD: return aux ? go(std::integral_constant<int, EPI_GELU_BWD>{}) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

hipError_t gemm_bf16_rows(float* c, long ldc, const uint16_t* a, long lda, const uint16_t* b, long ldb, int M, int N,
                          int K, float* partial, hipStream_t st) {
    if (M < 0 || N < 0 || K < 0 || lda % 8 || ldb % 8 || lda < M || ldb < N || !aligned16(a) || !aligned16(b))
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    Params p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = reinterpret_cast<const float*>(a);
    p.lda = lda;
    p.B = reinterpret_cast<const float*>(b);
    p.ldb = ldb;
    p.C = c;
    p.ldc = ldc;
    p.partial = partial;
    return launch<false, false, EPI_ACCUM, false, 128, true>(
        p, st,
        GEMM_BF_SPLITK ? pick_split_rounds<false, true, 128>(M, N, K, RESIDENT, GEMM_BF_WGRAD_MAX_ROUNDS,
                                                             GEMM_BF_WGRAD_MIN_UTIL)
                       : 0);
}

}  // namespace gpt2k
