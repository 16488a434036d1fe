// bfloat16 operand copies for the mixed-precision variant.
//
// The pages name mixed precision as llm.c's next step (新智元 article "千行C代码训完
// GPT-2", 纯CUDA也可训; "OpenAI创始大神手搓千行C代码训练GPT", opening).  Here every
// linear layer and the LM head multiply bfloat16 roundings of their operands on the
// matrix cores; master weights, activations and everything else stay fp32.  Each
// operand is written once as a bf16 copy in the layout its products read:
//   forward:   X (rows, in) and W (out, in) as they are;
//   dgrad:     dY (rows, out) as it is, W transposed (in, out), rows padded to 64 with
//              zeros;
//   wgrad:     dY and X as they are (the GEMM reads them row-contiguous, with
//              transposing LDS reads).
// The layers' inputs get their copies from their producers (LayerNorm, attention, the fc
// GEMM's GELU epilogue).  Here one 64x64-tile kernel reads an fp32 tensor once and
// writes the straight copy, optionally the transposed copy (through LDS; the weights)
// and, for an output gradient, the bias gradient's column sums per 128-row block (the
// bias gradient is summed from the unrounded fp32 values).  The LM head's output
// gradient, softmax minus one-hot over the rows' log-sum-exp, is formed by the same
// kernel from the logits.  All of these kernels are bound by HBM.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int TILE = 64, CT_THREADS = 256, LDT = TILE + 1;

struct XentArgs {
    const float* lse;
    const int32_t* targets;
    float scale;
    int V;
};

// Grid (column tiles of 64, row blocks of RB = 128 over rows rounded up to 64, batch).
// XENT: the input is the logits and each element becomes its loss gradient first.
constexpr int RB = 128;
template <bool XENT>
__global__ __launch_bounds__(CT_THREADS) void cast_tile_kernel(CastArgs a, XentArgs xa) {
    __shared__ float tile[RB][LDT];
    const int t = threadIdx.x;
    const int c0 = blockIdx.x * TILE, r0 = blockIdx.y * RB, z = blockIdx.z;
    const float* x = a.x + (long)z * a.sx;
    // load: 16 threads per row (4 columns each), 16 rows per pass, 8 passes in flight
    const int c4 = t & 15, rr = t >> 4;
    const int col = c0 + 4 * c4;
    float4 v[RB / 16];
#pragma unroll
    for (int j = 0; j < RB / 16; j++) {
        const int r = r0 + rr + 16 * j;
        v[j] = (r < a.rows && col < a.cols) ? *reinterpret_cast<const float4*>(x + (long)r * a.ldx + col)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < RB / 16; j++) {
        const int row = rr + 16 * j, r = r0 + row;
        if (XENT && r < a.rows && col < a.cols) {
            const float l = xa.lse[r];
            const int tg = xa.targets[r];
            float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int c = col + i;
                e[i] = c < xa.V ? (__expf(e[i] - l) - (c == tg ? 1.f : 0.f)) * xa.scale : 0.f;
            }
            v[j] = make_float4(e[0], e[1], e[2], e[3]);
        }
        if (a.xb && r < a.rows && col < a.cols) {
            uint2 o;
            o.x = bf16_pack2(v[j].x, v[j].y);
            o.y = bf16_pack2(v[j].z, v[j].w);
            *reinterpret_cast<uint2*>(a.xb + (long)z * a.sb + (long)r * a.ldb + col) = o;
        }
        tile[row][4 * c4 + 0] = v[j].x;
        tile[row][4 * c4 + 1] = v[j].y;
        tile[row][4 * c4 + 2] = v[j].z;
        tile[row][4 * c4 + 3] = v[j].w;
    }
    __syncthreads();
    if (a.xt) {
        // transposed: thread (cc, s) writes 16 rows of column cc as 16 bf16 per pass; rows
        // past the padded count (a multiple of 64) are not stored
        const int cc = t >> 2, s = t & 3;
        const long rpad = (a.rows + TILE - 1) / TILE * TILE;
        if (c0 + cc < a.cols) {
#pragma unroll
            for (int h = 0; h < RB / 64; h++) {
                const int rl = 64 * h + 16 * s;
                if (r0 + rl < rpad) {
                    uint32_t w[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) w[i] = bf16_pack2(tile[rl + 2 * i][cc], tile[rl + 2 * i + 1][cc]);
                    uint4* q = reinterpret_cast<uint4*>(a.xt + (long)z * a.st + (long)(c0 + cc) * a.ldt + r0 + rl);
                    q[0] = make_uint4(w[0], w[1], w[2], w[3]);
                    q[1] = make_uint4(w[4], w[5], w[6], w[7]);
                }
            }
        }
    }
    if (a.bpart) {
        // column sums of the block's rows: four threads per column, 32 rows each, added in
        // a fixed order
        __shared__ float ps[4][TILE];
        const int cl = t & 63, q = t >> 6;
        float sum = 0.f;
#pragma unroll 8
        for (int i = 0; i < RB / 4; i++) sum += tile[q * (RB / 4) + i][cl];
        ps[q][cl] = sum;
        __syncthreads();
        if (q == 0 && c0 + cl < a.cols)
            a.bpart[(long)blockIdx.y * a.cols + c0 + cl] = ((ps[0][cl] + ps[1][cl]) + ps[2][cl]) + ps[3][cl];
    }
}

// db[c] += sum over row blocks of bpart[rb][c]: 64 columns per block, sixteen threads per
// column each summing every sixteenth row block (eight loads in flight), then the sixteen
// partial sums added in a fixed order.
constexpr int BR_GROUPS = 16, BR_UNROLL = 8;
__global__ __launch_bounds__(TILE * BR_GROUPS) void bias_reduce_kernel(float* db, const float* bpart, int nrb, int cols) {
    __shared__ float part[BR_GROUPS][TILE];
    const int cl = threadIdx.x % TILE, q = threadIdx.x / TILE;
    const int c = blockIdx.x * TILE + cl;
    float s = 0.f;
    if (c < cols) {
        int rb = q;
        for (; rb + BR_GROUPS * (BR_UNROLL - 1) < nrb; rb += BR_GROUPS * BR_UNROLL) {
            float v[BR_UNROLL];
#pragma unroll
            for (int u = 0; u < BR_UNROLL; u++) v[u] = bpart[(long)(rb + BR_GROUPS * u) * cols + c];
#pragma unroll
            for (int u = 0; u < BR_UNROLL; u++) s += v[u];
        }
        for (; rb < nrb; rb += BR_GROUPS) s += bpart[(long)rb * cols + c];
    }
    part[q][cl] = s;
    __syncthreads();
    if (q == 0 && c < cols) {
        float t = part[0][cl];
#pragma unroll
        for (int j = 1; j < BR_GROUPS; j++) t += part[j][cl];
        db[c] += t;
    }
}

__global__ void cast_flat_kernel(uint2* xb, const float4* x, size_t n4) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const float4 v = x[i];
        xb[i] = make_uint2(bf16_pack2(v.x, v.y), bf16_pack2(v.z, v.w));
    }
}

bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

long pad64(long n) { return (n + TILE - 1) / TILE * TILE; }

template <bool XENT>
hipError_t launch_cast(const CastArgs& a, const XentArgs& xa, hipStream_t st, const char* name) {
    if (a.rows < 0 || a.cols < 0 || a.cols % 4 || a.ldx % 4 || a.ldx < a.cols || a.batch < 1 || !a.x || !a16(a.x))
        return hipErrorInvalidValue;
    if (a.xb && (a.ldb % 8 || a.ldb < a.cols || !a16(a.xb))) return hipErrorInvalidValue;
    if (a.xt && (a.ldt % 8 || a.ldt < pad64(a.rows) || !a16(a.xt))) return hipErrorInvalidValue;
    if (a.rows == 0 || a.cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.cols + TILE - 1) / TILE), (unsigned)((pad64(a.rows) + RB - 1) / RB), (unsigned)a.batch);
    const double n = (double)a.rows * a.cols * a.batch;
    ProfScope ps(st, name, 0.0, n * (4.0 + (a.xb ? 2.0 : 0.0) + (a.xt ? 2.0 : 0.0)));
    hipLaunchKernelGGL((cast_tile_kernel<XENT>), grid, dim3(CT_THREADS), 0, st, a, xa);
    return hipGetLastError();
}

}  // namespace

size_t bias_partial_floats(int rows, int cols) { return (size_t)((rows + RB - 1) / RB) * (size_t)cols; }

hipError_t cast_bf16(const CastArgs& a, hipStream_t st) {
    return launch_cast<false>(a, XentArgs{nullptr, nullptr, 0.f, 0}, st, "cast_tile_kernel<false>");
}

hipError_t bias_reduce(float* db, const float* bpart, int rows, int cols, hipStream_t st) {
    return bias_reduce_parts(db, bpart, (rows + RB - 1) / RB, cols, st);
}

hipError_t bias_reduce_parts(float* db, const float* bpart, int nrb, int cols, hipStream_t st) {
    if (nrb <= 0 || cols <= 0) return hipSuccess;
    ProfScope ps(st, "bias_reduce_kernel", 0.0, 4.0 * ((double)nrb * cols + 2.0 * cols));
    hipLaunchKernelGGL(bias_reduce_kernel, dim3((cols + TILE - 1) / TILE), dim3(TILE * BR_GROUPS), 0, st, db, bpart,
                       nrb, cols);
    return hipGetLastError();
}

hipError_t cast_bf16_flat(uint16_t* xb, const float* x, size_t n, hipStream_t st) {
    if (n % 4 || !a16(x) || ((uintptr_t)xb & 7)) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    const size_t n4 = n / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 4096);
    ProfScope ps(st, "cast_flat_kernel", 0.0, 6.0 * (double)n);
    hipLaunchKernelGGL(cast_flat_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<uint2*>(xb),
                       reinterpret_cast<const float4*>(x), n4);
    return hipGetLastError();
}

hipError_t xent_grad_bf16(uint16_t* db, const float* logits, long Vp, const float* lse, const int32_t* targets,
                          float scale, int N, int V, hipStream_t st) {
    if (Vp < V || Vp % 64 || !lse || !targets) return hipErrorInvalidValue;
    CastArgs a{};
    a.x = logits;
    a.ldx = Vp;
    a.xb = db;
    a.ldb = Vp;
    a.rows = N;
    a.cols = (int)Vp;
    a.batch = 1;
    return launch_cast<true>(a, XentArgs{lse, targets, scale, V}, st, "cast_tile_kernel<true>");
}

}  // namespace gpt2k
