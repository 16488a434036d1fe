// Token + position embedding, forward and backward, for gfx950.
//
// The pages name the layer (encoder_forward / encoder_backward: huxiu page
// "llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读 item 1): out = wte[token] + wpe[t].
// The backward is a scatter-add into the wte rows that were read.  Token frequencies
// are skewed (a few ids fill a large share of the positions), so instead of float
// atomics, which would serialise on the hot rows and make the sums order-dependent,
// one block sorts the (token, position) pairs in LDS (bitonic sort of 32-bit keys
// token << 16 | position, so equal tokens keep position order) and cuts the sorted list
// into one segment per distinct token; then one block per segment adds that token's
// rows in position order.  Results are therefore bitwise reproducible.  Batches too large
// for the one-block sort fall back to a first-occurrence scan: one block per distinct
// token walks all later positions.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace gpt2k {

namespace {

constexpr int STAGE = 4096;       // tokens staged in LDS per pass (fallback path)
constexpr int SORT_MAX = 32768;   // (token, position) keys one block sorts in LDS (128 KB)
constexpr int SORT_NT = 1024;

int pow2_at_least(int n) {
    int p = 2;
    while (p < n) p <<= 1;
    return p;
}

__global__ __launch_bounds__(256) void encoder_fwd_kernel(float* __restrict__ out, const int32_t* __restrict__ tok,
                                                          const float* __restrict__ wte, const float* __restrict__ wpe,
                                                          int BT, int T, int C, int V, int* flags) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= BT) return;
    int id = tok[row];
    if (id < 0 || id >= V) {
        if (lane == 0) atomicOr(flags, ERR_BAD_INPUT_TOKEN);
        id = 0;
    }
    const int t = row % T;
    const float4* we = reinterpret_cast<const float4*>(wte + (long)id * C);
    float4* o = reinterpret_cast<float4*>(out + (long)row * C);
    if (!wpe) {  // no position rows (the rotary variant puts positions into q and k)
        for (int i = lane; i < C / 4; i += 64) o[i] = we[i];
        return;
    }
    const float4* pe = reinterpret_cast<const float4*>(wpe + (long)t * C);
    for (int i = lane; i < C / 4; i += 64) {
        const float4 a = we[i], b = pe[i];
        o[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
}

// dwpe[t] += sum_b dout[b, t] (b in order); one thread per 4 channels of one t.
__global__ __launch_bounds__(256) void wpe_bwd_kernel(float* __restrict__ dwpe, const float* __restrict__ dout,
                                                      int B, int T, int C) {
    const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
    const int C4 = C / 4;
    if (i >= (long)T * C4) return;
    const int t = (int)(i / C4), c4 = (int)(i - (long)t * C4);
    float4 acc = reinterpret_cast<float4*>(dwpe + (long)t * C)[c4];
    for (int b = 0; b < B; b++) {
        const float4 d = reinterpret_cast<const float4*>(dout + ((long)b * T + t) * C)[c4];
        acc.x += d.x;
        acc.y += d.y;
        acc.z += d.z;
        acc.w += d.w;
    }
    reinterpret_cast<float4*>(dwpe + (long)t * C)[c4] = acc;
}

// For each position p, is it the first position holding its token id?  Such positions
// are appended to list (slot order does not matter: each one is processed alone); ids
// outside [0, V) are never listed.  work[0] is the list length and must be 0 on entry.
__global__ __launch_bounds__(256) void first_occurrence_kernel(int* work, const int32_t* __restrict__ tok, int BT,
                                                               int V) {
    __shared__ int s[STAGE];
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    const int v = p < BT ? tok[p] : -1;
    const int pmax = min(BT, (int)((blockIdx.x + 1) * blockDim.x));
    int found = 0;
    for (int base = 0; base < pmax; base += STAGE) {
        const int n = min(STAGE, pmax - base);
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += blockDim.x) s[i] = tok[base + i];
        __syncthreads();
        const int lim = min(n, p - base);
        for (int i = 0; i < lim; i++) found |= (s[i] == v);
    }
    if (p < BT && !found && v >= 0 && v < V) {
        const int slot = atomicAdd(work, 1);
        work[1 + slot] = p;
    }
}

// Block k owns the k-th listed first position p: dwte[tok[p]] += scale * (sum of src[q]
// over q >= p with the same id, q increasing).
__global__ __launch_bounds__(256) void wte_bwd_kernel(float* __restrict__ dwte, const float* __restrict__ src, long ld,
                                                      float scale, const int32_t* __restrict__ tok,
                                                      const int* __restrict__ work, int BT, int C) {
    __shared__ unsigned long long masks[4];
    if ((int)blockIdx.x >= work[0]) return;
    const int p = work[1 + blockIdx.x];
    const int v = tok[p];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int C4 = C / 4;
    float4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = p; base < BT; base += 256) {
        const int q = base + threadIdx.x;
        const bool hit = q < BT && tok[q] == v;
        const unsigned long long m = __ballot(hit);
        if (lane == 0) masks[wave] = m;
        __syncthreads();
        for (int w = 0; w < 4; w++) {
            unsigned long long mm = masks[w];
            while (mm) {
                const int bit = __ffsll((long long)mm) - 1;
                mm &= mm - 1;
                const float4* row = reinterpret_cast<const float4*>(src + (long)(base + w * 64 + bit) * ld);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int c = threadIdx.x + 256 * j;
                    if (c < C4) {
                        const float4 d = row[c];
                        acc[j].x += d.x;
                        acc[j].y += d.y;
                        acc[j].z += d.z;
                        acc[j].w += d.w;
                    }
                }
            }
        }
        __syncthreads();
    }
    float4* dst = reinterpret_cast<float4*>(dwte + (long)v * C);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int c = threadIdx.x + 256 * j;
        if (c < C4) {
            float4 o = dst[c];
            o.x += scale * acc[j].x;
            o.y += scale * acc[j].y;
            o.z += scale * acc[j].z;
            o.w += scale * acc[j].w;
            dst[c] = o;
        }
    }
}

__global__ void zero_int_kernel(int* x) { *x = 0; }

// One block: sorts keys token << 16 | position for the n positions (ids outside [0, V)
// sort last and are dropped), then lists the start of every run of equal tokens.
// work: [0] run count, [1, 1+np) sorted keys, [1+np, ...) run starts, then the end of the
// last run.
// Block b sorts list b (work_b, tok_b).
__global__ __launch_bounds__(SORT_NT) void sort_tokens_kernel(int* __restrict__ work0, const int32_t* __restrict__ tok0,
                                                              int* __restrict__ work1, const int32_t* __restrict__ tok1,
                                                              int n, int np, int V) {
    __shared__ unsigned keys[SORT_MAX];
    int* work = blockIdx.x == 0 ? work0 : work1;
    const int32_t* tok = blockIdx.x == 0 ? tok0 : tok1;
    __shared__ int wsum[SORT_NT / 64];
    const int tid = threadIdx.x;
    for (int i = tid; i < np; i += SORT_NT) {
        unsigned k = 0xFFFFFFFFu;
        if (i < n) {
            const int v = tok[i];
            if (v >= 0 && v < V) k = ((unsigned)v << 16) | (unsigned)i;
        }
        keys[i] = k;
    }
    __syncthreads();
    // bitonic sort, ascending: pass (size, stride) compares i and i + stride for every i
    // whose stride bit is clear, in the direction of bit `size` of i
    for (int size = 2; size <= np; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < np / 2; i += SORT_NT) {
                const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                const unsigned a = keys[lo], b = keys[hi];
                if ((a > b) == ((lo & size) == 0)) {
                    keys[lo] = b;
                    keys[hi] = a;
                }
            }
            __syncthreads();
        }
    // run starts, compacted in order: thread t owns keys [t*per, (t+1)*per)
    const int per = np / SORT_NT > 0 ? np / SORT_NT : 1;
    const int j0 = tid * per, j1 = min(np, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; j++)
        cnt += keys[j] != 0xFFFFFFFFu && (j == 0 || (keys[j] >> 16) != (keys[j - 1] >> 16));
    // exclusive scan of cnt over the block
    const int lane = tid & 63, wv = tid >> 6;
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wv; w++) off += wsum[w];
    int at = off + incl - cnt;
    int* runs = work + 1 + np;
    for (int j = j0; j < j1; j++)
        if (keys[j] != 0xFFFFFFFFu && (j == 0 || (keys[j] >> 16) != (keys[j - 1] >> 16))) runs[at++] = j;
    unsigned* out = reinterpret_cast<unsigned*>(work + 1);
    for (int i = tid; i < np; i += SORT_NT) out[i] = keys[i];
    if (tid == SORT_NT - 1) {
        int total = 0;
        for (int w = 0; w < SORT_NT / 64; w++) total += wsum[w];
        work[0] = total;
        // end of the last run: the number of valid keys
        int valid = np;
        while (valid > 0 && keys[valid - 1] == 0xFFFFFFFFu) valid--;
        runs[total] = valid;
    }
}

// Block r < run count owns run r of the sorted keys: dst[token] += scale * (sum of the
// run's source rows).  The block's G = blockDim / (C/4) thread groups each add every G-th
// row of the run in order, and the G partial sums are then added in group order, so the
// result is the same on every run.  The run's row ids are first copied into LDS (in
// chunks of SCATTER_CHUNK), so that a group's loads depend on no other load, and each
// thread keeps SCATTER_AHEAD rows in flight: the longest run (the most frequent token,
// hundreds of rows) is then a few memory latencies, not one per 8 rows and id fetch.
constexpr int SCATTER_NT = 1024, SCATTER_CHUNK = 4096, SCATTER_AHEAD = 16;
__global__ __launch_bounds__(SCATTER_NT) void scatter_rows_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                                  long ld, int C, float scale,
                                                                  const int* __restrict__ work, int np) {
    __shared__ float4 part[SCATTER_NT];
    __shared__ int rid[SCATTER_CHUNK];
    const int nrun = work[0];
    const unsigned* keys = reinterpret_cast<const unsigned*>(work + 1);
    const int* runs = work + 1 + np;
    const int C4 = C / 4, G = SCATTER_NT / C4;
    const int g = threadIdx.x / C4, c4 = threadIdx.x - g * C4;
    for (int r = blockIdx.x; r < nrun; r += gridDim.x) {
        const int j0 = runs[r], j1 = runs[r + 1];
        const int v = (int)(keys[j0] >> 16);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int cs = j0; cs < j1; cs += SCATTER_CHUNK) {
            const int ce = min(cs + SCATTER_CHUNK, j1);
            __syncthreads();  // the previous chunk's ids (or run) are no longer read
            for (int i = threadIdx.x; i < ce - cs; i += SCATTER_NT) rid[i] = (int)(keys[cs + i] & 0xFFFFu);
            __syncthreads();
            if (g < G) {
                // this group's rows are j0 + g + kG; the first one in [cs, ce)
                int j = cs + (g - (cs - j0) % G + G) % G;
                for (; j + (SCATTER_AHEAD - 1) * G < ce; j += SCATTER_AHEAD * G) {
                    float4 d[SCATTER_AHEAD];
#pragma unroll
                    for (int u = 0; u < SCATTER_AHEAD; u++)
                        d[u] = reinterpret_cast<const float4*>(src + (long)rid[j - cs + u * G] * ld)[c4];
#pragma unroll
                    for (int u = 0; u < SCATTER_AHEAD; u++) {
                        acc.x += d[u].x;
                        acc.y += d[u].y;
                        acc.z += d[u].z;
                        acc.w += d[u].w;
                    }
                }
                for (; j < ce; j += G) {
                    const float4 d = reinterpret_cast<const float4*>(src + (long)rid[j - cs] * ld)[c4];
                    acc.x += d.x;
                    acc.y += d.y;
                    acc.z += d.z;
                    acc.w += d.w;
                }
            }
        }
        if (g < G) part[threadIdx.x] = acc;
        __syncthreads();
        if (g == 0) {
            float4 t = part[c4];
            for (int h = 1; h < G; h++) {
                const float4 q = part[h * C4 + c4];
                t.x += q.x;
                t.y += q.y;
                t.z += q.z;
                t.w += q.w;
            }
            float4* o = reinterpret_cast<float4*>(dst + (long)v * C) + c4;
            float4 w = *o;
            w.x += scale * t.x;
            w.y += scale * t.y;
            w.z += scale * t.z;
            w.w += scale * t.w;
            *o = w;
        }
    }
}

}  // namespace

hipError_t encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe,
                           int B, int T, int C, int V, int* flags, hipStream_t st) {
    const int BT = B * T;
    if (C % 4) return hipErrorInvalidValue;
    if (BT == 0) return hipSuccess;
    ProfScope ps(st, "encoder_fwd_kernel", 0.0, 4.0 * ((double)BT * C * 3 + BT));
    hipLaunchKernelGGL(encoder_fwd_kernel, dim3((BT + 3) / 4), dim3(256), 0, st, out, tok, wte, wpe, BT, T, C, V, flags);
    return hipGetLastError();
}

size_t encoder_backward_work_ints(long BT) {
    if (BT <= SORT_MAX) return 2 + 2 * (size_t)pow2_at_least((int)std::max<long>(BT, 2));
    return 1 + (size_t)BT;
}

bool embedding_sortable(int n, int V) { return n <= SORT_MAX && V <= 65536; }

hipError_t sort_token_lists(int* work0, const int32_t* tok0, int* work1, const int32_t* tok1, int n, int V,
                            hipStream_t st) {
    if (!embedding_sortable(n, V)) return hipErrorInvalidValue;
    if (n <= 0) return hipSuccess;
    const int np = pow2_at_least(n);
    const int lists = tok1 ? 2 : 1;
    ProfScope ps(st, "sort_tokens_kernel", 0.0, 4.0 * lists * (n + 2.0 * np));
    hipLaunchKernelGGL(sort_tokens_kernel, dim3(lists), dim3(SORT_NT), 0, st, work0, tok0, work1, tok1, n, np, V);
    return hipGetLastError();
}

hipError_t scatter_sorted(float* dwte, int C, const float* src, long ld, float scale, const int* work, int n,
                          hipStream_t st) {
    if (C % 4 || ld % 4 || C > 4 * SCATTER_NT) return hipErrorInvalidValue;
    if (n <= 0) return hipSuccess;
    // rows read once; each touched wte row read and written once
    ProfScope ps(st, "scatter_rows_kernel", 0.0, 4.0 * ((double)n * C + 2.0 * (double)n * C));
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)std::min(n, 2048)), dim3(SCATTER_NT), 0, st, dwte, src, ld,
                       C, scale, work, pow2_at_least(n));
    return hipGetLastError();
}

hipError_t embedding_scatter(float* dwte, int V, int C, const int32_t* tok, int n, const float* src, long ld,
                             float scale, int* work, hipStream_t st) {
    if (C % 4 || ld % 4 || C > 4096) return hipErrorInvalidValue;
    if (n <= 0) return hipSuccess;
    if (embedding_sortable(n, V)) {
        hipError_t e = sort_token_lists(work, tok, nullptr, nullptr, n, V, st);
        if (e != hipSuccess) return e;
        return scatter_sorted(dwte, C, src, ld, scale, work, n, st);
    }
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, work);
    {
        ProfScope ps(st, "first_occurrence_kernel", 0.0, 4.0 * n);
        hipLaunchKernelGGL(first_occurrence_kernel, dim3((n + 255) / 256), dim3(256), 0, st, work, tok, n, V);
    }
    // rows of src read once; each touched wte row read and written once (at most n rows)
    ProfScope ps(st, "wte_bwd_kernel", 0.0, 4.0 * ((double)n * C + n));
    hipLaunchKernelGGL(wte_bwd_kernel, dim3(n), dim3(256), 0, st, dwte, src, ld, scale, tok, (const int*)work, n, C);
    return hipGetLastError();
}

hipError_t wpe_backward(float* dwpe, const float* dout, int B, int T, int C, hipStream_t st) {
    if (C % 4) return hipErrorInvalidValue;
    const long n = (long)T * (C / 4);
    if ((long)B * T == 0) return hipSuccess;
    ProfScope ps(st, "wpe_bwd_kernel", 0.0, 4.0 * ((double)B * T * C + 2.0 * T * C));
    hipLaunchKernelGGL(wpe_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dwpe, dout, B, T, C);
    return hipGetLastError();
}

}  // namespace gpt2k
