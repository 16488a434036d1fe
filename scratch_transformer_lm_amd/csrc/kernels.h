// Host-side launchers of the gfx950 kernels (internal to the library).
// All launchers enqueue on `st` and return the launch status; none synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace gpt2k {

// ---- linear layers (gemm.hip) -------------------------------------------------------
// `partial` is a scratch of gemm_partial_floats() floats for split partial tiles
// (nullptr: one tile per block, no sharing of tiles).  Operands must be 16-byte aligned
// with leading dimensions that are multiples of 4 floats.
size_t gemm_partial_floats();
// Tile width of the forward and dgrad GEMMs (process-wide; set it between launches, not
// while other host threads launch): automatic (96 where that gives whole rounds of
// resident blocks), or forced to 128 or 96 columns.  False for an unknown value.
enum { GEMM_TILES_AUTO = 0, GEMM_TILES_128 = 1, GEMM_TILES_96 = 2 };
bool gemm_set_tile_policy(int policy);
// out[M,N] (ld ldo) = inp[M,K] . w[N,K]^T, then by the non-null extras:
//   bias: + bias[n];  resid: out = resid + (...) (resid has ld ldo);
//   pre:  pre = (...) and out = gelu(pre) (pre has ld ldo).
//   lse_part (no bias/resid/pre): also the per-row log-sum-exp partials of out, for
//   lse_combine; it holds lse_partial_floats(M, N) floats.
hipError_t linear_forward(float* out, long ldo, const float* inp, const float* w,
                          const float* bias, const float* resid, float* pre, int M, int N, int K,
                          float* partial, hipStream_t st, float* lse_part = nullptr);
size_t lse_partial_floats(int M, int N);
// Marks a `dout` operand as logits whose gradient is formed while loading:
// dlogit = (exp(z - lse[row]) - [col == targets[row]]) * scale.  The logits' padding
// columns (up to the leading dimension) must be readable; their values are not used.
// linear_dgrad applies both terms; linear_wgrad only the softmax term, leaving
// dw[targets[row]] -= scale * inp[row] to the caller (embedding_scatter).
struct XentOperand {
    const float* lse;
    const int32_t* targets;
    float scale;
};
// din[M,N] = dout[M,K] (ld ld_dout) . w[K,N]; with gelu_pre: din *= gelu'(gelu_pre[M,N]).
hipError_t linear_dgrad(float* din, const float* dout, long ld_dout, const float* w,
                        const float* gelu_pre, int M, int N, int K, float* partial, hipStream_t st,
                        const XentOperand* xent = nullptr);
// dw[M,N] += dout[K,M]^T (dout ld ld_dout) . inp[K,N]; dbias (optional) += column sums of
// dout over its K rows.  M must be a multiple of 4 unless dout is a logits operand.
hipError_t linear_wgrad(float* dw, float* dbias, const float* dout, long ld_dout, const float* inp, int M,
                        int N, int K, float* partial, hipStream_t st, const XentOperand* xent = nullptr);

// Mixed precision: C[M,N] (ld ldc, fp32) = A[M,K] . B[N,K]^T with both operands bfloat16
// bit patterns, k-contiguous (leading dimensions lda, ldb multiples of 8, K even; pad
// columns of a padded K must be zero), products summed in fp32, then the epilogue:
//   BF16_STORE: C = .;  BF16_BIAS: C = . + bias;  BF16_BIAS_RESID: C = aux + (. + bias);
//   BF16_BIAS_GELU: pre = . + bias, C = gelu(pre);  BF16_ACCUM: C += .;
//   BF16_GELU_BWD: C = . * gelu'(aux).   aux has leading dimension ldaux, pre ldc.
enum { BF16_STORE = 0, BF16_BIAS, BF16_BIAS_RESID, BF16_BIAS_GELU, BF16_ACCUM, BF16_GELU_BWD };
// lse_part with BF16_STORE: the log-sum-exp partials as linear_forward's.  cb with
// BF16_BIAS_GELU or BF16_GELU_BWD: the bf16 rounding of C as well (leading dimension ldcb;
// N, ldcb even, cb 4-byte aligned).  csum with BF16_GELU_BWD: the column sums of C per
// 16-row slice, ceil(M/16) rows of N floats (bias_reduce_parts adds them).
hipError_t gemm_bf16(int epi, float* c, long ldc, const uint16_t* a, long lda, const uint16_t* b, long ldb, int M,
                     int N, int K, const float* bias, const float* aux, long ldaux, float* pre, float* partial,
                     hipStream_t st, float* lse_part = nullptr, uint16_t* cb = nullptr, long ldcb = 0,
                     float* csum = nullptr);
// C[M,N] += sum over k of A[k,m] B[k,n] with bfloat16 A, B stored row-contiguous, as
// [K][lda] and [K][ldb] (the weight gradients dW += dY^T X on the straight copies of dY and
// X): lda >= M, ldb >= N, both multiples of 8; 16-byte aligned; the elements of a row past
// M (N) are read but feed no stored output.
hipError_t gemm_bf16_rows(float* c, long ldc, const uint16_t* a, long lda, const uint16_t* b, long ldb, int M, int N,
                          int K, float* partial, hipStream_t st);

// ---- bfloat16 operand copies (bf16.hip) -----------------------------------------------
// Rounding is to nearest, ties to even.  x is (rows, cols) fp32 with leading dimension
// ldx (a multiple of 4); batch copies at strides sx / sb / st (elements) of x / xb / xt.
//   xb (optional): (rows, cols) bf16, leading dimension ldb (a multiple of 8).
//   xt (optional): the transpose (cols, rows_pad) bf16, leading dimension ldt >= rows_pad,
//     rows_pad = rows rounded up to 64, columns rows..rows_pad-1 zero.
//   bpart (optional): per 128-row block rb, bpart[rb * cols + c] = sum of x[r, c] over its
//     rows in order; bias_reduce then adds them into db in block order.
// cols must be a multiple of 4.
struct CastArgs {
    const float* x;
    long ldx;
    uint16_t* xb;
    long ldb;
    uint16_t* xt;
    long ldt;
    float* bpart;
    int rows, cols;
    int batch;
    long sx, sb, st;
};
hipError_t cast_bf16(const CastArgs& a, hipStream_t st);
size_t bias_partial_floats(int rows, int cols);
hipError_t bias_reduce(float* db, const float* bpart, int rows, int cols, hipStream_t st);
// db[c] += sum over p < nparts of bpart[p * cols + c], in a fixed order
hipError_t bias_reduce_parts(float* db, const float* bpart, int nparts, int cols, hipStream_t st);
// Flat copy: xb[i] = bf16(x[i]), n a multiple of 4.
hipError_t cast_bf16_flat(uint16_t* xb, const float* x, size_t n, hipStream_t st);
// The LM head's output gradient in bf16: d[r, c] = (exp(z[r, c] - lse[r]) - [c == targets[r]]) * scale for
// c < V, 0 for V <= c < Vp, written row-major (N, Vp) to db.  logits has leading dimension Vp.
hipError_t xent_grad_bf16(uint16_t* db, const float* logits, long Vp, const float* lse, const int32_t* targets,
                          float scale, int N, int V, hipStream_t st);

// ---- LayerNorm (norm.hip) -----------------------------------------------------------
// yb (nullable, 8-byte aligned): the bf16 rounding of y, same layout.
hipError_t layernorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w,
                             const float* b, int N, int C, float eps, hipStream_t st, uint16_t* yb = nullptr);
// dx (+)= ..., dw/db (+)= ...; accumulate flags choose += or =.  partial needs
// layernorm_partial_floats(N, C) floats.
size_t layernorm_partial_floats(int N, int C);
// st_red (with ev): the dw/db reduction of the partial rows runs on that stream after ev,
// recorded on st once the partial rows are written (the caller keeps partial untouched
// until st_red has run it).
hipError_t layernorm_backward(float* dx, float* dw, float* db, const float* dy, const float* x,
                              const float* w, const float* mean, const float* rstd, int N, int C,
                              bool accumulate_dx, bool accumulate_dwdb, float* partial,
                              hipStream_t st, hipStream_t st_red = nullptr, hipEvent_t ev = nullptr);
// RMSNorm (no mean subtraction, no bias): y = x r w, r = 1/sqrt(mean(x^2) + eps); mean[]
// is written as 0 so the LayerNorm activation layout still holds.  The backward adds
// only dw (same partial scratch as layernorm_backward, at most that size).
hipError_t rmsnorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w, int N, int C,
                           float eps, hipStream_t st, uint16_t* yb = nullptr);
hipError_t rmsnorm_backward(float* dx, float* dw, const float* dy, const float* x, const float* w,
                            const float* mean, const float* rstd, int N, int C, bool accumulate_dx,
                            bool accumulate_dw, float* partial, hipStream_t st, hipStream_t st_red = nullptr,
                            hipEvent_t ev = nullptr);

// ---- embedding (encoder.hip) --------------------------------------------------------
// out[b,t] = wte[tok[b,t]] + wpe[t]; wpe may be null (no position rows).
hipError_t encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe,
                           int B, int T, int C, int V, int* flags, hipStream_t st);
// Backward scatter-adds into wte, deterministic (each token's rows added in position
// order).  `work` is an int scratch of encoder_backward_work_ints(n) entries per list.
size_t encoder_backward_work_ints(long BT);
// Lists of up to 32768 positions with V <= 65536 go through a one-block sort.
bool embedding_sortable(int n, int V);
// Sorts the (token, position) pairs of tok0 (and of tok1 unless null) into work0 (work1),
// one launch; ids outside [0, V) are dropped.
hipError_t sort_token_lists(int* work0, const int32_t* tok0, int* work1, const int32_t* tok1, int n, int V,
                            hipStream_t st);
// dwte[token] += scale * src[position] (row stride ld) over a list sorted as above.
hipError_t scatter_sorted(float* dwte, int C, const float* src, long ld, float scale, const int* work, int n,
                          hipStream_t st);
// The same for a list of any size (sorts first, or falls back to a first-occurrence scan).
hipError_t embedding_scatter(float* dwte, int V, int C, const int32_t* tok, int n, const float* src, long ld,
                             float scale, int* work, hipStream_t st);
// dwpe[t] += sum over b of dout[b, t].
hipError_t wpe_backward(float* dwpe, const float* dout, int B, int T, int C, hipStream_t st);

// ---- attention (attention.hip) ------------------------------------------------------
// qkv (B,T,3C) -> out (B,T,C), lse (B,NH,T).
// sbuf (nullable, 16-byte aligned, attn_ds_floats(B, T, NH) floats): also store the raw
// scores q.k of every causal tile pair for the backward.
hipError_t attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                             hipStream_t st, float* sbuf = nullptr);
// dout (B,T,C) -> dqkv (B,T,3C) (overwritten); delta needs B*NH*T floats.  With ds (16-byte
// aligned, attn_ds_floats(B, T, NH) floats) the dK/dV kernel stores the score gradients
// and dQ is their product with K; without it dQ recomputes them.  With ds and sbuf (the
// raw scores the forward stored) the dK/dV kernel reads S instead of forming Q K^T.
size_t attn_ds_floats(int B, int T, int NH);
hipError_t attention_backward(float* dqkv, float* delta, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C, int NH,
                              hipStream_t st, float* ds = nullptr, const float* sbuf = nullptr);

// ---- attention of the mixed-precision variant (attention_bf16.hip) ------------------
// bf16 copies of each head, per (batch, head): row-major (T, HS) and transposed (HS, Tp)
// with the tokens of every 64-token tile permuted (Tp = T rounded up to 64, zero beyond
// T); attn_bf16_head_elems(B, T, C) bf16 elements hold one transposed tensor.
size_t attn_bf16_head_elems(int B, int T, int C);
// Copies of nsrc fp32 (B, T, ld) tensors src + z*zoff (head h at columns h*HS) into
// rm[z] and tr[z] (either may be null).  HS = C/NH must be 16, 32 or 64.
hipError_t attn_prep_bf16(const float* src, long ld, long zoff, int nsrc, uint16_t* const* rm, uint16_t* const* tr,
                          int B, int T, int C, int NH, hipStream_t st);
struct AttnBf16 {
    const uint16_t *q, *k, *v;     // row-major copies
    const uint16_t *qt, *kt, *vt;  // transposed copies
};
// out (B,T,C) fp32 and lse (B,NH,T) from bf16 q, k, vt (the probabilities unrounded);
// outb (nullable, 4-byte aligned): the bf16 rounding of out, same layout.
hipError_t attention_forward_bf16(float* out, uint16_t* outb, float* lse, const AttnBf16& a, int B, int T, int C,
                                  int NH, hipStream_t st);
// dqkv (B,T,3C) fp32 (overwritten) from bf16 dO (row-major dob, transposed dot), the fp32
// output `out`, lse, and q, k, v, qt, kt; delta needs B*NH*T floats.  Optional: dqkvb
// (4-byte aligned) gets the bf16 rounding of dqkv, same layout; bsum the column sums of
// dqkv per 64-row tile of each sequence, attn_bias_partial_rows(B, T) rows of 3C floats in
// (b, tile) order (bias_reduce_parts adds them).
hipError_t attention_backward_bf16(float* dqkv, uint16_t* dqkvb, float* bsum, float* delta, const uint16_t* dob,
                                   const uint16_t* dot, const float* out, const float* lse, const AttnBf16& a, int B,
                                   int T, int C, int NH, hipStream_t st);
size_t attn_bias_partial_floats(int B, int T, int C);
int attn_bias_partial_rows(int B, int T);

// ---- rotary positions (rope.hip) ------------------------------------------------------
// table: rope_table_floats(maxT, hs) floats of (cos, sin) pairs, filled by rope_table.
// rope_forward rotates q and k of qkv (B, T, 3C) in place; rope_backward applies the
// transpose to dq and dk of dqkv in place.  hs = C/NH must be even.
size_t rope_table_floats(int maxT, int hs);
hipError_t rope_table(float* table, int maxT, int hs, hipStream_t st);
hipError_t rope_forward(float* qkv, const float* table, int B, int T, int C, int NH, hipStream_t st);
hipError_t rope_backward(float* dqkv, const float* table, int B, int T, int C, int NH, hipStream_t st);

// ---- softmax + cross-entropy (softmax_xent.hip) -------------------------------------
// Per logits row (ld): lse = log sum exp and, when targets != NULL, loss = lse - z[target],
// from the partials an LSE-fused LM-head forward wrote (`parts` pairs per row,
// lse_partial_count of its shape and arithmetic); a target outside [0, V) sets
// ERR_BAD_TARGET_TOKEN in flags and a NaN loss.
int lse_partial_count(int M, int N, bool bf16);
hipError_t lse_combine(const float* lse_part, int parts, const float* logits, long ld, float* lse, float* losses,
                       const int32_t* targets, int N, int V, int* flags, hipStream_t st);
// Mean of losses[0..N) in double, written as float to *out.
hipError_t loss_mean(float* out, const float* losses, int N, hipStream_t st);
// tokens[i] = the sampled next token at logits row rows[i] for coins[i] in [0,1):
// the smallest j with coin < sum_{k<=j} exp(z_k - lse[row]) (V-1 if none).  Device
// arrays; rows must be valid rows of the last forward.
hipError_t sample_tokens(const float* logits, long ld, const float* lse, const int32_t* rows, const float* coins,
                         int n, int V, int32_t* tokens, hipStream_t st);

// ---- optimizer and fills (adamw.hip) ------------------------------------------------
hipError_t adamw(float* p, const float* g, float* m, float* v, size_t n, float lr, float b1,
                 float b2, float eps, float wd, float bc1, float bc2, hipStream_t st);
// AdamW over n <= ADAM_MAX_SEGS disjoint slices [off[i], off[i] + len[i]) of the flat
// buffers (offsets and lengths multiples of 4 floats): bitwise the update adamw gives
// those elements.
constexpr int ADAM_MAX_SEGS = 16;
struct AdamSegments {
    int n;
    size_t off4[ADAM_MAX_SEGS];    // first float4 of each slice
    size_t len4[ADAM_MAX_SEGS];    // float4s of each slice
    size_t start4[ADAM_MAX_SEGS + 1];  // first tile of each slice (tiles of the kernel's width)
};
hipError_t adamw_segments(float* p, const float* g, float* m, float* v, const size_t* off, const size_t* len, int n,
                          float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t st);
hipError_t fill_zero(float* x, size_t n, hipStream_t st);

}  // namespace gpt2k
