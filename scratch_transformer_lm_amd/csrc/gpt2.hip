// The C ABI of the GPT-2 fp32 training step: parameter layout, arena carving and the
// order of kernel launches for forward, zero_grad, backward and update.
//
// Structure follows the pages' train_gpt2.c walk-through (huxiu page "llm.c：Andrej
// Karpathy带你从零复现LLM", 核心代码解读): GPT2Config, ParameterTensors in one flat
// buffer, ActivationTensors in one flat arena carved once ("OpenAI创始大神手搓千行C代码
// 训练GPT", 手动实现每个层前向 / 反向传播), and the calls forward / zero_grad /
// backward / update.  The block is GPT-2's pre-LayerNorm block:
//   x += attproj(attention(qkv(ln1(x))));  x += fcproj(gelu(fc(ln2(x))))
// followed by a final LayerNorm and the LM head tied to the token embedding (the only
// reading that reproduces the 124,439,808 parameters the pages print).
//
// Differences from the plain layer-by-layer decomposition, none of which changes what
// is computed: residual adds and GELU run in the GEMM epilogues; attention keeps a
// per-row log-sum-exp instead of the two (B,NH,T,T) score tensors and recomputes the
// probabilities in its backward; activation gradients live in a small per-layer
// scratch that each backward rewrites (the residual stream's gradient is one buffer
// that every block adds into), so zero_grad only clears the parameter gradients.
#include <algorithm>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gpt2.h"
#include "common.h"
#include "kernels.h"
#include "prof.h"

using namespace gpt2k;

namespace {

constexpr int NP = GPT2_NUM_PARAM_TENSORS;
constexpr size_t ALIGN = 64;  // floats (256 bytes)

size_t align_up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

enum { P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB, P_LN2W, P_LN2B,
       P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB };

bool config_ok(const gpt2_config* c) {
    if (!c || c->max_seq_len <= 0 || c->vocab_size <= 0 || c->num_layers <= 0 || c->num_heads <= 0 ||
        c->channels <= 0)
        return false;
    if (c->channels % c->num_heads || c->channels % 4 || c->channels > 4096) return false;
    const int hs = c->channels / c->num_heads;
    return hs == 16 || hs == 32 || hs == 64;
}

void param_sizes(const gpt2_config* cfg, size_t len[NP]) {
    const size_t V = cfg->vocab_size, C = cfg->channels, L = cfg->num_layers, maxT = cfg->max_seq_len;
    const size_t s[NP] = {V * C, maxT * C, L * C, L * C, L * 3 * C * C, L * 3 * C, L * C * C, L * C,
                          L * C, L * C, L * 4 * C * C, L * 4 * C, L * C * 4 * C, L * C, C, C};
    for (int i = 0; i < NP; i++) len[i] = s[i];
}

// Where each activation lives: base offset, per-layer stride (0 for whole-model
// tensors), columns and leading dimension; rows are the current B*T (the lse tensor is
// (B, NH, T), stored as B*T rows of NH... see lse_index).
struct ActInfo {
    size_t off, layer_stride, cols, ld;
};

// bfloat16 copies of the mixed-precision variant: in the activation arena the weights as
// stored (W*) and transposed (WT*, (cols, rows rounded up to 64)) and the linear layers'
// inputs (per layer); in the scratch the output gradients (one buffer per kind) and the
// LM head's.  The weight gradients read the inputs and output gradients as they are,
// row-contiguous.  Attention's per-head copies of q, k, v (row-major and transposed, per
// layer) and of its output gradient (scratch) follow.
enum { BW_Q, BW_A, BW_F, BW_P, BW_WTE, BWT_Q, BWT_A, BWT_F, BWT_P, BWT_WTE, BA_LN1, BA_ATTY, BA_LN2, BA_FCHG, BA_LNF,
       BA_HQ, BA_HK, BA_HV, BA_HQT, BA_HKT, BA_HVT, NBA };
enum { BS_DRES, BS_DFCH, BS_DQKV, BS_DLOG, BS_HDO, BS_HDOT, NBS };

size_t pad64(size_t n) { return (n + 63) / 64 * 64; }

// Build option: with the fused backward + update on two backward streams, each layer's
// LayerNorm dw/db reductions run on the update stream (which applies them) instead of the
// main chain, from partial rows of their own (measured at the 124M shape: 54.15-54.28
// against 54.39-54.50 ms per step; 2 L partial-row buffers, 79 MB there).
#ifndef GPT2_LN_REDUCE_ASYNC
#define GPT2_LN_REDUCE_ASYNC 1
#endif
struct Layout {
    size_t BT, Vp;
    ActInfo a[GPT2_NUM_ACTS];
    size_t tok_in, tok_tgt;  // int32 arrays inside acts (offset in 4-byte words)
    size_t n_acts;
    // grad_scratch
    size_t dres, dln, datty, dqkv, dfch, delta, enc_work, enc_work_tgt, partial, n_partial, partial_w, lnpart, sample,
        rope, lsep, attn_ds, n_attn_ds, attn_s, n_scratch;
    // mixed precision: offsets (floats) of the bf16 arrays, per-layer strides (bf16 elements)
    size_t ba[NBA], ba_l[NBA], bs[NBS], bpart;
};

// floats of one output-gradient kind's bias partial sums: per 128-row block (the casts),
// per 64-row tile of each sequence (attention's dqkv) or per 16-row slice (the
// GELU-backward epilogue's dfch)
size_t bias_slot_floats(size_t B, size_t T, size_t C) {
    return std::max({bias_partial_floats((int)(B * T), (int)(4 * C)), attn_bias_partial_floats((int)B, (int)T, (int)C),
                     (B * T + 15) / 16 * 4 * C});
}

// The fp32 attention backward stores the score gradients once (dK/dV kernel) and forms
// dQ from them, instead of recomputing S and dP for dQ (build option; 0: recompute).
#ifndef GPT2_ATTN_DS
#define GPT2_ATTN_DS 1
#endif
// With it, the forward also stores the raw scores of every layer and the dK/dV kernel
// reads them instead of forming Q K^T again (build option; 0: recompute).
#ifndef GPT2_ATTN_S
#define GPT2_ATTN_S 1
#endif

Layout make_layout(const gpt2_config* c, int B, int T, int variant = 0) {
    Layout y{};
    const size_t C = c->channels, L = c->num_layers, NH = c->num_heads, V = c->vocab_size;
    const size_t BT = (size_t)B * T;
    y.BT = BT;
    y.Vp = (V + 63) / 64 * 64;
    size_t o = 0;
    auto put = [&](int id, size_t cols, size_t ld, bool per_layer, size_t rows) {
        const size_t slab = align_up(rows * ld);
        y.a[id] = ActInfo{o, per_layer ? slab : 0, cols, ld};
        o += per_layer ? L * slab : slab;
    };
    put(GPT2_ACT_ENCODED, C, C, false, BT);
    put(GPT2_ACT_LN1, C, C, true, BT);
    put(GPT2_ACT_LN1_MEAN, 1, 1, true, BT);
    put(GPT2_ACT_LN1_RSTD, 1, 1, true, BT);
    put(GPT2_ACT_QKV, 3 * C, 3 * C, true, BT);
    put(GPT2_ACT_ATTY, C, C, true, BT);
    put(GPT2_ACT_ATT_LSE, NH, NH, true, BT);
    put(GPT2_ACT_RESIDUAL2, C, C, true, BT);
    put(GPT2_ACT_LN2, C, C, true, BT);
    put(GPT2_ACT_LN2_MEAN, 1, 1, true, BT);
    put(GPT2_ACT_LN2_RSTD, 1, 1, true, BT);
    put(GPT2_ACT_FCH, 4 * C, 4 * C, true, BT);
    put(GPT2_ACT_FCH_GELU, 4 * C, 4 * C, true, BT);
    put(GPT2_ACT_RESIDUAL3, C, C, true, BT);
    put(GPT2_ACT_LNF, C, C, false, BT);
    put(GPT2_ACT_LNF_MEAN, 1, 1, false, BT);
    put(GPT2_ACT_LNF_RSTD, 1, 1, false, BT);
    put(GPT2_ACT_LOGITS, V, y.Vp, false, BT);
    put(GPT2_ACT_LOGITS_LSE, 1, 1, false, BT);
    put(GPT2_ACT_LOSSES, 1, 1, false, BT);
    y.tok_in = o;
    o += align_up(BT);
    y.tok_tgt = o;
    o += align_up(BT);
    if (variant & GPT2_VARIANT_BF16) {
        const size_t HT = attn_bf16_head_elems(B, T, (int)C);
        // (id, layers, elements per layer)
        const size_t spec[NBA][2] = {
            {L, 3 * C * C}, {L, C * C}, {L, 4 * C * C}, {L, 4 * C * C}, {1, V * C},
            {L, C * pad64(3 * C)}, {L, C * pad64(C)}, {L, C * pad64(4 * C)}, {L, 4 * C * pad64(C)}, {1, C * y.Vp},
            {L, BT * C}, {L, BT * C}, {L, BT * C}, {L, BT * 4 * C}, {1, BT * C},
            {L, BT * C}, {L, BT * C}, {L, BT * C}, {L, HT}, {L, HT}, {L, HT}};
        for (int i = 0; i < NBA; i++) {
            y.ba[i] = o;
            y.ba_l[i] = spec[i][1];
            o += align_up((spec[i][0] * spec[i][1] + 1) / 2);
        }
    }
    y.n_acts = o;

    size_t s = HDR_WORDS;
    auto take = [&](size_t n) {
        const size_t at = s;
        s += align_up(n);
        return at;
    };
    y.dres = take(BT * C);
    y.dln = take(BT * C);
    y.datty = take(BT * C);
    y.dqkv = take(BT * 3 * C);
    y.dfch = take(BT * 4 * C);
    y.delta = take(BT * NH);
    y.enc_work = take(encoder_backward_work_ints((long)BT));      // input tokens
    y.enc_work_tgt = take(encoder_backward_work_ints((long)BT));  // target tokens
    size_t np = gemm_partial_floats();
    np = std::max(np, layernorm_partial_floats((int)BT, (int)C));
    y.n_partial = np;
    y.partial = take(np);
    y.partial_w = take(gemm_partial_floats());  // split tiles of the weight-gradient stream
    // each LayerNorm backward's partial rows (two per layer, then the final norm's), when
    // their dw/db reductions run off the main stream
    y.lnpart = GPT2_LN_REDUCE_ASYNC ? take((2 * L + 1) * layernorm_partial_floats((int)BT, (int)C)) : 0;
    y.sample = take(3 * BT);                      // sampling requests: rows, coins, tokens
    y.rope = take(rope_table_floats(c->max_seq_len, (int)(C / NH)));  // rotary variant's (cos, sin) table
    y.lsep = take(lse_partial_floats((int)BT, (int)V));  // the LM head's per-tile log-sum-exp partials
    // fp32 attention backward: the score gradients of every causal tile pair of one layer
    y.n_attn_ds = (variant & GPT2_VARIANT_BF16) || !GPT2_ATTN_DS ? 0 : attn_ds_floats(B, T, (int)NH);
    y.attn_ds = y.n_attn_ds ? take(y.n_attn_ds) : 0;
    // ... and the raw scores the forward stores for it, one such buffer per layer
    y.attn_s = y.n_attn_ds && GPT2_ATTN_S ? take(L * y.n_attn_ds) : 0;
    if (variant & GPT2_VARIANT_BF16) {
        const size_t n[NBS] = {BT * C, BT * 4 * C, BT * 3 * C, BT * y.Vp, BT * C, attn_bf16_head_elems(B, T, (int)C)};
        for (int i = 0; i < NBS; i++) y.bs[i] = take((n[i] + 1) / 2);
        y.bpart = take(4 * bias_slot_floats(B, T, C));  // one per output-gradient kind
    }
    y.n_scratch = s;
    return y;
}

}  // namespace

struct gpt2 {
    gpt2_config cfg;
    int maxB, maxT;
    int B, T;
    Layout lay;
    hipStream_t st;
    // Backward runs the weight-gradient GEMMs on a second stream of the handle's own,
    // ordered against the main chain by events (see backward_impl).
    hipStream_t st_w;
    hipStream_t st_u;  // per-layer AdamW of gpt2_backward_update
    hipEvent_t ev[14];  // [13]: a LayerNorm backward's partial rows are written
    int backward_streams;  // 2: weight gradients on st_w; 1: everything on st
    int variant;           // GPT2_VARIANT_* bits (Llama-style layers)
    gpt2_buffers buf;
    size_t nparams;
    size_t poff[NP], plen[NP];
    int* host_ret;  // pinned: [loss bits, flags]
    int last_error;
    bool have_forward, have_targets;
    bool scores_stored;  // the last forward stored every layer's raw attention scores
    Profiler* prof;  // non-null while per-kernel timing is enabled
};

namespace {

// Makes the handle's profiler (if any) visible to the launchers for one ABI call.
struct ProfBind {
    explicit ProfBind(gpt2* g) { g_prof = g ? g->prof : nullptr; }
    ~ProfBind() { g_prof = nullptr; }
};

int fail(gpt2* g, int code) {
    if (g) g->last_error = code;
    return code;
}

#define HIPCHK(g, expr)                                    \
    do {                                                   \
        hipError_t e_ = (expr);                            \
        if (e_ != hipSuccess) return fail((g), GPT2_EDEVICE); \
    } while (0)

float* P(gpt2* g, int i) { return g->buf.params + g->poff[i]; }
float* G(gpt2* g, int i) { return g->buf.grads + g->poff[i]; }
float* A(gpt2* g, int id, int l = 0) { return g->buf.acts + g->lay.a[id].off + (size_t)l * g->lay.a[id].layer_stride; }
float* S(gpt2* g, size_t off) { return g->buf.grad_scratch + off; }
int32_t* tok_in(gpt2* g) { return reinterpret_cast<int32_t*>(g->buf.acts + g->lay.tok_in); }
int32_t* tok_tgt(gpt2* g) { return reinterpret_cast<int32_t*>(g->buf.acts + g->lay.tok_tgt); }
int* flags(gpt2* g) { return reinterpret_cast<int*>(g->buf.grad_scratch + HDR_FLAGS); }

bool aligned(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool bf_on(const gpt2* g) { return (g->variant & GPT2_VARIANT_BF16) != 0; }
uint16_t* BA(gpt2* g, int id, int l = 0) {
    return reinterpret_cast<uint16_t*>(g->buf.acts + g->lay.ba[id]) + (size_t)l * g->lay.ba_l[id];
}
uint16_t* BS(gpt2* g, int id) { return reinterpret_cast<uint16_t*>(g->buf.grad_scratch + g->lay.bs[id]); }

AttnBf16 attn_copies(gpt2* g, int l) {
    return AttnBf16{BA(g, BA_HQ, l), BA(g, BA_HK, l), BA(g, BA_HV, l), BA(g, BA_HQT, l), BA(g, BA_HKT, l),
                    BA(g, BA_HVT, l)};
}

// bf16 copy of an fp32 (rows, cols) output gradient (xb) and its bias gradient's per-block
// column sums (bpart).
hipError_t cast_rows(const float* x, int rows, int cols, uint16_t* xb, float* bpart, hipStream_t st) {
    CastArgs a{};
    a.x = x;
    a.ldx = cols;
    a.xb = xb;
    a.ldb = cols;
    a.bpart = bpart;
    a.rows = rows;
    a.cols = cols;
    a.batch = 1;
    return cast_bf16(a, st);
}

// The same for `batch` weight matrices (OC, IC) stored back to back.
hipError_t cast_weights(const float* w, int OC, int IC, int batch, uint16_t* wb, uint16_t* wt, hipStream_t st) {
    CastArgs a{};
    a.x = w;
    a.ldx = IC;
    a.xb = wb;
    a.ldb = IC;
    a.xt = wt;
    a.ldt = (long)pad64(OC);
    a.rows = OC;
    a.cols = IC;
    a.batch = batch;
    a.sx = (long)OC * IC;
    a.sb = (long)OC * IC;
    a.st = (long)IC * (long)pad64(OC);
    return cast_bf16(a, st);
}

// The block's normalisation: LayerNorm, or RMSNorm in the RMSNorm variant (its mean slot
// then holds 0 and the LayerNorm bias takes no part, keeping a zero gradient).
// yb (nullable): y's bf16 copy as well
hipError_t norm_fwd(gpt2* g, float* y, float* mean, float* rstd, const float* x, const float* w, const float* b,
                    int N, int C, hipStream_t st, uint16_t* yb = nullptr) {
    if (g->variant & GPT2_VARIANT_RMSNORM) return rmsnorm_forward(y, mean, rstd, x, w, N, C, 1e-5f, st, yb);
    return layernorm_forward(y, mean, rstd, x, w, b, N, C, 1e-5f, st, yb);
}

hipError_t norm_bwd(gpt2* g, float* dx, float* dw, float* db, const float* dy, const float* x, const float* w,
                    const float* mean, const float* rstd, int N, int C, bool acc_dx, bool acc_dw, float* part,
                    hipStream_t st, hipStream_t st_red = nullptr, hipEvent_t ev = nullptr) {
    if (g->variant & GPT2_VARIANT_RMSNORM)
        return rmsnorm_backward(dx, dw, dy, x, w, mean, rstd, N, C, acc_dx, acc_dw, part, st, st_red, ev);
    return layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, N, C, acc_dx, acc_dw, part, st, st_red, ev);
}

bool rope_on(const gpt2* g) { return (g->variant & GPT2_VARIANT_ROPE) != 0; }

int forward_impl(gpt2* g, const int32_t* inputs, const int32_t* targets, int B, int T, float* loss_out) {
    const gpt2_config& c = g->cfg;
    float* part = S(g, g->lay.partial);
    const int C = c.channels, L = c.num_layers, NH = c.num_heads, V = c.vocab_size;
    const int BT = B * T;
    const long Vp = (long)g->lay.Vp;
    hipStream_t st = g->st;
    g->B = B;
    g->T = T;
    g->have_forward = false;
    if (inputs != tok_in(g)) HIPCHK(g, hipMemcpyAsync(tok_in(g), inputs, (size_t)BT * 4, hipMemcpyDeviceToDevice, st));
    if (targets) HIPCHK(g, hipMemcpyAsync(tok_tgt(g), targets, (size_t)BT * 4, hipMemcpyDeviceToDevice, st));
    HIPCHK(g, hipMemsetAsync(g->buf.grad_scratch, 0, HDR_WORDS * sizeof(float), st));
    HIPCHK(g, encoder_forward(A(g, GPT2_ACT_ENCODED), tok_in(g), P(g, P_WTE), rope_on(g) ? nullptr : P(g, P_WPE), B, T,
                              C, V, flags(g), st));
    // Mixed precision: the weights' bf16 copies (as stored and transposed) are made from
    // the current parameters at every forward; each linear layer's input is written in
    // bf16 by its producer (LayerNorm, attention, the fc GEMM's GELU epilogue) next to its
    // fp32 value (the backward's weight gradients read it too).
    const bool bf = bf_on(g);
    if (bf) {
        HIPCHK(g, cast_weights(P(g, P_QKVW), 3 * C, C, L, BA(g, BW_Q), BA(g, BWT_Q), st));
        HIPCHK(g, cast_weights(P(g, P_ATTPROJW), C, C, L, BA(g, BW_A), BA(g, BWT_A), st));
        HIPCHK(g, cast_weights(P(g, P_FCW), 4 * C, C, L, BA(g, BW_F), BA(g, BWT_F), st));
        HIPCHK(g, cast_weights(P(g, P_FCPROJW), C, 4 * C, L, BA(g, BW_P), BA(g, BWT_P), st));
        HIPCHK(g, cast_weights(P(g, P_WTE), V, C, 1, BA(g, BW_WTE), BA(g, BWT_WTE), st));
    }
    auto bf_copy = [&](int id, int l) { return bf ? BA(g, id, l) : nullptr; };
    // y = x . W^T + epilogue, in fp32 or on the bf16 copies xb, wb (yb: y's bf16 copy, GELU only)
    auto linear = [&](int epi, float* out, long ldo, const float* x, const uint16_t* xb, const float* w,
                      const uint16_t* wb, const float* bias, const float* resid, float* pre, int N, int K,
                      uint16_t* yb = nullptr) {
        if (bf) return gemm_bf16(epi, out, ldo, xb, K, wb, K, BT, N, K, bias, resid, ldo, pre, part, st, nullptr, yb, N);
        return linear_forward(out, ldo, x, w, bias, resid, pre, BT, N, K, part, st);
    };
    // the raw attention scores for the backward (which needs targets), when this batch
    // shape's tile pairs fit
    const bool store_s = targets && !bf && g->lay.attn_s && attn_ds_floats(B, T, NH) <= g->lay.n_attn_ds;
    g->scores_stored = false;
    for (int l = 0; l < L; l++) {
        float* residual = l == 0 ? A(g, GPT2_ACT_ENCODED) : A(g, GPT2_ACT_RESIDUAL3, l - 1);
        HIPCHK(g, norm_fwd(g, A(g, GPT2_ACT_LN1, l), A(g, GPT2_ACT_LN1_MEAN, l), A(g, GPT2_ACT_LN1_RSTD, l), residual,
                           P(g, P_LN1W) + l * C, P(g, P_LN1B) + l * C, BT, C, st, bf_copy(BA_LN1, l)));
        HIPCHK(g, linear(BF16_BIAS, A(g, GPT2_ACT_QKV, l), 3 * C, A(g, GPT2_ACT_LN1, l), BA(g, BA_LN1, l),
                         P(g, P_QKVW) + (size_t)l * 3 * C * C, BA(g, BW_Q, l), P(g, P_QKVB) + l * 3 * C, nullptr,
                         nullptr, 3 * C, C));
        // rotary variant: q and k rotated in place (the stored qkv is the rotated one)
        if (rope_on(g)) HIPCHK(g, rope_forward(A(g, GPT2_ACT_QKV, l), S(g, g->lay.rope), B, T, C, NH, st));
        if (bf) {
            // bf16 per-head copies of q, k, v (kept for the backward), then attention on them
            uint16_t* rm[3] = {BA(g, BA_HQ, l), BA(g, BA_HK, l), BA(g, BA_HV, l)};
            uint16_t* tr[3] = {BA(g, BA_HQT, l), BA(g, BA_HKT, l), BA(g, BA_HVT, l)};
            HIPCHK(g, attn_prep_bf16(A(g, GPT2_ACT_QKV, l), 3 * C, C, 3, rm, tr, B, T, C, NH, st));
            HIPCHK(g, attention_forward_bf16(A(g, GPT2_ACT_ATTY, l), BA(g, BA_ATTY, l), A(g, GPT2_ACT_ATT_LSE, l),
                                             attn_copies(g, l), B, T, C, NH, st));
        } else {
            HIPCHK(g, attention_forward(A(g, GPT2_ACT_ATTY, l), A(g, GPT2_ACT_ATT_LSE, l), A(g, GPT2_ACT_QKV, l), B, T,
                                        C, NH, st, store_s ? S(g, g->lay.attn_s) + (size_t)l * g->lay.n_attn_ds : nullptr));
        }
        HIPCHK(g, linear(BF16_BIAS_RESID, A(g, GPT2_ACT_RESIDUAL2, l), C, A(g, GPT2_ACT_ATTY, l), BA(g, BA_ATTY, l),
                         P(g, P_ATTPROJW) + (size_t)l * C * C, BA(g, BW_A, l), P(g, P_ATTPROJB) + l * C, residual,
                         nullptr, C, C));
        HIPCHK(g, norm_fwd(g, A(g, GPT2_ACT_LN2, l), A(g, GPT2_ACT_LN2_MEAN, l), A(g, GPT2_ACT_LN2_RSTD, l),
                           A(g, GPT2_ACT_RESIDUAL2, l), P(g, P_LN2W) + l * C, P(g, P_LN2B) + l * C, BT, C, st,
                           bf_copy(BA_LN2, l)));
        HIPCHK(g, linear(BF16_BIAS_GELU, A(g, GPT2_ACT_FCH_GELU, l), 4 * C, A(g, GPT2_ACT_LN2, l), BA(g, BA_LN2, l),
                         P(g, P_FCW) + (size_t)l * 4 * C * C, BA(g, BW_F, l), P(g, P_FCB) + l * 4 * C, nullptr,
                         A(g, GPT2_ACT_FCH, l), 4 * C, C, bf_copy(BA_FCHG, l)));
        HIPCHK(g, linear(BF16_BIAS_RESID, A(g, GPT2_ACT_RESIDUAL3, l), C, A(g, GPT2_ACT_FCH_GELU, l), BA(g, BA_FCHG, l),
                         P(g, P_FCPROJW) + (size_t)l * 4 * C * C, BA(g, BW_P, l), P(g, P_FCPROJB) + l * C,
                         A(g, GPT2_ACT_RESIDUAL2, l), nullptr, C, 4 * C));
    }
    HIPCHK(g, norm_fwd(g, A(g, GPT2_ACT_LNF), A(g, GPT2_ACT_LNF_MEAN), A(g, GPT2_ACT_LNF_RSTD),
                       A(g, GPT2_ACT_RESIDUAL3, L - 1), P(g, P_LNFW), P(g, P_LNFB), BT, C, st, bf_copy(BA_LNF, 0)));
    // LM head: the GEMM's epilogue also leaves each tile's per-row (max, sum of exp), which
    // one small pass combines into the log-sum-exp and the loss (no second read of the
    // logits)
    float* lsep = S(g, g->lay.lsep);
    if (bf) {
        HIPCHK(g, gemm_bf16(BF16_STORE, A(g, GPT2_ACT_LOGITS), Vp, BA(g, BA_LNF), C, BA(g, BW_WTE), C, BT, V, C, nullptr,
                            nullptr, 0, nullptr, part, st, lsep));
    } else {
        HIPCHK(g, linear_forward(A(g, GPT2_ACT_LOGITS), Vp, A(g, GPT2_ACT_LNF), P(g, P_WTE), nullptr, nullptr, nullptr, BT,
                                 V, C, part, st, lsep));
    }
    HIPCHK(g, lse_combine(lsep, lse_partial_count(BT, V, bf), A(g, GPT2_ACT_LOGITS), Vp, A(g, GPT2_ACT_LOGITS_LSE),
                          A(g, GPT2_ACT_LOSSES), targets ? tok_tgt(g) : nullptr, BT, V, flags(g), st));
    if (targets) HIPCHK(g, loss_mean(g->buf.grad_scratch + HDR_LOSS, A(g, GPT2_ACT_LOSSES), BT, st));
    HIPCHK(g, hipMemcpyAsync(g->host_ret, g->buf.grad_scratch, 2 * sizeof(int), hipMemcpyDeviceToHost, st));
    HIPCHK(g, hipStreamSynchronize(st));
    if (g->host_ret[1] != 0) return fail(g, GPT2_EINVAL);
    float loss;
    memcpy(&loss, &g->host_ret[0], sizeof(float));
    *loss_out = targets ? loss : -1.0f;
    g->have_forward = true;
    g->have_targets = targets != nullptr;
    g->scores_stored = store_s;
    return GPT2_OK;
}

// Samples n next tokens from the last forward's logits (host arrays in and out).
int sample_impl(gpt2* g, const int32_t* rows, const float* coins, int n, int32_t* tokens) {
    if (n == 0) return GPT2_OK;
    if (n < 0 || !rows || !coins || !tokens) return GPT2_EINVAL;
    if (!g->have_forward) return GPT2_ESTATE;
    const long BT = (long)g->B * g->T;
    if (n > BT) return GPT2_EINVAL;
    for (int i = 0; i < n; i++)
        if (rows[i] < 0 || rows[i] >= BT || !(coins[i] >= 0.0f && coins[i] < 1.0f)) return GPT2_EINVAL;
    hipStream_t st = g->st;
    int32_t* drows = reinterpret_cast<int32_t*>(S(g, g->lay.sample));
    float* dcoins = S(g, g->lay.sample) + BT;
    int32_t* dtok = reinterpret_cast<int32_t*>(S(g, g->lay.sample) + 2 * BT);
    HIPCHK(g, hipMemcpyAsync(drows, rows, (size_t)n * 4, hipMemcpyHostToDevice, st));
    HIPCHK(g, hipMemcpyAsync(dcoins, coins, (size_t)n * 4, hipMemcpyHostToDevice, st));
    HIPCHK(g, sample_tokens(A(g, GPT2_ACT_LOGITS), (long)g->lay.Vp, A(g, GPT2_ACT_LOGITS_LSE), drows, dcoins, n,
                            g->cfg.vocab_size, dtok, st));
    HIPCHK(g, hipMemcpyAsync(tokens, dtok, (size_t)n * 4, hipMemcpyDeviceToHost, st));
    HIPCHK(g, hipStreamSynchronize(st));
    return GPT2_OK;
}

// The pages' generation loop: for t = prompt_len .. total_len-1, run the forward over
// tokens[0..t) as one row and sample tokens[t] from the logits at position t-1.
int generate_impl(gpt2* g, int32_t* tokens, int prompt_len, int total_len, const float* coins) {
    if (!tokens || !coins || prompt_len < 1 || total_len <= prompt_len || total_len > g->cfg.max_seq_len ||
        (long)(total_len - 1) > (long)g->maxB * g->maxT)
        return GPT2_EINVAL;
    for (int t = prompt_len; t < total_len; t++) {
        HIPCHK(g, hipMemcpyAsync(tok_in(g), tokens, (size_t)t * 4, hipMemcpyHostToDevice, g->st));
        float loss;
        const int rc = forward_impl(g, tok_in(g), nullptr, 1, t, &loss);
        if (rc != GPT2_OK) return rc;
        const int32_t row = t - 1;
        const int rs = sample_impl(g, &row, coins + (t - prompt_len), 1, tokens + t);
        if (rs != GPT2_OK) return rs;
    }
    return GPT2_OK;
}

// AdamW arguments of a fused backward + update (bias corrections precomputed).
struct UpdateArgs {
    float lr, b1, b2, eps, wd, bc1, bc2;
};

// AdamW over parameter tensors `ids` (16-tensor order) of layer l, or whole when l < 0.
hipError_t adam_tensors(gpt2* g, const int* ids, int n, int l, const UpdateArgs& u, hipStream_t s) {
    size_t off[ADAM_MAX_SEGS], len[ADAM_MAX_SEGS];
    const size_t L = (size_t)g->cfg.num_layers;
    for (int i = 0; i < n; i++) {
        const size_t per = l < 0 ? g->plen[ids[i]] : g->plen[ids[i]] / L;
        off[i] = g->poff[ids[i]] + (l < 0 ? 0 : (size_t)l * per);
        len[i] = per;
    }
    return adamw_segments(g->buf.params, g->buf.grads, g->buf.m, g->buf.v, off, len, n, u.lr, u.b1, u.b2, u.eps,
                          u.wd, u.bc1, u.bc2, s);
}

// With `up`, each layer's parameters are updated (AdamW) as soon as its gradients are
// final, on the weight-gradient stream, while the main chain continues with the layers
// below; wte, wpe and the final norm's parameters are updated at the end.  Every
// parameter goes through the same elementwise update as gpt2_update, so the result is
// bitwise that of gpt2_backward followed by gpt2_update.
int backward_impl(gpt2* g, const UpdateArgs* up) {
    const gpt2_config& c = g->cfg;
    const int C = c.channels, L = c.num_layers, NH = c.num_heads, V = c.vocab_size;
    const int B = g->B, T = g->T, BT = B * T;
    const long Vp = (long)g->lay.Vp;
    hipStream_t st = g->st;
    float* part = S(g, g->lay.partial);
    float* dres = S(g, g->lay.dres);
    float* dln = S(g, g->lay.dln);
    float* datty = S(g, g->lay.datty);
    float* dqkv = S(g, g->lay.dqkv);
    float* dfch = S(g, g->lay.dfch);
    float* logits = A(g, GPT2_ACT_LOGITS);

    // wte receives rows by token twice (targets' lnf rows below, inputs' residual-gradient
    // rows at the end): both token lists are sorted once, up front, on the second stream
    // (the main chain needs neither; that stream's first user is the targets' scatter, and
    // the main stream's input scatter comes after it waits for that stream's end)
    int* wk_in = reinterpret_cast<int*>(S(g, g->lay.enc_work));
    int* wk_tgt = reinterpret_cast<int*>(S(g, g->lay.enc_work_tgt));
    const bool sorted = embedding_sortable(BT, V);

    // LM head (tied): dlnf = dlogits . wte;  dwte += dlogits^T . lnf, where
    // dlogits = (softmax(logits) - onehot(target)) / (B*T) is formed as the GEMMs load the
    // logits (softmax = exp(logit - lse)).
    const XentOperand xo{A(g, GPT2_ACT_LOGITS_LSE), tok_tgt(g), 1.0f / (float)BT};
    // Weight gradients run on the handle's second stream (see below); the LM head's
    // (dwte += dlogits^T lnf, then the one-hot rows) go first, both on that stream since
    // both accumulate into dwte.
    hipStream_t sw = g->backward_streams == 2 ? g->st_w : st;
    float* part_w = S(g, g->lay.partial_w);
    enum { EV_DRES_A, EV_DFCH, EV_DRES_B, EV_DQKV, EV_W_FCPROJ, EV_W_FC, EV_W_ATTPROJ, EV_W_QKV, EV_LM, EV_W_LM, EV_LN1,
           EV_W_END, EV_U_END };
    hipStream_t su = g->backward_streams == 2 ? g->st_u : st;
    // the layers' LayerNorm dw/db reductions on the update stream, each from its own
    // partial rows (the update stream applies them after its layer's weight gradients)
    const bool lnred = GPT2_LN_REDUCE_ASYNC && up != nullptr && su != st;
    auto lnpart = [&](int i) {
        return S(g, g->lay.lnpart) + (size_t)i * layernorm_partial_floats((int)BT, (int)C);
    };
    auto mark = [&](int e, hipStream_t s) { return hipEventRecord(g->ev[e], s); };
    auto after = [&](hipStream_t s, int e) { return hipStreamWaitEvent(s, g->ev[e], 0); };
    // Mixed precision: every GEMM below multiplies bf16 copies.  dlogits is written once
    // in bf16; each output gradient dY gets its copy (and its bias gradient's partial sums,
    // from the fp32 values) on the main stream before its GEMMs, in a buffer per kind that
    // the events below protect exactly as they protect dY itself: the dgrad (main stream)
    // and the wgrad (second stream, reading dY and X row-contiguous) both read it.
    const bool bf = bf_on(g);
    // the bias gradient's column sums per row block, one buffer per kind of dY (0 fcproj,
    // 1 fc, 2 attproj, 3 qkv): the second stream adds them up (bias_w) ahead of the kind's
    // wgrad, and the events that let the main stream rewrite that kind's dY (and its copy)
    // in the next layer come after it
    auto bpart = [&](int kind) { return S(g, g->lay.bpart) + (size_t)kind * bias_slot_floats(B, T, C); };
    auto grad_copies = [&](const float* dy, int n, uint16_t* yb, int kind) -> hipError_t {
        return cast_rows(dy, BT, n, yb, bpart(kind), st);
    };
    auto bias_w = [&](float* db, int n, int kind) { return bias_reduce(db, bpart(kind), BT, n, sw); };
    // dW[M,N] += dY^T X (and, fp32 only, db += column sums of dY): dY (BT, M), X (BT, N);
    // yb, xb their bf16 copies
    auto wgrad = [&](float* dw, float* db, const float* dy, const uint16_t* yb, int M, const float* x,
                     const uint16_t* xb, int N) {
        if (bf) return gemm_bf16_rows(dw, N, yb, M, xb, N, M, N, BT, part_w, sw);
        return linear_wgrad(dw, db, dy, M, x, M, N, BT, part_w, sw);
    };
    // dX[BT,N] = dY[BT,K] . W[K,N] (times gelu'(gelu_pre) if given); yb = bf16 dY, wt = bf16
    // W^T (N, K padded)
    auto dgrad = [&](float* dx, const float* dy, const uint16_t* yb, int K, const float* w, const uint16_t* wt, int N,
                     const float* gelu_pre, uint16_t* xb = nullptr, float* xsum = nullptr) {
        if (bf) return gemm_bf16(gelu_pre ? BF16_GELU_BWD : BF16_STORE, dx, N, yb, K, wt, (long)pad64(K), BT, N, K,
                                 nullptr, gelu_pre, N, nullptr, part, st, nullptr, xb, N, xsum);
        return linear_dgrad(dx, dy, K, w, gelu_pre, BT, N, K, part, st);
    };
    uint16_t* dresb = bf ? BS(g, BS_DRES) : nullptr;
    uint16_t* dfchb = bf ? BS(g, BS_DFCH) : nullptr;
    uint16_t* dqkvb = bf ? BS(g, BS_DQKV) : nullptr;
    if (bf) {
        HIPCHK(g, xent_grad_bf16(BS(g, BS_DLOG), logits, Vp, A(g, GPT2_ACT_LOGITS_LSE), tok_tgt(g), xo.scale, BT, V,
                                 st));
        HIPCHK(g, mark(EV_LM, st));
        HIPCHK(g, after(sw, EV_LM));
        if (sorted) HIPCHK(g, sort_token_lists(wk_in, tok_in(g), wk_tgt, tok_tgt(g), BT, V, sw));
        HIPCHK(g, gemm_bf16_rows(G(g, P_WTE), C, BS(g, BS_DLOG), Vp, BA(g, BA_LNF), C, V, C, BT, part_w, sw));
        HIPCHK(g, mark(EV_W_LM, sw));
        HIPCHK(g, gemm_bf16(BF16_STORE, dln, C, BS(g, BS_DLOG), Vp, BA(g, BWT_WTE), Vp, BT, C, (int)Vp, nullptr, nullptr,
                            0, nullptr, part, st));
    } else {
        HIPCHK(g, mark(EV_LM, st));
        HIPCHK(g, after(sw, EV_LM));
        if (sorted) HIPCHK(g, sort_token_lists(wk_in, tok_in(g), wk_tgt, tok_tgt(g), BT, V, sw));
        HIPCHK(g, linear_wgrad(G(g, P_WTE), nullptr, logits, Vp, A(g, GPT2_ACT_LNF), V, C, BT, part_w, sw, &xo));
        // the one-hot part of dlogits: dwte[target] -= lnf / BT
        if (sorted) HIPCHK(g, scatter_sorted(G(g, P_WTE), C, A(g, GPT2_ACT_LNF), C, -xo.scale, wk_tgt, BT, sw));
        else HIPCHK(g, embedding_scatter(G(g, P_WTE), V, C, tok_tgt(g), BT, A(g, GPT2_ACT_LNF), C, -xo.scale, wk_tgt, sw));
        HIPCHK(g, mark(EV_W_LM, sw));
        HIPCHK(g, linear_dgrad(dln, logits, Vp, P(g, P_WTE), nullptr, BT, C, V, part, st, &xo));
    }
    // (the final norm's dw/db are only read by the last update, on the main stream after it
    // waits for the second stream's end: their reduction goes to the second stream)
    HIPCHK(g, norm_bwd(g, dres, G(g, P_LNFW), G(g, P_LNFB), dln, A(g, GPT2_ACT_RESIDUAL3, L - 1), P(g, P_LNFW),
                       A(g, GPT2_ACT_LNF_MEAN), A(g, GPT2_ACT_LNF_RSTD), BT, C, false, true,
                       lnred ? lnpart(2 * L) : part, st, lnred ? sw : nullptr, g->ev[13]));
    // Per layer, the weight gradients (dW += dY^T X, db) need only that layer's output
    // gradient, so they run on the handle's second stream and overlap the main chain
    // (dgrads, attention, LayerNorm).  Events order the two: the second stream waits for
    // each dY it reads; the main stream waits before it rewrites a buffer the second
    // stream still reads (dres by the LayerNorm backwards, dfch by the next layer's fcproj
    // dgrad, dqkv by the next layer's attention backward), and before returning.  The
    // arithmetic of every kernel is unchanged, so results are bitwise those of one stream.
    for (int l = L - 1; l >= 0; l--) {
        float* residual = l == 0 ? A(g, GPT2_ACT_ENCODED) : A(g, GPT2_ACT_RESIDUAL3, l - 1);
        const bool later = l < L - 1;  // the previous iteration's weight gradients exist
        // MLP projection: residual3 = residual2 + gelu(fch) . Wp^T + bp.
        if (bf) HIPCHK(g, grad_copies(dres, C, dresb, 0));
        HIPCHK(g, mark(EV_DRES_A, st));
        HIPCHK(g, after(sw, EV_DRES_A));
        if (bf) HIPCHK(g, bias_w(G(g, P_FCPROJB) + l * C, C, 0));
        HIPCHK(g, wgrad(G(g, P_FCPROJW) + (size_t)l * 4 * C * C, G(g, P_FCPROJB) + l * C, dres, dresb, C,
                        A(g, GPT2_ACT_FCH_GELU, l), bf ? BA(g, BA_FCHG, l) : nullptr, 4 * C));
        HIPCHK(g, mark(EV_W_FCPROJ, sw));
        if (later) HIPCHK(g, after(st, EV_W_FC));  // the fc wgrad above still reads dfch
        // (mixed precision: the GELU-backward epilogue also writes dfch's bf16 copy and the
        // fc bias gradient's column sums per 16-row slice)
        HIPCHK(g, dgrad(dfch, dres, dresb, C, P(g, P_FCPROJW) + (size_t)l * 4 * C * C, BA(g, BWT_P, l), 4 * C,
                        A(g, GPT2_ACT_FCH, l), dfchb, bf ? bpart(1) : nullptr));
        // MLP expansion: fch = ln2 . Wf^T + bf.
        HIPCHK(g, mark(EV_DFCH, st));
        HIPCHK(g, after(sw, EV_DFCH));
        if (bf) HIPCHK(g, bias_reduce_parts(G(g, P_FCB) + l * 4 * C, bpart(1), (BT + 15) / 16, 4 * C, sw));
        HIPCHK(g, wgrad(G(g, P_FCW) + (size_t)l * 4 * C * C, G(g, P_FCB) + l * 4 * C, dfch, dfchb, 4 * C,
                        A(g, GPT2_ACT_LN2, l), bf ? BA(g, BA_LN2, l) : nullptr, C));
        HIPCHK(g, mark(EV_W_FC, sw));
        HIPCHK(g, dgrad(dln, dfch, dfchb, 4 * C, P(g, P_FCW) + (size_t)l * 4 * C * C, BA(g, BWT_F, l), C, nullptr));
        HIPCHK(g, after(st, EV_W_FCPROJ));  // dres is about to change
        HIPCHK(g, norm_bwd(g, dres, G(g, P_LN2W) + l * C, G(g, P_LN2B) + l * C, dln, A(g, GPT2_ACT_RESIDUAL2, l),
                           P(g, P_LN2W) + l * C, A(g, GPT2_ACT_LN2_MEAN, l), A(g, GPT2_ACT_LN2_RSTD, l), BT, C, true,
                           true, lnred ? lnpart(2 * l) : part, st, lnred ? su : nullptr, g->ev[13]));
        // Attention projection: residual2 = residual + atty . Wa^T + ba.
        if (bf) HIPCHK(g, grad_copies(dres, C, dresb, 2));
        HIPCHK(g, mark(EV_DRES_B, st));
        HIPCHK(g, after(sw, EV_DRES_B));
        if (bf) HIPCHK(g, bias_w(G(g, P_ATTPROJB) + l * C, C, 2));
        HIPCHK(g, wgrad(G(g, P_ATTPROJW) + (size_t)l * C * C, G(g, P_ATTPROJB) + l * C, dres, dresb, C,
                        A(g, GPT2_ACT_ATTY, l), bf ? BA(g, BA_ATTY, l) : nullptr, C));
        HIPCHK(g, mark(EV_W_ATTPROJ, sw));
        HIPCHK(g, dgrad(datty, dres, dresb, C, P(g, P_ATTPROJW) + (size_t)l * C * C, BA(g, BWT_A, l), C, nullptr));
        if (later) HIPCHK(g, after(st, EV_W_QKV));  // the qkv wgrad above still reads dqkv
        if (bf) {
            uint16_t* rm[1] = {BS(g, BS_HDO)};
            uint16_t* tr[1] = {BS(g, BS_HDOT)};
            HIPCHK(g, attn_prep_bf16(datty, C, 0, 1, rm, tr, B, T, C, NH, st));
            // dqkv's bf16 copy and the qkv bias's partial sums come from the attention
            // kernels, or, in the rotary variant, from a cast after the rotation below
            const bool rot = rope_on(g);
            HIPCHK(g, attention_backward_bf16(dqkv, rot ? nullptr : dqkvb, rot ? nullptr : bpart(3), S(g, g->lay.delta),
                                              BS(g, BS_HDO), BS(g, BS_HDOT), A(g, GPT2_ACT_ATTY, l),
                                              A(g, GPT2_ACT_ATT_LSE, l), attn_copies(g, l), B, T, C, NH, st));
        } else {
            // the stored-score-gradient path when this batch shape's pairs fit the buffer
            // sized at build (a call may use another B, T with B*T within the built one)
            float* ds = g->lay.n_attn_ds && attn_ds_floats(B, T, NH) <= g->lay.n_attn_ds ? S(g, g->lay.attn_ds) : nullptr;
            const float* sb = ds && g->scores_stored ? S(g, g->lay.attn_s) + (size_t)l * g->lay.n_attn_ds : nullptr;
            HIPCHK(g, attention_backward(dqkv, S(g, g->lay.delta), datty, A(g, GPT2_ACT_QKV, l), A(g, GPT2_ACT_ATTY, l),
                                         A(g, GPT2_ACT_ATT_LSE, l), B, T, C, NH, st, ds, sb));
        }
        // QKV projection: qkv = ln1 . Wqkv^T + bqkv.
        // rotary variant: attention gave the gradient of the rotated q and k; rotate it back
        if (rope_on(g)) HIPCHK(g, rope_backward(dqkv, S(g, g->lay.rope), B, T, C, NH, st));
        if (bf && rope_on(g)) HIPCHK(g, grad_copies(dqkv, 3 * C, dqkvb, 3));
        HIPCHK(g, mark(EV_DQKV, st));
        HIPCHK(g, after(sw, EV_DQKV));
        if (bf && rope_on(g)) HIPCHK(g, bias_w(G(g, P_QKVB) + l * 3 * C, 3 * C, 3));
        if (bf && !rope_on(g))
            HIPCHK(g, bias_reduce_parts(G(g, P_QKVB) + l * 3 * C, bpart(3), attn_bias_partial_rows(B, T), 3 * C, sw));
        HIPCHK(g, wgrad(G(g, P_QKVW) + (size_t)l * 3 * C * C, G(g, P_QKVB) + l * 3 * C, dqkv, dqkvb, 3 * C,
                        A(g, GPT2_ACT_LN1, l), bf ? BA(g, BA_LN1, l) : nullptr, C));
        HIPCHK(g, mark(EV_W_QKV, sw));
        HIPCHK(g, dgrad(dln, dqkv, dqkvb, 3 * C, P(g, P_QKVW) + (size_t)l * 3 * C * C, BA(g, BWT_Q, l), C, nullptr));
        HIPCHK(g, after(st, EV_W_ATTPROJ));  // dres is about to change
        HIPCHK(g, norm_bwd(g, dres, G(g, P_LN1W) + l * C, G(g, P_LN1B) + l * C, dln, residual, P(g, P_LN1W) + l * C,
                           A(g, GPT2_ACT_LN1_MEAN, l), A(g, GPT2_ACT_LN1_RSTD, l), BT, C, true, true,
                           lnred ? lnpart(2 * l + 1) : part, st, lnred ? su : nullptr, g->ev[13]));
        if (up) {
            // layer l's gradients are final once its LayerNorm backwards (main stream, just
            // queued) and its weight gradients (last: the qkv wgrad on the second stream)
            // are done; a third stream updates its parameters without holding either up
            static const int layer_ids[12] = {P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB,
                                              P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPROJW, P_FCPROJB};
            HIPCHK(g, mark(EV_LN1, st));
            HIPCHK(g, after(su, EV_LN1));
            HIPCHK(g, after(su, EV_W_QKV));
            HIPCHK(g, adam_tensors(g, layer_ids, 12, l, *up, su));
        }
    }
    // the second stream's last operation ends all of its work (dwte is written below)
    HIPCHK(g, mark(EV_W_END, sw));
    HIPCHK(g, after(st, EV_W_END));
    if (!rope_on(g)) HIPCHK(g, wpe_backward(G(g, P_WPE), dres, B, T, C, st));
    if (sorted) HIPCHK(g, scatter_sorted(G(g, P_WTE), C, dres, C, 1.0f, wk_in, BT, st));
    else HIPCHK(g, embedding_scatter(G(g, P_WTE), V, C, tok_in(g), BT, dres, C, 1.0f, wk_in, st));
    if (up) {
        static const int global_ids[4] = {P_WTE, P_WPE, P_LNFW, P_LNFB};
        HIPCHK(g, adam_tensors(g, global_ids, 4, -1, *up, st));
        HIPCHK(g, mark(EV_U_END, su));
        HIPCHK(g, after(st, EV_U_END));
    }
    return GPT2_OK;
}

}  // namespace

extern "C" {

size_t gpt2_num_parameters(const gpt2_config* cfg) {
    if (!config_ok(cfg)) return 0;
    size_t len[NP], n = 0;
    param_sizes(cfg, len);
    for (int i = 0; i < NP; i++) n += len[i];
    return n;
}

int gpt2_param_layout(const gpt2_config* cfg, size_t off[NP], size_t len[NP]) {
    if (!config_ok(cfg) || !off || !len) return GPT2_EINVAL;
    param_sizes(cfg, len);
    size_t o = 0;
    for (int i = 0; i < NP; i++) {
        off[i] = o;
        o += len[i];
    }
    return GPT2_OK;
}

int gpt2_arena_sizes(const gpt2_config* cfg, int B, int T, size_t* n_acts, size_t* n_grad_scratch) {
    return gpt2_arena_sizes_variant(cfg, B, T, 0, n_acts, n_grad_scratch);
}

int gpt2_arena_sizes_variant(const gpt2_config* cfg, int B, int T, int variant, size_t* n_acts,
                             size_t* n_grad_scratch) {
    if (!config_ok(cfg) || B <= 0 || T <= 0 || T > cfg->max_seq_len || !n_acts || !n_grad_scratch)
        return GPT2_EINVAL;
    if (variant & ~(GPT2_VARIANT_RMSNORM | GPT2_VARIANT_ROPE | GPT2_VARIANT_BF16)) return GPT2_EINVAL;
    if ((long)B * T > (1L << 30)) return GPT2_EINVAL;
    const Layout y = make_layout(cfg, B, T, variant);
    *n_acts = y.n_acts;
    *n_grad_scratch = y.n_scratch;
    return GPT2_OK;
}

int gpt2_build(gpt2** out, const gpt2_config* cfg, int B, int T, const gpt2_buffers* bufs, void* stream) {
    return gpt2_build_variant(out, cfg, B, T, bufs, stream, 0);
}

int gpt2_build_variant(gpt2** out, const gpt2_config* cfg, int B, int T, const gpt2_buffers* bufs, void* stream,
                       int variant) {
    if (!out) return GPT2_EINVAL;
    *out = nullptr;
    if (!config_ok(cfg) || B <= 0 || T <= 0 || T > cfg->max_seq_len || !bufs) return GPT2_EINVAL;
    if (variant & ~(GPT2_VARIANT_RMSNORM | GPT2_VARIANT_ROPE | GPT2_VARIANT_BF16)) return GPT2_EINVAL;
    if ((variant & GPT2_VARIANT_ROPE) && (cfg->channels / cfg->num_heads) % 2) return GPT2_EINVAL;
    if ((variant & GPT2_VARIANT_BF16) && cfg->channels % 8) return GPT2_EINVAL;
    if ((long)B * T > (1L << 30)) return GPT2_EINVAL;
    const gpt2_buffers& b = *bufs;
    if (!b.params || !b.grads || !b.m || !b.v || !b.acts || !b.grad_scratch) return GPT2_EINVAL;
    if (!aligned(b.params) || !aligned(b.grads) || !aligned(b.m) || !aligned(b.v) || !aligned(b.acts) ||
        !aligned(b.grad_scratch))
        return GPT2_EINVAL;
    gpt2* g = (gpt2*)calloc(1, sizeof(gpt2));
    if (!g) return GPT2_ENOMEM;
    g->cfg = *cfg;
    g->maxB = B;
    g->maxT = T;
    g->B = B;
    g->T = T;
    g->lay = make_layout(cfg, B, T, variant);
    g->st = (hipStream_t)stream;
    g->backward_streams = 2;
    g->variant = variant;
    g->buf = b;
    g->nparams = gpt2_num_parameters(cfg);
    gpt2_param_layout(cfg, g->poff, g->plen);
    if (hipHostMalloc((void**)&g->host_ret, 2 * sizeof(int), hipHostMallocDefault) != hipSuccess) {
        free(g);
        return GPT2_EDEVICE;
    }
    // the weight-gradient stream (default priority, no implicit sync with the null stream)
    // and the events that order it against the main stream
    bool ok = hipStreamCreateWithFlags(&g->st_w, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipStreamCreateWithFlags(&g->st_u, hipStreamNonBlocking) == hipSuccess;
    int nev = 0;
    for (; ok && nev < 14; nev++) ok = hipEventCreateWithFlags(&g->ev[nev], hipEventDisableTiming) == hipSuccess;
    if (ok) {
        ok = fill_zero(b.grads, g->nparams, g->st) == hipSuccess && fill_zero(b.m, g->nparams, g->st) == hipSuccess &&
             fill_zero(b.v, g->nparams, g->st) == hipSuccess;
    }
    if (ok && (variant & GPT2_VARIANT_ROPE))
        ok = rope_table(S(g, g->lay.rope), cfg->max_seq_len, cfg->channels / cfg->num_heads, g->st) == hipSuccess;
    if (!ok) {
        for (int i = 0; i < nev; i++) (void)hipEventDestroy(g->ev[i]);
        if (g->st_w) (void)hipStreamDestroy(g->st_w);
        if (g->st_u) (void)hipStreamDestroy(g->st_u);
        (void)hipHostFree(g->host_ret);
        free(g);
        return GPT2_EDEVICE;
    }
    *out = g;
    return GPT2_OK;
}

float gpt2_forward(gpt2* g, const int32_t* inputs, const int32_t* targets, int B, int T) {
    if (!g) return NAN;
    g->last_error = GPT2_OK;
    if (!inputs || B <= 0 || T <= 0 || T > g->cfg.max_seq_len || (long)B * T > (long)g->maxB * g->maxT) {
        g->last_error = GPT2_EINVAL;
        return NAN;
    }
    // The mixed-precision variant's per-head attention copies and their bias partial
    // sums hold B rows of T positions rounded up to whole 64-position tiles, sized at
    // build: a batch whose rounded size exceeds the built one would not fit.
    if (bf_on(g) && (long)B * (long)pad64(T) > (long)g->maxB * (long)pad64(g->maxT)) {
        g->last_error = GPT2_EINVAL;
        return NAN;
    }
    float loss = NAN;
    ProfBind bind(g);
    const int rc = forward_impl(g, inputs, targets, B, T, &loss);
    if (rc != GPT2_OK) {
        g->last_error = rc;
        g->have_forward = false;
        return NAN;
    }
    return loss;
}

int gpt2_zero_grad(gpt2* g) {
    if (!g) return GPT2_EINVAL;
    ProfBind bind(g);
    HIPCHK(g, fill_zero(g->buf.grads, g->nparams, g->st));
    return GPT2_OK;
}

int gpt2_backward(gpt2* g) {
    if (!g) return GPT2_EINVAL;
    if (!g->have_forward || !g->have_targets) return fail(g, GPT2_ESTATE);
    ProfBind bind(g);
    return backward_impl(g, nullptr);
}

int gpt2_backward_update(gpt2* g, float lr, float beta1, float beta2, float eps, float weight_decay, int t) {
    if (!g) return GPT2_EINVAL;
    if (t < 1 || !g->have_forward || !g->have_targets) return fail(g, GPT2_ESTATE);
    const UpdateArgs up{lr, beta1, beta2, eps, weight_decay, (float)(1.0 - pow((double)beta1, (double)t)),
                        (float)(1.0 - pow((double)beta2, (double)t))};
    ProfBind bind(g);
    return backward_impl(g, &up);
}

int gpt2_update(gpt2* g, float lr, float beta1, float beta2, float eps, float weight_decay, int t) {
    if (!g) return GPT2_EINVAL;
    if (t < 1) return fail(g, GPT2_ESTATE);
    const float bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    const float bc2 = (float)(1.0 - pow((double)beta2, (double)t));
    ProfBind bind(g);
    HIPCHK(g, adamw(g->buf.params, g->buf.grads, g->buf.m, g->buf.v, g->nparams, lr, beta1, beta2, eps, weight_decay,
                    bc1, bc2, g->st));
    return GPT2_OK;
}

int gpt2_last_error(const gpt2* g) { return g ? g->last_error : GPT2_EINVAL; }

const char* gpt2_strerror(int code) {
    switch (code) {
        case GPT2_OK: return "ok";
        case GPT2_EINVAL: return "invalid argument, shape or token id";
        case GPT2_ESTATE: return "call out of order";
        case GPT2_EDEVICE: return "HIP call failed";
        case GPT2_ENOMEM: return "out of host memory";
        case GPT2_ESCRATCH: return "request larger than the library's fixed device scratch";
        default: return "unknown error";
    }
}

void gpt2_free(gpt2* g) {
    if (!g) return;
    (void)hipStreamSynchronize(g->st);
    (void)hipStreamSynchronize(g->st_w);
    (void)hipStreamSynchronize(g->st_u);
    for (hipEvent_t e : g->ev) (void)hipEventDestroy(e);
    (void)hipStreamDestroy(g->st_w);
    (void)hipStreamDestroy(g->st_u);
    if (g->prof) prof_destroy(g->prof);
    (void)hipHostFree(g->host_ret);
    free(g);
}

int gpt2_profile_enable(gpt2* g, int enable) {
    if (!g) return GPT2_EINVAL;
    if (hipStreamSynchronize(g->st) != hipSuccess || hipStreamSynchronize(g->st_w) != hipSuccess ||
        hipStreamSynchronize(g->st_u) != hipSuccess)
        return fail(g, GPT2_EDEVICE);
    if (enable && !g->prof) {
        g->prof = prof_create();
        if (!g->prof) return fail(g, GPT2_EDEVICE);
    } else if (enable) {
        prof_reset(g->prof);
    } else if (g->prof) {
        prof_destroy(g->prof);
        g->prof = nullptr;
    }
    return GPT2_OK;
}

int gpt2_profile_filter(gpt2* g, const char* kernel_name) {
    if (!g || !g->prof) return GPT2_ESTATE;
    prof_filter(g->prof, kernel_name);
    return GPT2_OK;
}

int gpt2_profile_collect(gpt2* g) {
    if (!g || !g->prof) return GPT2_ESTATE;
    const int n = prof_collect(g->prof);
    return n < 0 ? fail(g, GPT2_EDEVICE) : n;
}

int gpt2_profile_entry(gpt2* g, int i, const char** name, long* launches, double* total_ms, double* flops,
                       double* bytes) {
    if (!g || !g->prof || !name || !launches || !total_ms || !flops || !bytes) return GPT2_EINVAL;
    return prof_entry(g->prof, i, name, launches, total_ms, flops, bytes) == 0 ? GPT2_OK : GPT2_EINVAL;
}

int gpt2_activation_view(const gpt2* g, int tensor, int layer, size_t* offset, size_t* rows, size_t* cols,
                         size_t* ld) {
    if (!g || tensor < 0 || tensor >= GPT2_NUM_ACTS || !offset || !rows || !cols || !ld) return GPT2_EINVAL;
    const ActInfo& a = g->lay.a[tensor];
    if (a.layer_stride && (layer < 0 || layer >= g->cfg.num_layers)) return GPT2_EINVAL;
    *offset = a.off + (a.layer_stride ? (size_t)layer * a.layer_stride : 0);
    *rows = (size_t)g->B * g->T;
    *cols = a.cols;
    *ld = a.ld;
    if (tensor == GPT2_ACT_ATT_LSE) {  // stored (B, NH, T)
        *rows = (size_t)g->B * g->cfg.num_heads;
        *cols = (size_t)g->T;
        *ld = (size_t)g->T;
    }
    return GPT2_OK;
}

int gpt2_layernorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w, const float* b, int N,
                           int C, float eps, void* stream) {
    if (N < 0 || C <= 0 || C % 4 || C > 4096) return GPT2_EINVAL;
    if (N == 0) return GPT2_OK;
    if (!y || !mean || !rstd || !x || !w || !b) return GPT2_EINVAL;
    if (!aligned(y) || !aligned(x) || !aligned(w) || !aligned(b)) return GPT2_EINVAL;
    return layernorm_forward(y, mean, rstd, x, w, b, N, C, eps, (hipStream_t)stream) == hipSuccess ? GPT2_OK
                                                                                                      : GPT2_EDEVICE;
}

int gpt2_sample(gpt2* g, const int32_t* rows, const float* coins, int n, int32_t* tokens) {
    if (!g) return GPT2_EINVAL;
    g->last_error = GPT2_OK;
    ProfBind bind(g);
    const int rc = sample_impl(g, rows, coins, n, tokens);
    return rc == GPT2_OK ? GPT2_OK : fail(g, rc);
}

int gpt2_generate(gpt2* g, int32_t* tokens, int prompt_len, int total_len, const float* coins) {
    if (!g) return GPT2_EINVAL;
    g->last_error = GPT2_OK;
    ProfBind bind(g);
    const int rc = generate_impl(g, tokens, prompt_len, total_len, coins);
    return rc == GPT2_OK ? GPT2_OK : fail(g, rc);
}

int gpt2_set_backward_streams(gpt2* g, int streams) {
    if (!g || (streams != 1 && streams != 2)) return GPT2_EINVAL;
    g->backward_streams = streams;
    return GPT2_OK;
}

int gpt2_set_gemm_tiles(int policy) {
    static_assert(GPT2_GEMM_TILES_AUTO == GEMM_TILES_AUTO && GPT2_GEMM_TILES_128 == GEMM_TILES_128 &&
                      GPT2_GEMM_TILES_96 == GEMM_TILES_96,
                  "tile policy values");
    return gemm_set_tile_policy(policy) ? GPT2_OK : GPT2_EINVAL;
}

size_t gpt2_layernorm_backward_workspace(int N, int C) {
    if (N < 0 || C <= 0) return 0;
    return layernorm_partial_floats(N, C);
}

int gpt2_layernorm_backward(float* dx, float* dw, float* db, const float* dy, const float* x, const float* w,
                            const float* mean, const float* rstd, int N, int C, float* workspace,
                            size_t workspace_floats, void* stream) {
    if (!dw || !db || N < 0 || C <= 0 || C % 4 || C > 4096) return GPT2_EINVAL;
    if (N > 0 && (!dx || !dy || !x || !w || !mean || !rstd)) return GPT2_EINVAL;
    if (N > 0 && (!aligned(dx) || !aligned(dy) || !aligned(x) || !aligned(w))) return GPT2_EINVAL;
    if (N > 0 && (!workspace || workspace_floats < layernorm_partial_floats(N, C))) return GPT2_EINVAL;
    return layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, N, C, false, false, workspace,
                              (hipStream_t)stream) == hipSuccess
               ? GPT2_OK
               : GPT2_EDEVICE;
}

}  // extern "C"
