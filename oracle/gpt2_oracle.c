/*
 * gpt2_oracle.c -- plain CPU oracle of one GPT-2 training step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; it exists so that tests (and the CPU baseline of the benchmark) can
 * check the GPU library against a slow, obviously correct definition.  It shares no
 * code, header or table with the GPU library.
 *
 * What it computes follows the pages' own decomposition of llm.c's train_gpt2.c:
 *   - layer functions encoder/layernorm/matmul/attention/gelu/residual forward and
 *     backward, softmax, cross-entropy and the fused softmax+cross-entropy backward
 *     ("llm.c：Andrej Karpathy带你从零复现LLM", 核心代码解读：train_gpt2.c, item 1;
 *     新智元 article "千行C代码训完GPT-2", 纯CUDA也可训);
 *   - the model structs (config, 16 parameter tensors, activation tensors) and the
 *     five calls build / forward / zero_grad / backward / update with AdamW
 *     (same huxiu page, items 2 and 3);
 *   - one flat array for all parameters and one for all activations, allocated once
 *     ("OpenAI创始大神手搓千行C代码训练GPT", 手动实现每个层前向 / 反向传播;
 *     新智元 article, 纯CUDA也可训).
 * Where the pages stop (block wiring, GELU form, LayerNorm eps, attention scale and
 * mask, loss reduction, AdamW details) the plainest GPT-2 reading is taken; each
 * such reading is named at the function that makes it.
 *
 * Precision: `real` is double by default; -DORACLE_REAL_FLOAT builds the same code
 * in float (the pages' CPU reference is fp32).  Each reduction runs in one fixed
 * order, and OpenMP only splits independent outputs, so the bits do not depend on
 * the thread count.  Tiling in matmul splits only the set of outputs, never a sum.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_REAL_FLOAT
typedef float real;
#define R_EXP expf
#define R_LOG logf
#define R_SQRT sqrtf
#define R_TANH tanhf
#define R_POW powf
#define R_COS cosf
#define R_SIN sinf
#define R_POW powf
#else
typedef double real;
#define R_EXP exp
#define R_LOG log
#define R_SQRT sqrt
#define R_TANH tanh
#define R_POW pow
#define R_COS cos
#define R_SIN sin
#define R_POW pow
#endif

#define EXPORT __attribute__((visibility("default")))

enum { O_OK = 0, O_EINVAL = -1, O_ESTATE = -2, O_ENOMEM = -4 };

typedef struct {
    int max_seq_len, vocab_size, num_layers, num_heads, channels;
} oracle_config;

EXPORT int oracle_real_size(void) { return (int)sizeof(real); }

EXPORT void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

EXPORT int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Layers.  Every backward ADDS into its gradient outputs.                   */
/* ------------------------------------------------------------------------- */

/* Token plus position embedding: out[b,t,:] = wte[tok[b,t],:] + wpe[t,:].
 * Position restarts at 0 in every row (plain reading; the pages only name the
 * embedding, huxiu 核心代码解读 item 1). */
EXPORT void oracle_encoder_forward(real* out, const int32_t* tok, const real* wte,
                                   const real* wpe, int B, int T, int C) {
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            real* o = out + ((size_t)b * T + t) * C;
            const real* we = wte + (size_t)tok[b * T + t] * C;
            for (int c = 0; c < C; c++) o[c] = we[c];
            if (wpe) {  /* NULL: no position rows (the rotary variant) */
                const real* pe = wpe + (size_t)t * C;
                for (int c = 0; c < C; c++) o[c] += pe[c];
            }
        }
}

/* Backward of the embedding: scatter-add into the rows of wte that were read, and
 * add into wpe.  Positions are visited in (b,t) order for every channel. */
EXPORT void oracle_encoder_backward(real* dwte, real* dwpe, const real* dout,
                                    const int32_t* tok, int B, int T, int C) {
#pragma omp parallel for
    for (int c = 0; c < C; c++)
        for (int b = 0; b < B; b++)
            for (int t = 0; t < T; t++) {
                real d = dout[((size_t)b * T + t) * C + c];
                dwte[(size_t)tok[b * T + t] * C + c] += d;
                if (dwpe) dwpe[(size_t)t * C + c] += d;
            }
}

/* LayerNorm over the last axis: mean, biased variance, rstd = 1/sqrt(var + eps),
 * y = (x - mean) * rstd * w + b; mean and rstd are kept for the backward.  The
 * pages show LayerNorm as their worked layer (dakule, 手动实现每个层前向 / 反向传播;
 * skycaiji 教程).  eps is an argument; the model uses 1e-5 (PyTorch's default,
 * not printed on the pages). */
EXPORT void oracle_layernorm_forward(real* out, real* mean, real* rstd, const real* inp,
                                     const real* w, const real* b, int N, int C, real eps) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* x = inp + (size_t)i * C;
        real m = 0;
        for (int c = 0; c < C; c++) m += x[c];
        m = m / C;
        real v = 0;
        for (int c = 0; c < C; c++) {
            real d = x[c] - m;
            v += d * d;
        }
        v = v / C;
        real s = (real)1 / R_SQRT(v + eps);
        real* y = out + (size_t)i * C;
        for (int c = 0; c < C; c++) y[c] = (x[c] - m) * s * w[c] + b[c];
        mean[i] = m;
        rstd[i] = s;
    }
}

/* LayerNorm backward, derived by hand from the forward above.  With xh = (x-mean)*rstd
 * and g = w*dy:  dx += rstd * (g - mean(g) - xh * mean(g*xh)),  dw += sum_rows dy*xh,
 * db += sum_rows dy.  Row part and column part are separate loops so each sum has one
 * fixed order. */
EXPORT void oracle_layernorm_backward(real* dinp, real* dw, real* db, const real* dout,
                                      const real* inp, const real* w, const real* mean,
                                      const real* rstd, int N, int C) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* x = inp + (size_t)i * C;
        const real* dy = dout + (size_t)i * C;
        real m = mean[i], s = rstd[i];
        real gmean = 0, gxmean = 0;
        for (int c = 0; c < C; c++) {
            real xh = (x[c] - m) * s;
            real g = w[c] * dy[c];
            gmean += g;
            gxmean += g * xh;
        }
        gmean = gmean / C;
        gxmean = gxmean / C;
        real* dx = dinp + (size_t)i * C;
        for (int c = 0; c < C; c++) {
            real xh = (x[c] - m) * s;
            real g = w[c] * dy[c];
            dx[c] += s * (g - gmean - xh * gxmean);
        }
    }
#pragma omp parallel for
    for (int c = 0; c < C; c++) {
        real sw = 0, sb = 0;
        for (int i = 0; i < N; i++) {
            real xh = (inp[(size_t)i * C + c] - mean[i]) * rstd[i];
            real dy = dout[(size_t)i * C + c];
            sw += dy * xh;
            sb += dy;
        }
        dw[c] += sw;
        db[c] += sb;
    }
}

/* RMSNorm, the normalisation of the Llama-style layers the pages name as other model
 * families (新智元 article, 纯CUDA也可训; lianzai README, 项目简介): no mean subtraction
 * and no bias; r = 1/sqrt(mean(x^2) + eps), y = x * r * w.  The pages give no formula:
 * this is the published RMSNorm (Zhang & Sennrich, 2019), with eps = 1e-5 like the
 * LayerNorm here.  r is kept for the backward. */
EXPORT void oracle_rmsnorm_forward(real* out, real* rstd, const real* inp, const real* w,
                                   int N, int C, real eps) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* x = inp + (size_t)i * C;
        real ms = 0;
        for (int c = 0; c < C; c++) ms += x[c] * x[c];
        ms = ms / C;
        real s = (real)1 / R_SQRT(ms + eps);
        real* y = out + (size_t)i * C;
        for (int c = 0; c < C; c++) y[c] = x[c] * s * w[c];
        rstd[i] = s;
    }
}

/* RMSNorm backward, by hand from the forward: with xh = x*r and g = w*dy,
 * dr/dx_j = -r^3 x_j / C gives dx += r * (g - xh * mean(g*xh)); dw += sum_rows dy*xh. */
EXPORT void oracle_rmsnorm_backward(real* dinp, real* dw, const real* dout, const real* inp,
                                    const real* w, const real* rstd, int N, int C) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* x = inp + (size_t)i * C;
        const real* dy = dout + (size_t)i * C;
        real s = rstd[i];
        real gxmean = 0;
        for (int c = 0; c < C; c++) gxmean += w[c] * dy[c] * x[c] * s;
        gxmean = gxmean / C;
        real* dx = dinp + (size_t)i * C;
        for (int c = 0; c < C; c++) dx[c] += s * (w[c] * dy[c] - x[c] * s * gxmean);
    }
#pragma omp parallel for
    for (int c = 0; c < C; c++) {
        real sw = 0;
        for (int i = 0; i < N; i++) sw += dout[(size_t)i * C + c] * inp[(size_t)i * C + c] * rstd[i];
        dw[c] += sw;
    }
}

/* Rotary position embedding, the positional encoding of the same Llama-style layers (the
 * pages name it as a variant, not its formula): the published RoPE (Su et al., 2021).
 * In every head of q and k, dimension pair (2i, 2i+1) at position t (restarting at 0 in
 * every row) is rotated by the angle t * 10000^(-2i/hs):
 *   q'[2i] = q[2i] cos - q[2i+1] sin,  q'[2i+1] = q[2i] sin + q[2i+1] cos;  v is copied.
 * inp and out are (B, T, 3C) with q, k, v the column blocks. */
EXPORT void oracle_rope_forward(real* out, const real* inp, int B, int T, int C, int NH) {
    int hs = C / NH;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const real* x = inp + ((size_t)b * T + t) * 3 * C;
            real* y = out + ((size_t)b * T + t) * 3 * C;
            for (int c = 0; c < 3 * C; c++) y[c] = x[c];
            for (int part = 0; part < 2; part++)
                for (int h = 0; h < NH; h++)
                    for (int i = 0; i < hs / 2; i++) {
                        real ang = (real)t * R_POW((real)10000, -(real)(2 * i) / (real)hs);
                        real cs = R_COS(ang), sn = R_SIN(ang);
                        size_t o = (size_t)part * C + (size_t)h * hs + 2 * i;
                        y[o] = x[o] * cs - x[o + 1] * sn;
                        y[o + 1] = x[o] * sn + x[o + 1] * cs;
                    }
        }
}

/* Backward: a rotation's transpose is the rotation by the opposite angle, so
 * dinp += R(-angle) dout on q and k, and dinp += dout on v. */
EXPORT void oracle_rope_backward(real* dinp, const real* dout, int B, int T, int C, int NH) {
    int hs = C / NH;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const real* d = dout + ((size_t)b * T + t) * 3 * C;
            real* dx = dinp + ((size_t)b * T + t) * 3 * C;
            for (int c = 2 * C; c < 3 * C; c++) dx[c] += d[c];
            for (int part = 0; part < 2; part++)
                for (int h = 0; h < NH; h++)
                    for (int i = 0; i < hs / 2; i++) {
                        real ang = (real)t * R_POW((real)10000, -(real)(2 * i) / (real)hs);
                        real cs = R_COS(ang), sn = R_SIN(ang);
                        size_t o = (size_t)part * C + (size_t)h * hs + 2 * i;
                        dx[o] += d[o] * cs + d[o + 1] * sn;
                        dx[o + 1] += -d[o] * sn + d[o + 1] * cs;
                    }
        }
}

/* Linear layer: out[r,o] = bias[o] + sum_{i=0..IC-1} inp[r,i] * w[o,i], with w stored
 * (OC, IC) row-major like PyTorch's Linear (the pages stress layer-for-layer
 * compatibility with PyTorch, huxiu 傻瓜式复现GPT-2).  bias may be NULL.
 * w is first copied transposed so the inner loop runs along outputs; each output's
 * sum still starts from the bias and adds i = 0, 1, ... in order. */
#define MM_ROWS 8
#define MM_COLS 256
EXPORT void oracle_matmul_forward(real* out, const real* inp, const real* w, const real* bias,
                                  int N, int IC, int OC) {
    real* wt = (real*)malloc((size_t)IC * OC * sizeof(real));
#pragma omp parallel for
    for (int i = 0; i < IC; i++)
        for (int o = 0; o < OC; o++) wt[(size_t)i * OC + o] = w[(size_t)o * IC + i];
    int nrb = (N + MM_ROWS - 1) / MM_ROWS, ncb = (OC + MM_COLS - 1) / MM_COLS;
#pragma omp parallel for collapse(2) schedule(static)
    for (int rb = 0; rb < nrb; rb++)
        for (int cb = 0; cb < ncb; cb++) {
            real acc[MM_ROWS][MM_COLS];
            int r0 = rb * MM_ROWS, o0 = cb * MM_COLS;
            int nr = N - r0 < MM_ROWS ? N - r0 : MM_ROWS;
            int no = OC - o0 < MM_COLS ? OC - o0 : MM_COLS;
            for (int r = 0; r < nr; r++)
                for (int o = 0; o < no; o++) acc[r][o] = bias ? bias[o0 + o] : (real)0;
            for (int i = 0; i < IC; i++) {
                const real* wrow = wt + (size_t)i * OC + o0;
                for (int r = 0; r < nr; r++) {
                    real a = inp[(size_t)(r0 + r) * IC + i];
                    for (int o = 0; o < no; o++) acc[r][o] += a * wrow[o];
                }
            }
            for (int r = 0; r < nr; r++)
                for (int o = 0; o < no; o++) out[(size_t)(r0 + r) * OC + o0 + o] = acc[r][o];
        }
    free(wt);
}

/* Linear backward:  dinp[r,i] += sum_o dout[r,o] w[o,i];  dw[o,i] += sum_r dout[r,o] inp[r,i];
 * dbias[o] += sum_r dout[r,o].  Sums run in index order (o, then r); dbias may be NULL. */
EXPORT void oracle_matmul_backward(real* dinp, real* dw, real* dbias, const real* dout,
                                   const real* inp, const real* w, int N, int IC, int OC) {
    int nrb = (N + MM_ROWS - 1) / MM_ROWS, ncb = (IC + MM_COLS - 1) / MM_COLS;
#pragma omp parallel for collapse(2) schedule(static)
    for (int rb = 0; rb < nrb; rb++)
        for (int cb = 0; cb < ncb; cb++) {
            real acc[MM_ROWS][MM_COLS];
            int r0 = rb * MM_ROWS, i0 = cb * MM_COLS;
            int nr = N - r0 < MM_ROWS ? N - r0 : MM_ROWS;
            int ni = IC - i0 < MM_COLS ? IC - i0 : MM_COLS;
            for (int r = 0; r < nr; r++)
                for (int i = 0; i < ni; i++) acc[r][i] = dinp[(size_t)(r0 + r) * IC + i0 + i];
            for (int o = 0; o < OC; o++) {
                const real* wrow = w + (size_t)o * IC + i0;
                for (int r = 0; r < nr; r++) {
                    real d = dout[(size_t)(r0 + r) * OC + o];
                    for (int i = 0; i < ni; i++) acc[r][i] += d * wrow[i];
                }
            }
            for (int r = 0; r < nr; r++)
                for (int i = 0; i < ni; i++) dinp[(size_t)(r0 + r) * IC + i0 + i] = acc[r][i];
        }
    int nob = (OC + MM_ROWS - 1) / MM_ROWS;
#pragma omp parallel for collapse(2) schedule(static)
    for (int ob = 0; ob < nob; ob++)
        for (int cb = 0; cb < ncb; cb++) {
            real acc[MM_ROWS][MM_COLS];
            int o0 = ob * MM_ROWS, i0 = cb * MM_COLS;
            int no = OC - o0 < MM_ROWS ? OC - o0 : MM_ROWS;
            int ni = IC - i0 < MM_COLS ? IC - i0 : MM_COLS;
            for (int o = 0; o < no; o++)
                for (int i = 0; i < ni; i++) acc[o][i] = dw[(size_t)(o0 + o) * IC + i0 + i];
            for (int r = 0; r < N; r++) {
                const real* xrow = inp + (size_t)r * IC + i0;
                for (int o = 0; o < no; o++) {
                    real d = dout[(size_t)r * OC + o0 + o];
                    for (int i = 0; i < ni; i++) acc[o][i] += d * xrow[i];
                }
            }
            for (int o = 0; o < no; o++)
                for (int i = 0; i < ni; i++) dw[(size_t)(o0 + o) * IC + i0 + i] = acc[o][i];
        }
    if (dbias) {
#pragma omp parallel for
        for (int o = 0; o < OC; o++) {
            real s = 0;
            for (int r = 0; r < N; r++) s += dout[(size_t)r * OC + o];
            dbias[o] += s;
        }
    }
}

/* bfloat16 rounding, for the mixed-precision variant (the pages name mixed precision
 * as llm.c's next step: 新智元 article "千行C代码训完GPT-2", 纯CUDA也可训 and its
 * outlook; OpenAI创始大神手搓千行C代码训练GPT, opening).  bfloat16 keeps the float
 * exponent range and 8 significant bits (7 stored); a value is rounded to the nearest
 * such number, ties to the one with an even last bit.  Written from that definition:
 * x = m 2^e with 0.5 <= |m| < 1, and m 2^8 is rounded to an integer (nearbyint rounds
 * ties to even in the default rounding mode).  Values below the normal bfloat16 range,
 * infinities and NaN are outside what the model produces and are passed through. */
EXPORT real oracle_bf16_round(real x) {
    if (x == 0 || !isfinite(x)) return x;
    int e;
    double m = frexp((double)x, &e);
    return (real)ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

EXPORT void oracle_bf16_round_array(real* dst, const real* src, size_t n) {
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) dst[i] = oracle_bf16_round(src[i]);
}

/* Causal multi-head self-attention (huxiu 傻瓜式复现GPT-2 names multi-head attention;
 * mask, scale and head split are the plain GPT-2 reading).  inp is (B,T,3C) holding
 * q | k | v; head h uses channels [h*hs, (h+1)*hs) of each, hs = C/NH.
 * preatt[b,h,t,u] = (q_t . k_u) / sqrt(hs) for u <= t; att = softmax over u <= t
 * (max subtracted); entries u > t are exactly 0 in both; out_t = sum_u att[t,u] v_u. */
EXPORT void oracle_attention_forward(real* out, real* preatt, real* att, const real* inp,
                                     int B, int T, int C, int NH) {
    int hs = C / NH;
    int C3 = 3 * C;
    real scale = (real)1 / R_SQRT((real)hs);
#pragma omp parallel for collapse(3)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++)
            for (int h = 0; h < NH; h++) {
                const real* q = inp + ((size_t)b * T + t) * C3 + h * hs;
                real* pre = preatt + (((size_t)b * NH + h) * T + t) * T;
                real* a = att + (((size_t)b * NH + h) * T + t) * T;
                real mx = -INFINITY;
                for (int u = 0; u <= t; u++) {
                    const real* k = inp + ((size_t)b * T + u) * C3 + C + h * hs;
                    real dot = 0;
                    for (int i = 0; i < hs; i++) dot += q[i] * k[i];
                    pre[u] = dot * scale;
                    if (pre[u] > mx) mx = pre[u];
                }
                real sum = 0;
                for (int u = 0; u <= t; u++) {
                    a[u] = R_EXP(pre[u] - mx);
                    sum += a[u];
                }
                real inv = (real)1 / sum;
                for (int u = 0; u <= t; u++) a[u] *= inv;
                for (int u = t + 1; u < T; u++) {
                    a[u] = 0;
                    pre[u] = 0;
                }
                real* o = out + ((size_t)b * T + t) * C + h * hs;
                for (int i = 0; i < hs; i++) o[i] = 0;
                for (int u = 0; u <= t; u++) {
                    const real* v = inp + ((size_t)b * T + u) * C3 + 2 * C + h * hs;
                    for (int i = 0; i < hs; i++) o[i] += a[u] * v[i];
                }
            }
}

/* Attention backward, derived from the forward:
 *   datt[t,u] = dout_t . v_u;   dv_u += att[t,u] dout_t;
 *   dpreatt[t,u] = att[t,u] (datt[t,u] - sum_w att[t,w] datt[t,w])   (softmax backward);
 *   dq_t += scale sum_u dpreatt[t,u] k_u;   dk_u += scale dpreatt[t,u] q_t.
 * Parallel over (b,h) only: each pair writes its own head's columns of dinp. */
EXPORT void oracle_attention_backward(real* dinp, real* dpreatt, real* datt, const real* dout,
                                      const real* inp, const real* att, int B, int T, int C,
                                      int NH) {
    int hs = C / NH;
    int C3 = 3 * C;
    real scale = (real)1 / R_SQRT((real)hs);
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                const real* a = att + (((size_t)b * NH + h) * T + t) * T;
                real* da = datt + (((size_t)b * NH + h) * T + t) * T;
                real* dpre = dpreatt + (((size_t)b * NH + h) * T + t) * T;
                const real* dy = dout + ((size_t)b * T + t) * C + h * hs;
                const real* q = inp + ((size_t)b * T + t) * C3 + h * hs;
                real* dq = dinp + ((size_t)b * T + t) * C3 + h * hs;
                for (int u = 0; u <= t; u++) {
                    const real* v = inp + ((size_t)b * T + u) * C3 + 2 * C + h * hs;
                    real* dv = dinp + ((size_t)b * T + u) * C3 + 2 * C + h * hs;
                    real s = 0;
                    for (int i = 0; i < hs; i++) {
                        s += dy[i] * v[i];
                        dv[i] += a[u] * dy[i];
                    }
                    da[u] += s;
                }
                real adot = 0;
                for (int w = 0; w <= t; w++) adot += a[w] * da[w];
                for (int u = 0; u <= t; u++) dpre[u] += a[u] * (da[u] - adot);
                for (int u = 0; u <= t; u++) {
                    const real* k = inp + ((size_t)b * T + u) * C3 + C + h * hs;
                    real* dk = dinp + ((size_t)b * T + u) * C3 + C + h * hs;
                    real g = dpre[u] * scale;
                    for (int i = 0; i < hs; i++) {
                        dq[i] += g * k[i];
                        dk[i] += g * q[i];
                    }
                }
            }
        }
}

/* GELU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).  The pages name a
 * GELU layer without its form (huxiu 核心代码解读 item 1); the tanh form is the one
 * GPT-2 was trained with, whose weights the pages fine-tune (skycaiji 快速入门). */
#define GELU_K0 0.7978845608028654 /* sqrt(2/pi) */
#define GELU_K1 0.044715
EXPORT void oracle_gelu_forward(real* out, const real* inp, size_t n) {
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        real u = inp[i];
        real z = (real)GELU_K0 * (u + (real)GELU_K1 * u * u * u);
        out[i] = (real)0.5 * u * ((real)1 + R_TANH(z));
    }
}

/* d/du of the tanh GELU: 0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) sqrt(2/pi) (1 + 3*0.044715 u^2). */
EXPORT void oracle_gelu_backward(real* dinp, const real* inp, const real* dout, size_t n) {
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        real u = inp[i];
        real z = (real)GELU_K0 * (u + (real)GELU_K1 * u * u * u);
        real th = R_TANH(z);
        real dz = (real)GELU_K0 * ((real)1 + (real)3 * (real)GELU_K1 * u * u);
        real g = (real)0.5 * ((real)1 + th) + (real)0.5 * u * ((real)1 - th * th) * dz;
        dinp[i] += g * dout[i];
    }
}

EXPORT void oracle_residual_forward(real* out, const real* a, const real* b, size_t n) {
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) out[i] = a[i] + b[i];
}

EXPORT void oracle_residual_backward(real* da, real* db, const real* dout, size_t n) {
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        da[i] += dout[i];
        db[i] += dout[i];
    }
}

/* Softmax over the whole vocabulary (no padding), max subtracted. */
EXPORT void oracle_softmax_forward(real* probs, const real* logits, int N, int V) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* z = logits + (size_t)i * V;
        real* p = probs + (size_t)i * V;
        real mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if (z[v] > mx) mx = z[v];
        real sum = 0;
        for (int v = 0; v < V; v++) {
            p[v] = R_EXP(z[v] - mx);
            sum += p[v];
        }
        for (int v = 0; v < V; v++) p[v] = p[v] / sum;
    }
}

/* sample_mult (huxiu page, 核心代码解读 item 5: draw an index from a probability
 * distribution): walk the distribution in index order, accumulating its mass, and
 * return the first index whose running total exceeds the coin; if rounding leaves the
 * total at or below the coin, the last index. */
EXPORT int oracle_sample_mult(const real* probs, int n, real coin) {
    real cdf = 0;
    for (int i = 0; i < n; i++) {
        cdf += probs[i];
        if (coin < cdf) return i;
    }
    return n - 1;
}

/* loss[i] = -log probs[i, target[i]]; every position counts (no ignored index). */
EXPORT void oracle_crossentropy_forward(real* losses, const real* probs, const int32_t* targets,
                                        int N, int V) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) losses[i] = -R_LOG(probs[(size_t)i * V + targets[i]]);
}

/* Fused softmax + cross-entropy backward: dlogits += (probs - onehot(target)) * dloss. */
EXPORT void oracle_crossentropy_softmax_backward(real* dlogits, const real* dlosses,
                                                 const real* probs, const int32_t* targets,
                                                 int N, int V) {
#pragma omp parallel for
    for (int i = 0; i < N; i++) {
        const real* p = probs + (size_t)i * V;
        real* d = dlogits + (size_t)i * V;
        for (int v = 0; v < V; v++) {
            real ind = v == targets[i] ? (real)1 : (real)0;
            d[v] += (p[v] - ind) * dlosses[i];
        }
    }
}

/* AdamW with decoupled weight decay on every element of the flat buffer (the pages
 * call the update AdamW, huxiu 核心代码解读 item 3, and run it at lr 1e-4, skycaiji
 * 快速入门).  t counts from 1; both moments start at 0:
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;  mh = m/(1-b1^t);  vh = v/(1-b2^t);
 *   p -= lr (mh / (sqrt(vh) + eps) + wd p). */
EXPORT void oracle_adamw(real* p, const real* g, real* m, real* v, size_t n, real lr,
                         real b1, real b2, real eps, real wd, int t) {
    real c1 = (real)1 - R_POW(b1, (real)t);
    real c2 = (real)1 - R_POW(b2, (real)t);
#pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        real mi = b1 * m[i] + ((real)1 - b1) * g[i];
        real vi = b2 * v[i] + ((real)1 - b2) * g[i] * g[i];
        m[i] = mi;
        v[i] = vi;
        real mh = mi / c1;
        real vh = vi / c2;
        p[i] -= lr * (mh / (R_SQRT(vh) + eps) + wd * p[i]);
    }
}

/* ------------------------------------------------------------------------- */
/* Model.                                                                    */
/* ------------------------------------------------------------------------- */

#define NPARAM 16
#define NACT 23
enum {
    A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_PREATT, A_ATT, A_ATTPROJ,
    A_RESIDUAL2, A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU, A_FCPROJ, A_RESIDUAL3,
    A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_PROBS, A_LOSSES
};

static int config_ok(const oracle_config* c) {
    return c && c->max_seq_len > 0 && c->vocab_size > 0 && c->num_layers > 0 &&
           c->num_heads > 0 && c->channels > 0 && c->channels % c->num_heads == 0;
}

/* The 16 parameter tensors, in the order the pages list them (huxiu 核心代码解读
 * item 2: token embedding, position embedding, LayerNorm, attention and MLP
 * parameters), biases on all four linears, a final LayerNorm, and the LM head tied
 * to wte (no separate head tensor).  This set reproduces the printed parameter count
 * of the 124M model (skycaiji 快速入门). */
static void param_sizes(const oracle_config* cfg, size_t len[NPARAM]) {
    size_t V = cfg->vocab_size, C = cfg->channels, L = cfg->num_layers, maxT = cfg->max_seq_len;
    len[0] = V * C;
    len[1] = maxT * C;
    len[2] = L * C;
    len[3] = L * C;
    len[4] = L * 3 * C * C;
    len[5] = L * 3 * C;
    len[6] = L * C * C;
    len[7] = L * C;
    len[8] = L * C;
    len[9] = L * C;
    len[10] = L * 4 * C * C;
    len[11] = L * 4 * C;
    len[12] = L * C * 4 * C;
    len[13] = L * C;
    len[14] = C;
    len[15] = C;
}

/* Every intermediate the plain forward keeps, including both (B,NH,T,T) attention
 * score tensors per layer.  This inventory reproduces the printed activation count of
 * the pages' run (skycaiji 快速入门). */
static void act_sizes(const oracle_config* cfg, int B, int T, size_t len[NACT]) {
    size_t C = cfg->channels, L = cfg->num_layers, NH = cfg->num_heads, V = cfg->vocab_size;
    size_t BT = (size_t)B * T;
    len[A_ENCODED] = BT * C;
    len[A_LN1] = L * BT * C;
    len[A_LN1_MEAN] = L * BT;
    len[A_LN1_RSTD] = L * BT;
    len[A_QKV] = L * BT * 3 * C;
    len[A_ATTY] = L * BT * C;
    len[A_PREATT] = L * B * NH * (size_t)T * T;
    len[A_ATT] = L * B * NH * (size_t)T * T;
    len[A_ATTPROJ] = L * BT * C;
    len[A_RESIDUAL2] = L * BT * C;
    len[A_LN2] = L * BT * C;
    len[A_LN2_MEAN] = L * BT;
    len[A_LN2_RSTD] = L * BT;
    len[A_FCH] = L * BT * 4 * C;
    len[A_FCH_GELU] = L * BT * 4 * C;
    len[A_FCPROJ] = L * BT * C;
    len[A_RESIDUAL3] = L * BT * C;
    len[A_LNF] = BT * C;
    len[A_LNF_MEAN] = BT;
    len[A_LNF_RSTD] = BT;
    len[A_LOGITS] = BT * V;
    len[A_PROBS] = BT * V;
    len[A_LOSSES] = BT;
}

EXPORT size_t oracle_gpt2_num_parameters(const oracle_config* cfg) {
    if (!config_ok(cfg)) return 0;
    size_t len[NPARAM], n = 0;
    param_sizes(cfg, len);
    for (int i = 0; i < NPARAM; i++) n += len[i];
    return n;
}

EXPORT int oracle_gpt2_param_layout(const oracle_config* cfg, size_t off[NPARAM], size_t len[NPARAM]) {
    if (!config_ok(cfg)) return O_EINVAL;
    param_sizes(cfg, len);
    size_t o = 0;
    for (int i = 0; i < NPARAM; i++) {
        off[i] = o;
        o += len[i];
    }
    return O_OK;
}

EXPORT size_t oracle_gpt2_num_activations(const oracle_config* cfg, int B, int T) {
    if (!config_ok(cfg) || B <= 0 || T <= 0) return 0;
    size_t len[NACT], n = 0;
    act_sizes(cfg, B, T, len);
    for (int i = 0; i < NACT; i++) n += len[i];
    return n;
}

typedef struct oracle_gpt2 {
    oracle_config cfg;
    int maxB, maxT;      /* shape the arenas were sized for */
    int B, T;            /* shape of the last forward */
    real *params, *grads, *m, *v;
    size_t num_params;
    real* p[NPARAM];     /* parameter tensors inside params */
    real* gp[NPARAM];    /* same inside grads */
    real* acts;          /* one block for every activation */
    real* dacts;         /* one block for every activation gradient */
    size_t num_acts;
    real* a[NACT];
    real* da[NACT];
    int32_t* inputs;
    int32_t* targets;
    int have_targets;
    int have_forward;
    real mean_loss;
    int last_error;
    int variant;         /* ORACLE_VARIANT_* bits */
    real* qkvr;          /* rotary variant: q and k rotated, per layer (L, B, T, 3C) */
    real* dqkvr;
} oracle_gpt2;

/* Llama-style layer variants: RMSNorm in place of every LayerNorm (the
 * LayerNorm biases then take no part and keep zero gradients), and rotary position
 * embedding on q and k in place of the position rows (wpe then takes no part). */
#define ORACLE_VARIANT_RMSNORM 1
#define ORACLE_VARIANT_ROPE 2
/* Mixed precision (bfloat16 rounding defined at oracle_bf16_round): every linear layer and the LM head multiply the
 * bfloat16 roundings of their two operands (input and weight forward; output gradient
 * and weight, or output gradient and input, backward), the products summed exactly;
 * the bias gradient sums the unrounded output gradient.  Attention multiplies the
 * roundings of q, k, v (forward and backward) and of its output gradient (backward);
 * its probabilities and score gradients are not rounded.  Everything else -- the fp32
 * master weights, LayerNorm, GELU, residuals, softmax and cross-entropy, AdamW -- is
 * unchanged. */
#define ORACLE_VARIANT_BF16 4

static void carve(oracle_gpt2* g, int B, int T) {
    size_t len[NACT];
    act_sizes(&g->cfg, B, T, len);
    size_t o = 0;
    for (int i = 0; i < NACT; i++) {
        g->a[i] = g->acts + o;
        g->da[i] = g->dacts ? g->dacts + o : NULL;
        o += len[i];
    }
}

/* The activation-gradient block, allocated on first use. */
static int ensure_dacts(oracle_gpt2* g) {
    if (!g->grads) return O_ESTATE;
    if (!g->dacts) {
        g->dacts = (real*)calloc(g->num_acts, sizeof(real));
        if (!g->dacts) return O_ENOMEM;
        carve(g, g->B ? g->B : g->maxB, g->T ? g->T : g->maxT);
    }
    return O_OK;
}

/* Build: borrow the caller-owned flat buffers (params already initialised; grads, m,
 * v zeroed here), allocate the activation block once.  grads, m and v may all be NULL
 * for a forward-only model; the activation-gradient block is allocated on the first
 * zero_grad or backward. */
EXPORT int oracle_gpt2_build_variant(oracle_gpt2** out, const oracle_config* cfg, int B, int T,
                                     real* params, real* grads, real* m, real* v, int variant) {
    if (!out || !config_ok(cfg) || B <= 0 || T <= 0 || T > cfg->max_seq_len || !params)
        return O_EINVAL;
    if (variant & ~(ORACLE_VARIANT_RMSNORM | ORACLE_VARIANT_ROPE | ORACLE_VARIANT_BF16)) return O_EINVAL;
    if ((variant & ORACLE_VARIANT_ROPE) && (cfg->channels / cfg->num_heads) % 2) return O_EINVAL;
    if ((grads || m || v) && !(grads && m && v)) return O_EINVAL;
    oracle_gpt2* g = (oracle_gpt2*)calloc(1, sizeof(oracle_gpt2));
    if (!g) return O_ENOMEM;
    g->cfg = *cfg;
    g->variant = variant;
    g->maxB = B;
    g->maxT = T;
    g->params = params;
    g->grads = grads;
    g->m = m;
    g->v = v;
    g->num_params = oracle_gpt2_num_parameters(cfg);
    size_t off[NPARAM], len[NPARAM];
    oracle_gpt2_param_layout(cfg, off, len);
    for (int i = 0; i < NPARAM; i++) {
        g->p[i] = params + off[i];
        g->gp[i] = grads ? grads + off[i] : NULL;
    }
    if (grads) {
        memset(grads, 0, g->num_params * sizeof(real));
        memset(m, 0, g->num_params * sizeof(real));
        memset(v, 0, g->num_params * sizeof(real));
    }
    g->num_acts = oracle_gpt2_num_activations(cfg, B, T);
    g->acts = (real*)calloc(g->num_acts, sizeof(real));
    g->inputs = (int32_t*)calloc((size_t)B * T, sizeof(int32_t));
    g->targets = (int32_t*)calloc((size_t)B * T, sizeof(int32_t));
    if (variant & ORACLE_VARIANT_ROPE) {
        size_t n = (size_t)cfg->num_layers * B * T * 3 * cfg->channels;
        g->qkvr = (real*)calloc(n, sizeof(real));
        g->dqkvr = (real*)calloc(n, sizeof(real));
    }
    if (!g->acts || !g->inputs || !g->targets || ((variant & ORACLE_VARIANT_ROPE) && (!g->qkvr || !g->dqkvr))) {
        free(g->acts);
        free(g->dacts);
        free(g->inputs);
        free(g->targets);
        free(g->qkvr);
        free(g->dqkvr);
        free(g);
        return O_ENOMEM;
    }
    carve(g, B, T);
    *out = g;
    return O_OK;
}

EXPORT int oracle_gpt2_build(oracle_gpt2** out, const oracle_config* cfg, int B, int T,
                             real* params, real* grads, real* m, real* v) {
    return oracle_gpt2_build_variant(out, cfg, B, T, params, grads, m, v, 0);
}

EXPORT void oracle_gpt2_free(oracle_gpt2* g) {
    if (!g) return;
    free(g->qkvr);
    free(g->dqkvr);
    free(g->acts);
    free(g->dacts);
    free(g->inputs);
    free(g->targets);
    free(g);
}

EXPORT int oracle_gpt2_last_error(const oracle_gpt2* g) { return g ? g->last_error : O_EINVAL; }

/* The model's linear layers: plain, or on bfloat16-rounded operands (mixed-precision
 * variant).  The rounded copies are temporary; the stored activations stay unrounded. */
static real* bf16_copy(const real* x, size_t n) {
    real* r = (real*)malloc(n * sizeof(real));
    if (r) oracle_bf16_round_array(r, x, n);
    return r;
}

static int linear_forward(const oracle_gpt2* g, real* out, const real* inp, const real* w, const real* bias,
                          int N, int IC, int OC) {
    if (!(g->variant & ORACLE_VARIANT_BF16)) {
        oracle_matmul_forward(out, inp, w, bias, N, IC, OC);
        return O_OK;
    }
    real* ri = bf16_copy(inp, (size_t)N * IC);
    real* rw = bf16_copy(w, (size_t)OC * IC);
    int rc = ri && rw ? O_OK : O_ENOMEM;
    if (rc == O_OK) oracle_matmul_forward(out, ri, rw, bias, N, IC, OC);
    free(ri);
    free(rw);
    return rc;
}

static int linear_backward(const oracle_gpt2* g, real* dinp, real* dw, real* dbias, const real* dout,
                           const real* inp, const real* w, int N, int IC, int OC) {
    if (!(g->variant & ORACLE_VARIANT_BF16)) {
        oracle_matmul_backward(dinp, dw, dbias, dout, inp, w, N, IC, OC);
        return O_OK;
    }
    real* rd = bf16_copy(dout, (size_t)N * OC);
    real* ri = bf16_copy(inp, (size_t)N * IC);
    real* rw = bf16_copy(w, (size_t)OC * IC);
    int rc = rd && ri && rw ? O_OK : O_ENOMEM;
    if (rc == O_OK) {
        oracle_matmul_backward(dinp, dw, NULL, rd, ri, rw, N, IC, OC);
        if (dbias) {
#pragma omp parallel for
            for (int o = 0; o < OC; o++) {
                real s = 0;
                for (int r = 0; r < N; r++) s += dout[(size_t)r * OC + o];
                dbias[o] += s;
            }
        }
    }
    free(rd);
    free(ri);
    free(rw);
    return rc;
}

/* The block's normalisation: LayerNorm, or RMSNorm in the RMSNorm variant (whose mean
 * slot then holds 0 and whose bias takes no part). */
static void norm_forward(int rms, real* out, real* mean, real* rstd, const real* x, const real* w,
                         const real* b, int N, int C) {
    if (rms) {
        oracle_rmsnorm_forward(out, rstd, x, w, N, C, (real)1e-5);
        for (int i = 0; i < N; i++) mean[i] = 0;
    } else {
        oracle_layernorm_forward(out, mean, rstd, x, w, b, N, C, (real)1e-5);
    }
}

static void norm_backward(int rms, real* dx, real* dw, real* db, const real* dy, const real* x, const real* w,
                          const real* mean, const real* rstd, int N, int C) {
    if (rms) oracle_rmsnorm_backward(dx, dw, dy, x, w, rstd, N, C);
    else oracle_layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, N, C);
}

/* Forward: GPT-2 pre-LN blocks,
 *   x = x + attproj(attention(qkv(ln1(x))));  x = x + fcproj(gelu(fc(ln2(x)))),
 * then the final LayerNorm, the tied LM head, softmax and cross-entropy.  Returns the
 * mean of the per-position losses (accumulated in double), -1 without targets, NaN on
 * invalid input (then last_error is set). */
EXPORT double oracle_gpt2_forward(oracle_gpt2* g, const int32_t* inputs, const int32_t* targets,
                                  int B, int T) {
    if (!g) return NAN;
    const oracle_config* cfg = &g->cfg;
    int V = cfg->vocab_size, C = cfg->channels, L = cfg->num_layers, NH = cfg->num_heads;
    if (!inputs || B <= 0 || T <= 0 || T > cfg->max_seq_len || (size_t)B * T > (size_t)g->maxB * g->maxT) {
        g->last_error = O_EINVAL;
        return NAN;
    }
    for (int i = 0; i < B * T; i++)
        if (inputs[i] < 0 || inputs[i] >= V || (targets && (targets[i] < 0 || targets[i] >= V))) {
            g->last_error = O_EINVAL;
            return NAN;
        }
    g->last_error = O_OK;
    g->B = B;
    g->T = T;
    carve(g, B, T);
    memcpy(g->inputs, inputs, (size_t)B * T * sizeof(int32_t));
    if (targets) memcpy(g->targets, targets, (size_t)B * T * sizeof(int32_t));
    g->have_targets = targets != NULL;

    real** P = g->p;
    real** A = g->a;
    size_t BT = (size_t)B * T;
    size_t att_l = (size_t)B * NH * T * T;
    const int rms = g->variant & ORACLE_VARIANT_RMSNORM, rope = g->variant & ORACLE_VARIANT_ROPE;
    int bad = 0;  /* a linear layer could not allocate its rounded operands */
    oracle_encoder_forward(A[A_ENCODED], inputs, P[0], rope ? NULL : P[1], B, T, C);
    for (int l = 0; l < L; l++) {
        real* residual = l == 0 ? A[A_ENCODED] : A[A_RESIDUAL3] + (size_t)(l - 1) * BT * C;
        real* ln1 = A[A_LN1] + l * BT * C;
        real* ln1m = A[A_LN1_MEAN] + l * BT;
        real* ln1r = A[A_LN1_RSTD] + l * BT;
        real* qkv = A[A_QKV] + l * BT * 3 * C;
        real* atty = A[A_ATTY] + l * BT * C;
        real* preatt = A[A_PREATT] + l * att_l;
        real* att = A[A_ATT] + l * att_l;
        real* attproj = A[A_ATTPROJ] + l * BT * C;
        real* res2 = A[A_RESIDUAL2] + l * BT * C;
        real* ln2 = A[A_LN2] + l * BT * C;
        real* ln2m = A[A_LN2_MEAN] + l * BT;
        real* ln2r = A[A_LN2_RSTD] + l * BT;
        real* fch = A[A_FCH] + l * BT * 4 * C;
        real* fchg = A[A_FCH_GELU] + l * BT * 4 * C;
        real* fcproj = A[A_FCPROJ] + l * BT * C;
        real* res3 = A[A_RESIDUAL3] + l * BT * C;
        norm_forward(rms, ln1, ln1m, ln1r, residual, P[2] + l * C, P[3] + l * C, (int)BT, C);
        bad |= linear_forward(g, qkv, ln1, P[4] + (size_t)l * 3 * C * C, P[5] + l * 3 * C, (int)BT, C, 3 * C);
        real* qkv_in = qkv;
        if (rope) {
            qkv_in = g->qkvr + (size_t)l * BT * 3 * C;
            oracle_rope_forward(qkv_in, qkv, B, T, C, NH);
        }
        if (g->variant & ORACLE_VARIANT_BF16) {
            /* attention multiplies the bf16 roundings of q, k and v (the probabilities
             * stay unrounded) */
            real* rq = bf16_copy(qkv_in, BT * 3 * C);
            bad |= rq ? O_OK : O_ENOMEM;
            if (rq) oracle_attention_forward(atty, preatt, att, rq, B, T, C, NH);
            free(rq);
        } else {
            oracle_attention_forward(atty, preatt, att, qkv_in, B, T, C, NH);
        }
        bad |= linear_forward(g, attproj, atty, P[6] + (size_t)l * C * C, P[7] + l * C, (int)BT, C, C);
        oracle_residual_forward(res2, residual, attproj, BT * C);
        norm_forward(rms, ln2, ln2m, ln2r, res2, P[8] + l * C, P[9] + l * C, (int)BT, C);
        bad |= linear_forward(g, fch, ln2, P[10] + (size_t)l * 4 * C * C, P[11] + l * 4 * C, (int)BT, C, 4 * C);
        oracle_gelu_forward(fchg, fch, BT * 4 * C);
        bad |= linear_forward(g, fcproj, fchg, P[12] + (size_t)l * 4 * C * C, P[13] + l * C, (int)BT, 4 * C, C);
        oracle_residual_forward(res3, res2, fcproj, BT * C);
    }
    real* last = A[A_RESIDUAL3] + (size_t)(L - 1) * BT * C;
    norm_forward(rms, A[A_LNF], A[A_LNF_MEAN], A[A_LNF_RSTD], last, P[14], P[15], (int)BT, C);
    bad |= linear_forward(g, A[A_LOGITS], A[A_LNF], P[0], NULL, (int)BT, C, V);
    if (bad) {
        g->last_error = O_ENOMEM;
        return NAN;
    }
    oracle_softmax_forward(A[A_PROBS], A[A_LOGITS], (int)BT, V);
    g->have_forward = 1;
    if (!targets) {
        g->mean_loss = -1;
        return -1.0;
    }
    oracle_crossentropy_forward(A[A_LOSSES], A[A_PROBS], targets, (int)BT, V);
    double s = 0;
    for (size_t i = 0; i < BT; i++) s += (double)A[A_LOSSES][i];
    g->mean_loss = (real)(s / (double)BT);
    return s / (double)BT;
}

/* Zero the gradients of the parameters and of every activation (huxiu 核心代码解读
 * item 3 says zero_grad clears both). */
EXPORT int oracle_gpt2_zero_grad(oracle_gpt2* g) {
    if (!g) return O_EINVAL;
    int rc = ensure_dacts(g);
    if (rc != O_OK) return g->last_error = rc;
    memset(g->grads, 0, g->num_params * sizeof(real));
    memset(g->dacts, 0, g->num_acts * sizeof(real));
    return O_OK;
}

/* Backward: the loss is the mean over B*T positions, so every position's loss
 * gradient is 1/(B*T); then each layer's backward in reverse order, all adding.
 * Parameter gradients accumulate across calls (zero_grad resets them); activation
 * gradients belong to one call and are cleared first, so two calls without a
 * zero_grad in between give exactly twice the parameter gradients. */
EXPORT int oracle_gpt2_backward(oracle_gpt2* g) {
    if (!g) return O_EINVAL;
    if (!g->have_forward || !g->have_targets) {
        g->last_error = O_ESTATE;
        return O_ESTATE;
    }
    int rc = ensure_dacts(g);
    if (rc != O_OK) return g->last_error = rc;
    const oracle_config* cfg = &g->cfg;
    int B = g->B, T = g->T;
    int V = cfg->vocab_size, C = cfg->channels, L = cfg->num_layers, NH = cfg->num_heads;
    size_t BT = (size_t)B * T;
    size_t att_l = (size_t)B * NH * T * T;
    real** P = g->p;
    real** G = g->gp;
    real** A = g->a;
    real** D = g->da;
    memset(g->dacts, 0, g->num_acts * sizeof(real));
    const int rms = g->variant & ORACLE_VARIANT_RMSNORM, rope = g->variant & ORACLE_VARIANT_ROPE;
    if (rope) memset(g->dqkvr, 0, (size_t)L * BT * 3 * C * sizeof(real));
    int bad = 0;  /* a linear layer could not allocate its rounded operands */
    real dl = (real)1 / (real)BT;
    for (size_t i = 0; i < BT; i++) D[A_LOSSES][i] = dl;
    oracle_crossentropy_softmax_backward(D[A_LOGITS], D[A_LOSSES], A[A_PROBS], g->targets, (int)BT, V);
    bad |= linear_backward(g, D[A_LNF], G[0], NULL, D[A_LOGITS], A[A_LNF], P[0], (int)BT, C, V);
    real* last = A[A_RESIDUAL3] + (size_t)(L - 1) * BT * C;
    real* dlast = D[A_RESIDUAL3] + (size_t)(L - 1) * BT * C;
    norm_backward(rms, dlast, G[14], G[15], D[A_LNF], last, P[14], A[A_LNF_MEAN], A[A_LNF_RSTD], (int)BT, C);
    for (int l = L - 1; l >= 0; l--) {
        real* residual = l == 0 ? A[A_ENCODED] : A[A_RESIDUAL3] + (size_t)(l - 1) * BT * C;
        real* dresidual = l == 0 ? D[A_ENCODED] : D[A_RESIDUAL3] + (size_t)(l - 1) * BT * C;
        size_t o1 = l * BT * C, o3 = l * BT * 3 * C, o4 = l * BT * 4 * C, oa = l * att_l, os = l * BT;
        /* MLP half, backwards. */
        oracle_residual_backward(D[A_RESIDUAL2] + o1, D[A_FCPROJ] + o1, D[A_RESIDUAL3] + o1, BT * C);
        bad |= linear_backward(g, D[A_FCH_GELU] + o4, G[12] + (size_t)l * 4 * C * C, G[13] + l * C,
                               D[A_FCPROJ] + o1, A[A_FCH_GELU] + o4, P[12] + (size_t)l * 4 * C * C,
                               (int)BT, 4 * C, C);
        oracle_gelu_backward(D[A_FCH] + o4, A[A_FCH] + o4, D[A_FCH_GELU] + o4, BT * 4 * C);
        bad |= linear_backward(g, D[A_LN2] + o1, G[10] + (size_t)l * 4 * C * C, G[11] + l * 4 * C,
                               D[A_FCH] + o4, A[A_LN2] + o1, P[10] + (size_t)l * 4 * C * C,
                               (int)BT, C, 4 * C);
        norm_backward(rms, D[A_RESIDUAL2] + o1, G[8] + l * C, G[9] + l * C, D[A_LN2] + o1,
                      A[A_RESIDUAL2] + o1, P[8] + l * C, A[A_LN2_MEAN] + os, A[A_LN2_RSTD] + os, (int)BT, C);
        /* Attention half, backwards. */
        oracle_residual_backward(dresidual, D[A_ATTPROJ] + o1, D[A_RESIDUAL2] + o1, BT * C);
        bad |= linear_backward(g, D[A_ATTY] + o1, G[6] + (size_t)l * C * C, G[7] + l * C,
                               D[A_ATTPROJ] + o1, A[A_ATTY] + o1, P[6] + (size_t)l * C * C,
                               (int)BT, C, C);
        {
            /* bf16 variant: the attention backward's products take the bf16 roundings of
             * q, k, v and of the output gradient; probabilities and score gradients stay
             * unrounded (the softmax backward is unchanged) */
            const int bf = g->variant & ORACLE_VARIANT_BF16;
            const real* ain = rope ? g->qkvr + o3 : A[A_QKV] + o3;
            const real* adout = D[A_ATTY] + o1;
            real* rin = bf ? bf16_copy(ain, BT * 3 * C) : NULL;
            real* rdout = bf ? bf16_copy(adout, BT * C) : NULL;
            if (bf && (!rin || !rdout)) {
                bad |= O_ENOMEM;
            } else {
                oracle_attention_backward(rope ? g->dqkvr + o3 : D[A_QKV] + o3, D[A_PREATT] + oa, D[A_ATT] + oa,
                                          bf ? rdout : adout, bf ? rin : ain, A[A_ATT] + oa, B, T, C, NH);
            }
            free(rin);
            free(rdout);
            if (rope) oracle_rope_backward(D[A_QKV] + o3, g->dqkvr + o3, B, T, C, NH);
        }
        bad |= linear_backward(g, D[A_LN1] + o1, G[4] + (size_t)l * 3 * C * C, G[5] + l * 3 * C,
                               D[A_QKV] + o3, A[A_LN1] + o1, P[4] + (size_t)l * 3 * C * C,
                               (int)BT, C, 3 * C);
        norm_backward(rms, dresidual, G[2] + l * C, G[3] + l * C, D[A_LN1] + o1, residual,
                      P[2] + l * C, A[A_LN1_MEAN] + os, A[A_LN1_RSTD] + os, (int)BT, C);
    }
    oracle_encoder_backward(G[0], rope ? NULL : G[1], D[A_ENCODED], g->inputs, B, T, C);
    if (bad) return g->last_error = O_ENOMEM;
    return O_OK;
}

EXPORT int oracle_gpt2_update(oracle_gpt2* g, real lr, real b1, real b2, real eps, real wd, int t) {
    if (!g) return O_EINVAL;
    if (t < 1 || !g->grads) {
        g->last_error = O_ESTATE;
        return O_ESTATE;
    }
    oracle_adamw(g->params, g->grads, g->m, g->v, g->num_params, lr, b1, b2, eps, wd, t);
    return O_OK;
}

/* Pointer to activation tensor `id` (layer `layer` for per-layer tensors) at the shape
 * of the last forward; *count gets its element count.  grad != 0 selects the
 * activation-gradient block instead. */
EXPORT real* oracle_gpt2_activation(oracle_gpt2* g, int id, int layer, int grad, size_t* count) {
    if (g && id == NACT && g->qkvr) {  /* the rotary variant's rotated qkv, per layer */
        if (layer < 0 || layer >= g->cfg.num_layers) return NULL;
        size_t n = (size_t)(g->B ? g->B : g->maxB) * (g->T ? g->T : g->maxT) * 3 * g->cfg.channels;
        if (count) *count = n;
        return (grad ? g->dqkvr : g->qkvr) + (size_t)layer * n;
    }
    if (!g || id < 0 || id >= NACT) return NULL;
    size_t len[NACT];
    act_sizes(&g->cfg, g->B ? g->B : g->maxB, g->T ? g->T : g->maxT, len);
    int per_layer = id >= A_LN1 && id <= A_RESIDUAL3;
    size_t n = per_layer ? len[id] / g->cfg.num_layers : len[id];
    if (per_layer && (layer < 0 || layer >= g->cfg.num_layers)) return NULL;
    if (count) *count = n;
    real* base = grad ? g->da[id] : g->a[id];
    if (!base) return NULL;
    return base + (per_layer ? (size_t)layer * n : 0);
}
