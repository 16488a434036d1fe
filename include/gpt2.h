/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 fp32 training step.
 *
 * The library follows the decomposition the pages give for llm.c's train_gpt2.c
 * ("llm.c：Andrej Karpathy带你从零复现LLM", section 核心代码解读：train_gpt2.c):
 * a model config, a flat parameter tensor set, an activation set, and the calls
 * build, forward (outputs and loss), zero_grad, backward and an AdamW update.  As on
 * the pages, all memory is laid out once in flat 1-D buffers and never reallocated
 * ("OpenAI创始大神手搓千行C代码训练GPT", section 手动实现每个层前向 / 反向传播; 新智元
 * article "千行C代码训完GPT-2", section 纯CUDA也可训).  Checkpoint loading is replaced by
 * gpt2_build on caller-initialised parameters.
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory of the current
 *     HIP device; the library borrows them and never frees them.  Host pointers are
 *     only read during the call.
 *   - float buffers must be 16-byte aligned.
 *   - Work is enqueued on the hipStream_t passed to gpt2_build (or to the standalone
 *     calls); NULL means the default stream.  Only gpt2_forward synchronises.
 *   - A gpt2 handle is not thread-safe; calls on one handle must not overlap.
 *   - Errors: status codes below; gpt2_forward returns NaN and records the code,
 *     readable through gpt2_last_error.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model shape: the five fields the pages' log prints for GPT2Config (新智元 article,
 * 快速入门).  channels must be a multiple of num_heads and of 4; head size
 * channels/num_heads must be 16, 32 or 64. */
typedef struct gpt2_config {
    int max_seq_len;
    int vocab_size;
    int num_layers;
    int num_heads;
    int channels;
} gpt2_config;

typedef struct gpt2 gpt2; /* opaque model handle */

enum {
    GPT2_OK = 0,
    GPT2_EINVAL = -1,  /* bad argument, shape or token id */
    GPT2_ESTATE = -2,  /* call out of order (backward without a forward with targets, t < 1) */
    GPT2_EDEVICE = -3, /* a HIP call failed */
    GPT2_ENOMEM = -4,  /* host allocation failed */
    GPT2_ESCRATCH = -5 /* request larger than the library's fixed device scratch */
};

#define GPT2_NUM_PARAM_TENSORS 16

/* Number of parameters: V*C + maxT*C + L*(12*C*C + 13*C) + 2*C (124,439,808 for the
 * 124M shape the pages print).  0 for an invalid config.  Host-only. */
size_t gpt2_num_parameters(const gpt2_config* cfg);

/* Offsets and lengths (in floats) of the 16 parameter tensors inside the flat buffer,
 * in this order, each row-major, linear weights stored (out, in):
 *   wte (V,C), wpe (maxT,C), ln1w (L,C), ln1b (L,C), qkvw (L,3C,C), qkvb (L,3C),
 *   attprojw (L,C,C), attprojb (L,C), ln2w (L,C), ln2b (L,C), fcw (L,4C,C), fcb (L,4C),
 *   fcprojw (L,C,4C), fcprojb (L,C), lnfw (C), lnfb (C).
 * The order is the pages' ParameterTensors listing (huxiu page, 核心代码解读 item 2).
 * grads, m and v use the same offsets.  Host-only; returns GPT2_OK or GPT2_EINVAL. */
int gpt2_param_layout(const gpt2_config* cfg, size_t off[GPT2_NUM_PARAM_TENSORS],
                      size_t len[GPT2_NUM_PARAM_TENSORS]);

/* Sizes (in floats) of the two arenas a model of batch shape (B, T) needs: the
 * activation arena and the gradient scratch arena.  Host-only.  In the fp32 variants the
 * scratch also holds the attention's raw scores of every layer and one layer's score
 * gradients (B x heads 64x64 blocks per causal pair of 64-position tiles each: about
 * 2.8 GB in all for GPT-2 124M at B=8, T=1024); the backward falls back to recomputing
 * them for batch shapes whose pairs do not fit. */
int gpt2_arena_sizes(const gpt2_config* cfg, int B, int T, size_t* n_acts, size_t* n_grad_scratch);
/* The same for a model built with gpt2_build_variant(..., variant): GPT2_VARIANT_BF16
 * adds the bfloat16 operand copies (weights, their transposes and the linear layers'
 * inputs in the activation arena; the output-gradient copies in the scratch).
 * GPT2_EINVAL for an unknown bit. */
int gpt2_arena_sizes_variant(const gpt2_config* cfg, int B, int T, int variant, size_t* n_acts,
                             size_t* n_grad_scratch);

/* The six caller-owned device buffers.  params, grads, m, v hold
 * gpt2_num_parameters floats each; acts and grad_scratch the sizes gpt2_arena_sizes
 * returns.  They must outlive the handle. */
typedef struct gpt2_buffers {
    float* params;
    float* grads;
    float* m;
    float* v;
    float* acts;
    float* grad_scratch;
} gpt2_buffers;

/* Validate the config, carve the arenas for batches of at most B*T positions with
 * T <= max_seq_len, zero grads, m and v on `stream` (a hipStream_t or NULL).  The caller
 * writes the initial parameters.  *out receives the handle.  Allocates only a small
 * host struct and a small pinned host block for the loss read-back. */
int gpt2_build(gpt2** out, const gpt2_config* cfg, int B, int T, const gpt2_buffers* bufs,
               void* stream);

/* Model variants, a bit mask.  The Llama-style layers: the pages name Llama 2, Gemma and
 * Mistral as further llm.c targets (新智元 article 纯CUDA也可训) but give no formulas, so
 * the published definitions are used:
 *   GPT2_VARIANT_RMSNORM: every LayerNorm becomes RMSNorm, y = x r w with
 *     r = 1/sqrt(mean(x^2) + 1e-5); no mean subtraction, no bias (ln1b, ln2b, lnfb take no
 *     part and keep zero gradients; their mean activations read 0);
 *   GPT2_VARIANT_ROPE: no position rows (wpe takes no part); after the qkv projection, in
 *     every head of q and k the pair (2i, 2i+1) at position t is rotated by
 *     t * 10000^(-2i/hs); the qkv activation then holds the rotated q and k.  Needs an
 *     even head size.
 * Mixed precision, the pages' stated next step for llm.c (新智元 article 纯CUDA也可训;
 * "OpenAI创始大神手搓千行C代码训练GPT", opening):
 *   GPT2_VARIANT_BF16: every linear layer and the LM head multiply the bfloat16 roundings
 *     (nearest, ties to even) of their two operands on the bf16 matrix cores, summing the
 *     products in fp32: forward input and weight; backward output gradient and weight
 *     (dgrad), output gradient and input (wgrad).  Bias gradients sum the unrounded fp32
 *     output gradient.  Parameters, gradients, AdamW moments, every activation and every
 *     other operation (LayerNorm, attention, GELU, softmax, cross-entropy, AdamW) stay
 *     fp32.  Needs C a multiple of 8, and the larger arenas gpt2_arena_sizes_variant gives.
 * The parameter layout, buffers and every other call are those of gpt2_build (variant 0).
 * Returns as gpt2_build, and GPT2_EINVAL for an unknown bit, an odd head size with
 * GPT2_VARIANT_ROPE or C not a multiple of 8 with GPT2_VARIANT_BF16. */
#define GPT2_VARIANT_RMSNORM 1
#define GPT2_VARIANT_ROPE 2
#define GPT2_VARIANT_BF16 4
int gpt2_build_variant(gpt2** out, const gpt2_config* cfg, int B, int T, const gpt2_buffers* bufs, void* stream,
                       int variant);

/* Forward pass (huxiu page 核心代码解读 item 3: outputs and loss).  inputs and targets
 * are device pointers to B*T int32 token ids, row-major (B,T); ids must lie in
 * [0, vocab_size).  Requires 1 <= T <= max_seq_len and B*T <= the built B*T; a model
 * built with GPT2_VARIANT_BF16 also requires B*ceil64(T) <= B0*ceil64(T0), where (B0, T0)
 * is the built shape and ceil64 rounds up to a multiple of 64 (its per-head attention
 * copies are sized in whole 64-position tiles).
 * Returns the mean cross-entropy over the B*T positions.  With targets == NULL the
 * logits and each row's log-sum-exp (which gives the softmax) are computed and -1.0f is
 * returned.  Synchronises the
 * stream.  Returns NaN on error (GPT2_EINVAL for bad shapes or token ids found on the
 * device, GPT2_EDEVICE for a HIP failure). */
float gpt2_forward(gpt2* model, const int32_t* inputs, const int32_t* targets, int B, int T);

/* Zero the gradients (huxiu page 核心代码解读 item 3: zero_grad clears the gradients of
 * the parameters and of the activations).  Here the activation gradients are scratch
 * that each backward rewrites, so only the parameter gradients need clearing.  Enqueue
 * only. */
int gpt2_zero_grad(gpt2* model);

/* Backward pass of the last forward (huxiu page 核心代码解读 item 3: the hand-derived
 * backward of every layer, from the loss back to the embeddings), which must have had
 * targets, else GPT2_ESTATE.  ADDS into grads: two calls without gpt2_zero_grad give
 * twice the gradients.  Enqueue only. */
int gpt2_backward(gpt2* model);

/* AdamW over the whole flat buffer (huxiu page 核心代码解读 item 3; lr 1e-4 on the
 * 新智元 page 快速入门):  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 * p -= lr * (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + weight_decay * p).
 * t is the 1-based step count (GPT2_ESTATE if t < 1).  Enqueue only. */
int gpt2_update(gpt2* model, float lr, float beta1, float beta2, float eps, float weight_decay,
                int t);

/* gpt2_backward followed by gpt2_update(lr, beta1, beta2, eps, weight_decay, t) in one
 * call, bitwise the same result: every parameter gets the same elementwise AdamW.  Each
 * layer's parameters are updated as soon as its gradients are final (after its
 * LayerNorm backward and weight-gradient GEMMs), on a third stream the handle owns (the
 * update stream, next to the main and weight-gradient streams), while the gradients of
 * the layers below are still being formed; the layers' LayerNorm weight and bias
 * gradients are also summed there, just before their update.  wte, wpe and the final
 * norm are updated last.  Gradients are left in `grads` as gpt2_backward leaves them.
 * Returns GPT2_OK, GPT2_EINVAL for a null model, GPT2_ESTATE without a forward with
 * targets or with t < 1, GPT2_EDEVICE on a HIP error. */
int gpt2_backward_update(gpt2* model, float lr, float beta1, float beta2, float eps, float weight_decay, int t);

/* Last error recorded on the handle (GPT2_OK if none). */
int gpt2_last_error(const gpt2* model);

/* Static string for a status code. */
const char* gpt2_strerror(int code);

/* Release the handle (not the caller's buffers).  Synchronises the stream first. */
void gpt2_free(gpt2* model);

/* Activation tensors inside `acts`, for inspection and tests. */
enum {
    GPT2_ACT_ENCODED = 0,  /* (B*T, C) token + position embedding */
    GPT2_ACT_LN1,          /* per layer (B*T, C) */
    GPT2_ACT_LN1_MEAN,     /* per layer (B*T) */
    GPT2_ACT_LN1_RSTD,     /* per layer (B*T) */
    GPT2_ACT_QKV,          /* per layer (B*T, 3C) */
    GPT2_ACT_ATTY,         /* per layer (B*T, C) attention output, heads concatenated */
    GPT2_ACT_ATT_LSE,      /* per layer (B, NH, T) log-sum-exp of each softmax row */
    GPT2_ACT_RESIDUAL2,    /* per layer (B*T, C) */
    GPT2_ACT_LN2,          /* per layer (B*T, C) */
    GPT2_ACT_LN2_MEAN,     /* per layer (B*T) */
    GPT2_ACT_LN2_RSTD,     /* per layer (B*T) */
    GPT2_ACT_FCH,          /* per layer (B*T, 4C) pre-GELU */
    GPT2_ACT_FCH_GELU,     /* per layer (B*T, 4C) */
    GPT2_ACT_RESIDUAL3,    /* per layer (B*T, C) */
    GPT2_ACT_LNF,          /* (B*T, C) */
    GPT2_ACT_LNF_MEAN,     /* (B*T) */
    GPT2_ACT_LNF_RSTD,     /* (B*T) */
    GPT2_ACT_LOGITS,       /* (B*T, V) with leading dimension ld >= V (rows 256-byte aligned) */
    GPT2_ACT_LOGITS_LSE,   /* (B*T) log-sum-exp of each logits row: softmax = exp(logit - lse) */
    GPT2_ACT_LOSSES,       /* (B*T) per-position cross-entropy */
    GPT2_NUM_ACTS
};

/* Where tensor `tensor` of layer `layer` (ignored for whole-model tensors) lives:
 * offset in floats from `acts`, rows, columns and leading dimension, at the batch shape
 * of the last forward (the built shape before any forward).  Host-only. */
int gpt2_activation_view(const gpt2* model, int tensor, int layer, size_t* offset, size_t* rows,
                         size_t* cols, size_t* ld);

/* Per-kernel timing (profiling aid; the pages only print whole-step times).
 * gpt2_profile_enable(model, 1) synchronises the stream and creates a pool of HIP
 * events (outside any step); from then on every kernel launch of the model records an
 * event pair around itself on the model's stream, with that launch's algorithmic work.
 * Enabling again clears the records; enable = 0 releases the pool.  gpt2_profile_collect
 * waits for the recorded events and returns the number of distinct kernels seen (< 0 on
 * error); gpt2_profile_entry(i) then gives kernel i's name (valid until the next
 * enable or free), launch count, summed duration in ms, and summed algorithmic flops
 * and bytes.  gpt2_profile_filter(model, name) limits recording to the kernel of that
 * name (NULL: all kernels), so that a timed run carries events around one kernel only. */
int gpt2_profile_enable(gpt2* model, int enable);
int gpt2_profile_filter(gpt2* model, const char* kernel_name);
int gpt2_profile_collect(gpt2* model);
int gpt2_profile_entry(gpt2* model, int i, const char** name, long* launches, double* total_ms,
                       double* flops, double* bytes);

/* Next-token sampling, the pages' sample_mult (huxiu page "llm.c：Andrej Karpathy带你从零
 * 复现LLM", 核心代码解读 item 5: draw an index from a probability distribution; the main
 * loop samples with it to generate text).  For each request i, row rows[i] (= b*T + t of
 * the last gpt2_forward, which may have had targets == NULL) gives the distribution
 * p = softmax(logits[row, 0..V)), and tokens[i] is the smallest index j with
 * coins[i] < p_0 + ... + p_j, or V-1 if rounding leaves the total at or below the coin.
 * The coins are the random numbers the caller draws, uniform in [0, 1): the library
 * holds no random state, so a run is reproducible from its coins.
 * Host arrays of n entries (the caller owns them); the call synchronises the model's
 * stream.  The probabilities are fp32 exp(z - lse) with fp64 running sums, so a coin
 * within ~1e-6 of a cumulative boundary may land on either neighbour.
 * Returns GPT2_OK; GPT2_EINVAL for a null model or array, n < 0, n > B*T of the last
 * forward, a row outside it or a coin outside [0, 1); GPT2_ESTATE without a forward. */
int gpt2_sample(gpt2* model, const int32_t* rows, const float* coins, int n, int32_t* tokens);

/* The pages' generation loop (新智元 article, 快速入门: the program ends by generating a
 * sample; the printed samples start from token 50256).  tokens is a host array of
 * total_len entries whose first prompt_len are given; for t = prompt_len .. total_len-1
 * it runs gpt2_forward over tokens[0..t) as one row (B = 1, no targets) and sets
 * tokens[t] = gpt2_sample of row t-1 with coins[t - prompt_len].  Each step recomputes
 * the whole prefix (no key/value cache), as the pages' loop does.  Needs
 * 1 <= prompt_len < total_len <= max_seq_len and total_len - 1 <= the build's B*T.
 * Afterwards the model holds the last step's forward (B = 1, no targets).
 * Returns GPT2_OK, GPT2_EINVAL (arguments, or a token outside [0, V)), or an error of
 * the underlying forward or sample. */
int gpt2_generate(gpt2* model, int32_t* tokens, int prompt_len, int total_len, const float* coins);

/* Stream schedule of gpt2_backward.  streams = 2 (the default): each layer's weight
 * gradients (dW += dY^T X and the bias sums, which need only that layer's output
 * gradient) run on a second stream the handle owns, overlapping the main chain of
 * dgrads, attention and LayerNorm; events order the two streams and gpt2_backward's work
 * is complete, in order, on the model's stream when everything enqueued after it runs.
 * streams = 1 runs everything on the model's stream.  Both schedules compute bitwise
 * the same results (every kernel's arithmetic is the same).  Returns GPT2_OK, or
 * GPT2_EINVAL for a null model or another value. */
int gpt2_set_backward_streams(gpt2* model, int streams);

/* Tile width of the forward and dgrad matmuls (process-wide; call it between steps, not
 * while another host thread launches work).  GPT2_GEMM_TILES_AUTO (the default) uses
 * 128 x 96 output tiles where their count is a whole number of rounds of the chip's 512
 * resident blocks and the 128 x 128 count is not (for 8192 rows: N = 768 and N = 2304),
 * and 128 x 128 tiles elsewhere; _128 and _96 force one width for every forward and
 * dgrad matmul.  Results agree between widths to rounding: each output sums its k terms
 * in the same order within a block, and split tiles add their k segments in k order.
 * Returns GPT2_OK, or GPT2_EINVAL for an unknown value (the setting is then unchanged). */
#define GPT2_GEMM_TILES_AUTO 0
#define GPT2_GEMM_TILES_128 1
#define GPT2_GEMM_TILES_96 2
int gpt2_set_gemm_tiles(int policy);

/* Standalone LayerNorm forward, overwrite semantics (the pages' worked layer: dakule
 * page 手动实现每个层前向 / 反向传播; 新智元 page 教程).  Device pointers: x, y (N,C);
 * w, b (C); mean, rstd (N).  y = (x - mean) * rstd * w + b with biased variance and
 * rstd = 1/sqrt(var + eps).  C must be a multiple of 4 and at most 4096. */
int gpt2_layernorm_forward(float* y, float* mean, float* rstd, const float* x, const float* w,
                           const float* b, int N, int C, float eps, void* stream);

/* Floats of device workspace gpt2_layernorm_backward needs for (N, C). */
size_t gpt2_layernorm_backward_workspace(int N, int C);

/* Standalone LayerNorm backward, overwrite semantics: writes dx (N,C), dw and db (C)
 * from dy, x, w, and the mean and rstd the forward kept.  `workspace` is a device
 * buffer of at least gpt2_layernorm_backward_workspace(N, C) floats (GPT2_EINVAL if
 * smaller); its contents on entry do not matter.  Deterministic. */
int gpt2_layernorm_backward(float* dx, float* dw, float* db, const float* dy, const float* x,
                            const float* w, const float* mean, const float* rstd, int N, int C,
                            float* workspace, size_t workspace_floats, void* stream);

/* Measurement probes, not part of the training step: the chip's ceilings at its running
 * clock, which the benchmark reports beside the datasheet peaks (the pages only print
 * whole-step times, so these are aids of the measurement, not of the method).
 * gpt2_probe_mfma: one launch of `blocks` (1..4096) blocks of 256 threads, each wave
 * running `iters` rounds of 16 independent matrix-core products held in registers, with
 * no memory traffic: kind 0 = fp32 16x16x4, kind 1 = bf16 16x16x32 (the shapes the
 * step's kernels use).  `out` is a device buffer of gpt2_probe_mfma_out_floats() floats
 * that receives one value per thread (so nothing is optimised away); *flops (host)
 * receives the flops the launch executes.
 * gpt2_probe_copy: dst[i] = src[i] for n floats (n a multiple of 4, 16-byte aligned
 * device buffers that do not overlap), float4 loads and stores, by a grid-stride loop
 * over `blocks` (1..65536) blocks of 256 threads.
 * Both enqueue on `stream` only; GPT2_EINVAL for bad arguments, GPT2_EDEVICE if the
 * launch fails. */
size_t gpt2_probe_mfma_out_floats(void);
int gpt2_probe_mfma(int kind, int iters, int blocks, float* out, double* flops, void* stream);
int gpt2_probe_copy(float* dst, const float* src, size_t n, int blocks, void* stream);

/* gpt2_layernorm_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and determinism as
 * gpt2_layernorm_backward (the same kernels run), but the partial rows go to a fixed
 * device array inside the library: at most gpt2_layernorm_backward_noalloc_max_floats()
 * floats (16 MiB), held on every device the library runs on until the process ends.  No
 * call allocates: the array's device address is looked up on a device's first call.
 * Every call on a device shares that device's array (nothing in it needs to start at
 * any value; a call leaves its partial rows there), so calls that overlap on one
 * device, on different streams or from different host threads, race and must not be
 * issued.  Returns GPT2_OK; GPT2_EINVAL for the argument errors of
 * gpt2_layernorm_backward; GPT2_ESCRATCH if (N, C) needs more than the fixed array;
 * GPT2_EDEVICE if the array's address cannot be found or a launch fails. */
size_t gpt2_layernorm_backward_noalloc_max_floats(void);
int gpt2_layernorm_backward_noalloc(float* dx, float* dw, float* db, const float* dy, const float* x,
                                    const float* w, const float* mean, const float* rstd, int N, int C,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_MI355X_H */
