/*
 * gpt2.h -- C ABI of the GPT-2 training-step library for MI355X (gfx950).
 *
 * One GPT-2 training step (the method the llm.c pages describe) on one GPU:
 * token + position embedding, L pre-LayerNorm transformer blocks (LayerNorm,
 * QKV / attention-projection / MLP linears, causal multi-head attention,
 * GELU, residual adds), a tied classifier with a fused softmax
 * cross-entropy, a hand-derived backward pass and an AdamW update, all over
 * ONE device buffer whose layout is planned up front.
 *
 * Sources (the pages): "llm.c: GPT-2 training in plain C, with every
 * gradient written by hand" (fernfant learning-robotics lesson), section 2
 * "How the code works" (gpt2_forward, gpt2_backward, gpt2_update over a
 * GPT2 struct with a single allocation; the per-layer call sequence) and
 * section 3 "Run it, tested" (the GPT-2 124M config); the pyshine.com tour
 * of llm.c (fused classifier, AdamW and global-norm headers, mixed
 * precision); "llm.c's Origin and the Future of LLM Compilers", sections
 * "Pure C" and "Avengers" (one up-front allocation, fp32 vs bf16 per tensor,
 * kernel fusion).
 *
 * Conventions
 *  - Every call returns 0 on success or a negative errno-style code
 *    (GPT2_E*), and then gpt2_last_error() holds a message for the calling
 *    thread.  No C++ exception crosses the ABI.
 *  - Device memory is owned by the caller: gpt2_build() carves the buffer
 *    it is given (size from gpt2_plan()) and never allocates device memory
 *    itself.  The library owns only the small host handle (gpt2_destroy).
 *  - All GPU work is queued on the HIP stream given to gpt2_build(), in
 *    call order.  A call blocks the host only when it returns a value read
 *    from the device (a loss, a norm, a copy to host memory).
 *  - Host arrays passed in may be freed or reused as soon as a call returns.
 *  - Layouts: parameters are one flat fp32 array of N floats holding, in
 *    this order, wte (Vp,C), wpe (maxT,C), ln1w (L,C), ln1b (L,C),
 *    qkvw (L,3C,C), qkvb (L,3C), attprojw (L,C,C), attprojb (L,C),
 *    ln2w (L,C), ln2b (L,C), fcw (L,4C,C), fcb (L,4C), fcprojw (L,C,4C),
 *    fcprojb (L,C), lnfw (C), lnfb (C); matrices are (out,in) row-major;
 *    the classifier reuses wte.  N = Vp*C + maxT*C + L*(12C^2+13C) + 2C.
 *    Token arrays are int32 [B,T] row-major.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* error codes */
#define GPT2_OK 0
#define GPT2_EINVAL (-22)  /* bad argument or configuration */
#define GPT2_ENOMEM (-12)  /* device buffer smaller than gpt2_plan() asked for */
#define GPT2_EPERM (-1)    /* call out of order (e.g. backward before a forward with targets) */
#define GPT2_ERANGE (-34)  /* non-finite gradient norm; the AdamW update is refused */
#define GPT2_EIO (-5)      /* a HIP runtime call failed */

/* arithmetic modes */
#define GPT2_FP32 0        /* fp32 everywhere (params, activations, matmuls) */
#define GPT2_BF16_MIXED 1  /* bf16 activations and MFMA matmuls with fp32 accumulation;
                              fp32 master params, grads, AdamW m/v, LN statistics, losses */
#define GPT2_BF16_SR 2     /* as BF16_MIXED, but the bf16 weights ARE the parameters (no fp32
                              master): AdamW rounds each updated value to bf16 stochastically
                              ("llm.c's Origin and the Future of LLM Compilers", section
                              "Avengers": stochastic rounding).  Grads, m, v stay fp32. */

typedef struct {
    int32_t num_layers;        /* L */
    int32_t channels;          /* C; multiple of num_heads */
    int32_t num_heads;         /* NH; head size hs = C/NH (64 required in the bf16 modes) */
    int32_t max_seq_len;       /* maxT: rows of wpe */
    int32_t vocab_size;        /* V: real vocabulary, softmax runs over v < V */
    int32_t padded_vocab_size; /* Vp >= V: rows of wte and columns of the logits */
    int32_t batch_size;        /* B */
    int32_t seq_len;           /* T <= maxT */
    int32_t precision;         /* GPT2_FP32, GPT2_BF16_MIXED or GPT2_BF16_SR */
    int32_t fused_classifier;  /* 0: the logits are stored, then the softmax cross-entropy pass turns
                                  them into dlogits in place (B*T*Vp activations).  1 (bf16 modes
                                  only): the classifier product computes each row's softmax
                                  statistics in its epilogue and the logits are never stored; the
                                  backward recomputes them in chunks of at most 4096 rows, turning
                                  each tile into dlogits as it leaves the product (the pyshine.com
                                  tour's fused classifier; "llm.c's Origin and the Future of LLM
                                  Compilers", "Avengers": recompute during the backward).  Uses
                                  less memory, adds one classifier product. */
    int32_t recompute_gelu;    /* 0: the forward keeps every layer's GELU output (the fcproj input
                                  its weight gradient reads) beside GELU'.  1 (bf16 modes only):
                                  it keeps only the pre-activation, rounded to bf16, and one layer's
                                  GELU output for the next product; the backward recomputes each
                                  layer's GELU output from the kept pre-activation (the same values
                                  the forward used) for that layer's fcproj weight gradient, and
                                  GELU' in the fcproj backward-data product ("llm.c's Origin and
                                  the Future of LLM Compilers", "Avengers": recompute settings).
                                  Saves (L-1)*B*T*4C*2 bytes, costs one GELU pass per layer. */
    int32_t recompute_layernorm; /* 0: the forward keeps every layer's two LayerNorm outputs (the
                                  qkv and fc inputs their weight gradients read).  1 (bf16 modes
                                  only): it keeps one layer's of each; the backward runs each
                                  layer's LayerNorm forwards again (the same kernel on the same
                                  inputs: the same values) before that layer's qkv and fc weight
                                  gradients, which then run in the block loop.  Saves
                                  2*(L-1)*B*T*C*2 bytes (same recompute settings as above). */
} gpt2_config;

typedef struct gpt2_model gpt2_t;

/* Size in bytes of the single device buffer for cfg: parameters, gradients,
 * AdamW m and v, the bf16 weights (BF16_MIXED, BF16_SR), every activation the
 * backward needs, activation gradients and small scratch, each region
 * 256-byte aligned.  Pure host function.  GPT2_EINVAL on a bad config:
 * C % NH != 0, T > maxT, V > Vp, a non-positive size, an unknown precision,
 * or in the bf16 modes: hs != 64, or C, Vp or T not a multiple of 64. */
int gpt2_plan(const gpt2_config* cfg, size_t* device_bytes);

/* Carve device_buf (device memory of at least gpt2_plan() bytes, 256-byte
 * aligned, owned by the caller and kept alive until gpt2_destroy) and
 * initialise the parameters from seed: wte rows [0,V), wpe, qkvw and fcw
 * ~ N(0, 0.02); attprojw and fcprojw ~ N(0, 0.02/sqrt(2L)); biases 0, LN
 * gains 1, padded wte rows 0 (the GPT-2 init the workloads fix).  Normals
 * come from SplitMix64 draws 2g+1 and 2g+2 for flat parameter index g and
 * the Box-Muller cosine branch in double, rounded once to fp32.  Gradients
 * and AdamW state start at zero.  hip_stream is a hipStream_t (NULL = the
 * default stream).  On success *out holds the handle. */
int gpt2_build(const gpt2_config* cfg, uint64_t seed, void* device_buf, size_t bytes,
               void* hip_stream, gpt2_t** out);

/* Forward pass on host int32 arrays tokens[B*T] and targets[B*T] (ids in
 * [0,V), checked on the host: GPT2_EINVAL otherwise).  With targets, the
 * fused softmax cross-entropy also writes d(loss)/d(logits) in place of the
 * logits for gpt2_backward, and *mean_loss receives the mean over the B*T
 * positions of -log softmax(logits)[target] (one stream sync).  With
 * targets == NULL the logits are kept (no backward possible) and
 * *mean_loss, if given, is NaN.  mean_loss may be NULL: then nothing is
 * read back and the call does not block. */
int gpt2_forward(gpt2_t* m, const int32_t* tokens, const int32_t* targets, float* mean_loss);

/* As gpt2_forward, but tokens and targets are device int32 arrays already
 * resident on the GPU (targets may be NULL).  They are read in stream order
 * by the forward's first kernel, which copies them into the model (the
 * caller keeps them unchanged until the stream has reached that point, as for
 * an asynchronous copy; the model keeps no reference after it).  Ids are
 * checked on the device: an id outside [0,V) is replaced by 0 in the model's
 * copy and flagged, and the next call that reads a value back (mean_loss
 * here, or gpt2_read_loss) reports GPT2_EINVAL. */
int gpt2_forward_device(gpt2_t* m, const int32_t* d_tokens, const int32_t* d_targets,
                        float* mean_loss);

/* Mean loss of the last forward with targets (blocks on the stream).  Like
 * every call that reads a value back, it also reports a device-side
 * condition raised since the last report (see gpt2_sync): the loss is still
 * written when the report is GPT2_ERANGE. */
int gpt2_read_loss(gpt2_t* m, float* mean_loss);

/* Block until all queued work is done and report, then clear, the
 * conditions the kernels raise on the device (they cannot return an error
 * themselves): GPT2_EINVAL if a device token or target id was outside
 * [0,V) (gpt2_forward_device), else GPT2_ERANGE if an AdamW update was
 * refused because the gradient norm was not finite (gpt2_adamw_step after
 * gpt2_clip_grad_norm with norm == NULL); 0 otherwise.  The global-norm
 * clipping and its outlier guard follow the pyshine.com tour of llm.c
 * (global-norm header). */
int gpt2_sync(gpt2_t* m);

/* Parameter gradients <- 0.  (Activation gradients are overwritten by every
 * backward, never accumulated.)  In the bf16 modes the clear is deferred:
 * the next gpt2_backward stores into every gradient element instead of
 * adding, and a gradient reader that comes first (clip, AdamW, copy,
 * gpt2_device_grads) queues the clear before it reads.  Either way every
 * later observer sees zeros plus what backward added. */
int gpt2_zero_grad(gpt2_t* m);

/* Backward pass of the last forward-with-targets: the forward's layers in
 * reverse, ACCUMULATING (+=) into the parameter gradients.  GPT2_EPERM if
 * there was no forward with targets since the last build/update. */
int gpt2_backward(gpt2_t* m);

/* Global-norm gradient clipping: n = ||g||_2 over all N gradients, computed
 * on the device; with max_norm > 0 and n > max_norm the next
 * gpt2_adamw_step uses g * max_norm/n (the gradients in memory are not
 * rewritten).  max_norm <= 0 only measures.  If norm != NULL, *norm = n
 * (one stream sync); a non-finite n returns GPT2_ERANGE and makes the next
 * gpt2_adamw_step refuse to update.  With norm == NULL nothing is read back:
 * a non-finite n is caught on the device instead, where the next AdamW
 * kernel leaves every parameter, m and v (and the bf16 copy) unchanged and
 * raises the condition gpt2_sync and the next read-back report. */
int gpt2_clip_grad_norm(gpt2_t* m, float max_norm, float* norm);

/* AdamW (decoupled weight decay, bias-corrected, step t >= 1) over all N
 * parameters, then the bf16 weight shadow is refreshed (BF16_MIXED):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   theta -= lr * ( m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd * theta ).
 * BF16_SR: theta is the bf16 parameter; the fp32 result x of the update is
 * rounded to bf16 stochastically: with u the top 16 bits of the SplitMix64
 * output function (Steele, Lea & Flood 2014) at state k + (i+1)*gamma, where
 * i is the flat parameter index, gamma = 0x9E3779B97F4A7C15 and k the same
 * function at state seed + (2^62 + t)*gamma (seed: the build seed), the bf16
 * result is the top half of bits(x) + u, i.e. x moves away from zero to the
 * next bf16 value with probability (low 16 bits of x) / 65536 (unbiased).
 * The fp32 region then holds float(bf16) of the LayerNorm and bias tensors
 * (the kernels read those in fp32); there is no fp32 copy of the others
 * (gpt2_plan leaves it out: 4 bytes less per matrix parameter).
 * GPT2_EINVAL if t < 1. */
int gpt2_adamw_step(gpt2_t* m, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int t);

/* Free the handle (not the device buffer). NULL is accepted. */
int gpt2_destroy(gpt2_t* m);

/* Message of the last failed call on this thread ("" if none). */
const char* gpt2_last_error(void);

/* ---- inspection and test access (block on the stream) ---------------- */

/* Number of parameters N. */
size_t gpt2_num_params(const gpt2_t* m);

/* Offsets (in floats) of the 16 parameter tensors in the flat layout. */
int gpt2_param_offsets(const gpt2_t* m, size_t offsets[16]);

/* Copy fp32 master parameters / gradients / AdamW m and v to host arrays of
 * N floats; m_dst or v_dst may be NULL.  In BF16_SR mode the parameters are
 * the bf16 values widened (exact). */
int gpt2_copy_params(gpt2_t* m, float* host_dst);
int gpt2_copy_grads(gpt2_t* m, float* host_dst);
int gpt2_copy_opt_state(gpt2_t* m, float* m_dst, float* v_dst);

/* Copy the last forward's logits [B*T, Vp] to host as fp32.  Only valid
 * after a forward with targets == NULL (a forward with targets overwrites
 * them with dlogits); GPT2_EPERM otherwise, and always with the fused
 * classifier (which keeps no logits; its forward without targets stops
 * after the final LayerNorm). */
int gpt2_copy_logits(gpt2_t* m, float* host_dst);

/* Copy the per-position losses [B*T] of the last forward with targets. */
int gpt2_copy_losses(gpt2_t* m, float* host_dst);

/* Overwrite the parameter gradients from a host array of N floats (a
 * pending deferred clear is dropped).  For tests of the update and of the
 * non-finite guard. */
int gpt2_set_grads(gpt2_t* m, const float* host_src);

/* Overwrite the fp32 master parameters from a host array of N floats and
 * refresh the bf16 shadow.  In BF16_SR mode the bf16 parameters are set to
 * the values rounded to nearest-even, and the fp32 copies to those. */
int gpt2_set_params(gpt2_t* m, const float* host_src);

/* Device pointer of the planned buffer region holding the fp32 master
 * parameters, gradients and the bf16 weight shadow (NULL in FP32 mode).
 * In BF16_SR mode the shadow holds the parameters and the fp32 region holds
 * only the LayerNorm and bias tensors (ln1w, ln1b, qkvb, attprojb, ln2w,
 * ln2b, fcb, fcprojb, lnfw, lnfb), packed in that order.
 * gpt2_device_grads first queues a deferred gpt2_zero_grad clear, if one is
 * pending, on the model's stream. */
void* gpt2_device_params(gpt2_t* m);
void* gpt2_device_grads(gpt2_t* m);
void* gpt2_device_shadow(gpt2_t* m);

/* ---- single-kernel entry points, for kernel tests and timing ---------- */

/* Kernel timing: when enabled, HIP events bracket every launch of the
 * named kernel class on the library's stream; gpt2_kernel_timing_read()
 * blocks on the stream and returns the launch count and summed milliseconds
 * since the last enable.  Class names: "gemm_classifier_fwd",
 * "gemm_classifier_dw", "gemm_classifier_dx", "gemm_fwd", "gemm_dx",
 * "gemm_dw", "attention_fwd", "attention_bwd", "softmax_ce", "adamw",
 * "layernorm_fwd", "layernorm_bwd". */
int gpt2_kernel_timing_enable(gpt2_t* m, const char* kernel_class, int enable);
int gpt2_kernel_timing_read(gpt2_t* m, int* launches, double* total_ms);

/* out[M,N] (dtype of precision) = A[M,K] * W[N,K]^T (+ bias[N] fp32), all
 * row-major device arrays in the model's activation dtype (fp32 or bf16);
 * the same kernel the forward linears use.  Runs on the model's stream. */
int gpt2_test_gemm_nt(gpt2_t* m, void* out, const void* a, const void* w, const float* bias,
                      int M, int N, int K);
/* dX[M,K] = dY[M,N] * W[N,K]   (the backward-data kernel) */
int gpt2_test_gemm_nn(gpt2_t* m, void* dx, const void* dy, const void* w, int M, int N, int K);
/* dW[N,K] (fp32) += dY[M,N]^T * X[M,K]   (the backward-weight kernel) */
int gpt2_test_gemm_tn(gpt2_t* m, float* dw, const void* dy, const void* x, int M, int N, int K);

/* Causal attention kernels on device arrays in the model's activation
 * dtype: qkv [B,T,3C] (q|k|v, head h owns channels [h*hs,(h+1)*hs) of
 * each), out [B,T,C], lse [B,NH,T] fp32 (natural-log sum of exp of the
 * scaled scores of each query row), dout [B,T,C], dqkv [B,T,3C].
 * B*NH*T may not exceed the model's batch_size*num_heads*seq_len (the
 * backward keeps its row sums D = rowsum(dout o out) in the model's buffer).
 * The same kernels the training step runs. */
int gpt2_test_attention_fwd(gpt2_t* m, void* out, float* lse, const void* qkv, int B, int T, int C, int NH);
int gpt2_test_attention_bwd(gpt2_t* m, void* dqkv, const void* dout, const void* qkv, const void* out,
                            const float* lse, int B, int T, int C, int NH);

/* ---- allocation-free variant ------------------------------------------ */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the causal
 * attention backward of gpt2_test_attention_bwd (bf16 flash kernels, head
 * size 64, T a multiple of 64; same arguments and layouts) without a model.
 * Its per-row scratch (2*B*NH*T floats) is a static device array of the
 * library, 8 MiB per GPU, held until the process ends: B*NH*T may not exceed
 * 1048576 (GPT2_EINVAL otherwise).  Runs on hip_stream (a hipStream_t of the
 * current device; NULL = the default stream) and allocates nothing.  Every
 * call on one GPU shares that array, so calls that overlap on one GPU (other
 * streams, other threads) race; calls in one stream are ordered. */
int gpt2_attention_bwd_noalloc(void* hip_stream, void* dqkv, const void* dout, const void* qkv, const void* out,
                               const float* lse, int B, int T, int C, int NH);

#ifdef __cplusplus
}
#endif
#endif
