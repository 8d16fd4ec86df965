/*
 * ncgpt.h -- C ABI of the MI355X (gfx950) forward / loss / backward of a
 * nanochat-style decoder-only GPT stack.
 *
 * What is computed (sources by page and section):
 *   x0 = wte[ids]                                   untied embedding ("nanochat 项目深度分析" §2.1 item 3)
 *        (embed_norm = 1: x0 = rmsnorm(wte[ids]), a block variant)
 *   per layer l:                                    pre-norm block (devpress.csdn.net guide §4.1)
 *     u   = rmsnorm(x)                              parameter-free RMSNorm (§2.1 item 5)
 *     q,k,v = u Wq^T, u Wk^T, u Wv^T                bias-free linears, n_head / n_kv_head (§2.1 items 5, 6)
 *     q,k = rmsnorm_D(rope_t(q)), rmsnorm_D(rope_t(k))   RoPE then QK-norm (§2.1 items 1, 2; §5.3)
 *     y   = causal_softmax(q k^T / sqrt(D)) v       query head h reads kv head h / (n_head/n_kv_head)
 *     x   = x + y Wo^T
 *     x   = x + relu(rmsnorm(x) Wfc^T)^2 Wproj^T    ReLU^2 MLP of width 4 n_embd (§2.1 item 4; woshipm.com §五.1)
 *   z = rmsnorm(x) Wlm^T                            untied lm_head
 *        (logit_softcap = c > 0: z = c tanh(z / c), the reading given to the logit stabilisation that
 *        woshipm.com §三 item 1 names without a formula)
 *   loss = mean over targets >= 0 of (logsumexp(z) - z[target])
 * The compute dtype mirrors the pages' COMPUTE_DTYPE scheme ("nanochat：低成本跑通大模型训练全流程",
 * precision paragraph): weights are fp32 masters, cast to the compute dtype for every linear, no autocast;
 * activations are stored in the compute dtype; products, norms, softmax and the loss accumulate in fp32;
 * gradients are returned in fp32.
 *
 * RoPE: pair (i, i + D/2) at position t (restarting at 0 for each sequence) is rotated by the angle
 * t * rope_base^(-2i/D) with y_i = x_i cos + x_{i+D/2} sin, y_{i+D/2} = -x_i sin + x_{i+D/2} cos.
 * RMSNorm: y = x / sqrt(mean(x^2) + norm_eps).
 *
 * Memory: every pointer argument is a device pointer unless stated otherwise.  The caller owns all device
 * memory (parameters, gradients, token ids, targets, the loss scalar and the workspace); the library owns
 * only the host-side context.  Every call is asynchronous on the HIP stream given to ncgpt_bind; the
 * library never synchronises except in ncgpt_check, ncgpt_probe and the timing readout.
 *
 * Errors: functions return ncgpt_status.  Argument and shape errors are detected on the host and returned
 * synchronously; ncgpt_last_error(ctx) then holds a message.  Device-side conditions (a token id outside
 * [0, vocab), a target >= vocab, no valid target) set a flag in the workspace that ncgpt_check reports as
 * NCGPT_EDEVICE.  Nothing aborts or throws across the ABI.  A context is not thread-safe; distinct
 * contexts are independent.
 */
#ifndef NCGPT_H
#define NCGPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NCGPT_OK = 0,
    NCGPT_EINVAL = -1,       /* null pointer, bad enum, inconsistent sizes */
    NCGPT_EUNSUPPORTED = -2, /* shape outside what the kernels handle (see ncgpt_create) */
    NCGPT_ENOMEM = -3,       /* host allocation failed, or workspace too small */
    NCGPT_EHIP = -4,         /* a HIP runtime call or kernel launch failed */
    NCGPT_ESTATE = -5,       /* calls out of order (loss before forward, backward before loss, unbound ctx) */
    NCGPT_EDEVICE = -6       /* device-side error flag set (reported by ncgpt_check) */
} ncgpt_status;

/* Compute dtype: mirrors COMPUTE_DTYPE (fp32, or bf16 with fp32 master weights; "nanochat：低成本跑通大模型训练全流程",
 * precision paragraph).  NCGPT_F16 is the float16 setting for GPUs without bf16 ([poetries] tuning tips; the
 * devpress.csdn.net guide's precision notes): the same scheme in fp16, whose small range makes gradients underflow
 * unless the loss is scaled -- pass the scale as ncgpt_backward's grad_scale (the returned fp32 gradients carry
 * it), check them with ncgpt_grads_finite and divide before the optimizer step. */
typedef enum { NCGPT_F32 = 0, NCGPT_BF16 = 1, NCGPT_F16 = 2 } ncgpt_dtype;

typedef struct {
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, mlp_dim, vocab_size, batch, seq_len;
    float rope_base;     /* 10000 */
    float norm_eps;      /* 2^-23, the epsilon F.rms_norm uses when none is given */
    float logit_softcap; /* 0 (off), or c > 0: the logits become c tanh(z / c) before the loss and in decode */
    int32_t embed_norm;  /* 0 (off), or 1: an RMSNorm right after the embedding */
} ncgpt_config;

typedef struct ncgpt_ctx ncgpt_ctx;

/* Packed fp32 parameter count P.  Packing order: wte [V,C]; then for each layer Wq [H*D,C], Wk [Hkv*D,C],
 * Wv [Hkv*D,C] (contiguous, together the [(H+2Hkv)D, C] qkv weight), Wo [C,H*D], Wfc [F,C], Wproj [C,F];
 * then lm_head [V,C].  Every matrix is [out, in] row-major.  Gradients use the same packing.
 * Returns 0 for a null or invalid config. */
size_t ncgpt_num_params(const ncgpt_config* cfg);

/* Offset (in elements) and shape of one packed tensor.  layer = -1 selects which = 0 (wte) or 1 (lm_head);
 * layer in [0, n_layer) selects which = 0..5 (Wq, Wk, Wv, Wo, Wfc, Wproj).  EINVAL on a bad selector. */
ncgpt_status ncgpt_param_slice(const ncgpt_config* cfg, int layer, int which, size_t* offset, int64_t* rows,
                               int64_t* cols);

/* Create a context (host memory only; no device work).  EUNSUPPORTED unless head_dim is 64 or 128
 * (128 for NCGPT_BF16 and NCGPT_F16), n_head % n_kv_head == 0, n_embd, mlp_dim and vocab_size are multiples
 * of 64, vocab_size <= 65536, seq_len is a multiple of 128 for the 16-bit dtypes (of 64 for NCGPT_F32), and
 * batch*seq_len*vocab fits the workspace plan.  EINVAL for a null pointer or non-positive size, a negative
 * norm_eps, rope_base <= 0, a negative or non-finite logit_softcap, or embed_norm other than 0 or 1.
 * *out receives the context; free it with ncgpt_destroy. */
ncgpt_status ncgpt_create(const ncgpt_config* cfg, ncgpt_dtype dtype, ncgpt_ctx** out);

/* Bytes of device workspace the context needs (saved activations, cast weights, logits, scratch). */
ncgpt_status ncgpt_workspace_size(const ncgpt_ctx* ctx, size_t* bytes);

/* Attach a caller-owned device workspace of at least ncgpt_workspace_size bytes (256-byte aligned) and the
 * HIP stream (hipStream_t, may be NULL for the null stream) every later call enqueues on.  Uploads the RoPE
 * tables and clears the device error flag (asynchronously on that stream).  May be called again to rebind. */
ncgpt_status ncgpt_bind(ncgpt_ctx* ctx, void* workspace, size_t bytes, void* hip_stream);

/* Variant of ncgpt_bind for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the workspace is a file-scope device array
 * inside the library, 64 MiB (NCGPT_STATIC_SCRATCH_BYTES) on each GPU it runs on, held until the process
 * ends.  Binds ctx to that array on the device current at the call (the stream must belong to it) and
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.  The caller still passes
 * ids, params, targets, loss and grads to the other calls.  Returns NCGPT_ENOMEM, with a message naming
 * both sizes, when ncgpt_workspace_size exceeds the array; nothing is bound then.
 * One array per GPU is shared by every context bound to it and keeps the last call's contents (the
 * error flag is cleared here).  Binding a second context to it takes the array over: the first context's
 * later calls return NCGPT_ESTATE until it is bound again.  Calls of contexts bound to the same GPU's
 * array that overlap in time (other threads or streams) race on its contents. */
#define NCGPT_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
ncgpt_status ncgpt_bind_static(ncgpt_ctx* ctx, void* hip_stream);

/* Forward pass of the block stack up to the final RMSNorm (the LM head runs in ncgpt_loss, where the
 * targets are known).  ids: int32 [batch*seq_len] (row b*seq_len + t).  params: fp32 [P] packed as above.
 * Both must stay valid and unmodified until ncgpt_backward has been enqueued: the context remembers them. */
ncgpt_status ncgpt_forward(ncgpt_ctx* ctx, const int32_t* ids, const float* params);

/* LM head and cross-entropy of the last forward ("nanochat 项目深度分析" §2.1 item 3, §2.3; woshipm.com §三
 * item 1).  targets: int32 [batch*seq_len]; a negative target is ignored.  loss: fp32 [1], receives the mean
 * over valid targets of logsumexp(z) - z[target] (NaN if none, with the device flag set; a target >= vocab
 * also sets the flag).  In NCGPT_BF16 the LM-head GEMM's epilogue forms each row's softmax statistics and
 * target logit from its accumulators, so no pass over the [N, vocab] logits is needed for the loss; the
 * logits are kept for the backward only in NCGPT_LOGITS_STORED mode.  targets must stay valid until
 * ncgpt_backward has been enqueued.  ESTATE before ncgpt_forward. */
ncgpt_status ncgpt_loss(ncgpt_ctx* ctx, const int32_t* targets, float* loss);

/* Where the backward's dz = softmax(z) - onehot(target) comes from (NCGPT_BF16 only; takes effect at the
 * next ncgpt_loss):
 *   NCGPT_LOGITS_STORED      ncgpt_loss stores the bf16 logits; ncgpt_backward turns them into dz in place
 *                            (one read + one write of [N, vocab]).  The default.
 *   NCGPT_LOGITS_RECOMPUTED  ncgpt_loss stores no logits; ncgpt_backward recomputes them with the LM-head
 *                            GEMM, whose epilogue writes dz directly (one more GEMM, no logit read).
 * Both give bitwise identical results.  EINVAL for another value, EUNSUPPORTED for RECOMPUTED in NCGPT_F32. */
typedef enum { NCGPT_LOGITS_STORED = 0, NCGPT_LOGITS_RECOMPUTED = 1 } ncgpt_lm_head_mode;
ncgpt_status ncgpt_set_lm_head_mode(ncgpt_ctx* ctx, int mode);

/* Backward of the last loss.  grads: fp32 [P] receives grad_scale * d loss / d params (accumulate = 0) or
 * has it added (accumulate = 1).  For k micro-batches of gradient accumulation pass grad_scale = 1/k and
 * accumulate = 1 after the first ("nanochat 项目深度分析" §4.3).  The stored logits (if any) are consumed.
 * ESTATE unless ncgpt_loss followed the last ncgpt_forward. */
ncgpt_status ncgpt_backward(ncgpt_ctx* ctx, float* grads, int accumulate, float grad_scale);

/* FP8 forward linears (NCGPT_BF16 only; off by default).  With on = 1 the five forward products -- qkv,
 * attention output, MLP up and down, and the LM head (also its recomputation in NCGPT_LOGITS_RECOMPUTED) --
 * take OCP E4M3 operands ("supports FP8" on woshipm §一 and §六 and on the devpress.csdn.net guide, which give no
 * recipe): every weight row and every activation row (token) is scaled by its own amax / 448 and rounded to
 * nearest even, the products accumulate in fp32 and are multiplied back by both row scales before the
 * epilogue.  Weights are quantised from the fp32 parameters in every ncgpt_forward; the backward and the
 * decode step stay bf16.  EUNSUPPORTED for NCGPT_F32 or when n_embd, n_head * head_dim or mlp_dim is not a
 * multiple of 128; EINVAL for on outside {0, 1}.  The next call on the context must be ncgpt_forward. */
ncgpt_status ncgpt_set_fp8(ncgpt_ctx* ctx, int on);

/* The optimizer step that follows the backward ("nanochat 项目深度分析" §2.2 and §4.2): Muon for every layer
 * matrix (Wq, Wk, Wv, Wo, Wfc, Wproj), AdamW for wte and lm_head, each group at its own learning rate.
 * Muon is taken in the form of the published Muon description (the pages leave the iteration out):
 *   buf = mu buf + (1 - mu) g;  u = (1 - mu) g + mu buf (muon_nesterov) or buf;
 *   X = u / max(||u||_F, ns_eps) in bf16, then ns_steps times: A = X X^T (X^T X when rows > cols),
 *   B = ns_b A + ns_c A A, X = ns_a X + B X (X B when rows > cols), all bf16 MFMA products;
 *   p = p (1 - matrix_lr weight_decay) - matrix_lr sqrt(max(1, rows / cols)) X.
 * AdamW (decoupled weight decay, bias-corrected, fp32): m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
 *   p = p (1 - lr weight_decay) - lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + adam_eps).
 * Typical values: matrix_lr 0.02, embedding_lr 0.2, unembedding_lr 0.004 (the pages); muon_momentum 0.95,
 * ns_steps 5, (ns_a, ns_b, ns_c) = (3.4445, -4.7750, 2.0315), ns_eps 1e-7 (the Muon description). */
typedef struct {
    float matrix_lr, embedding_lr, unembedding_lr;
    float muon_momentum;
    int32_t muon_nesterov, ns_steps;
    float ns_a, ns_b, ns_c, ns_eps;
    float adam_beta1, adam_beta2, adam_eps;
    float weight_decay;
} ncgpt_optim_config;

/* fp32 elements of the optimizer state: a momentum buffer per layer matrix (the packed matrix range, in
 * packing order), then AdamW's m and v for wte, then m and v for lm_head.  The caller zeroes it before the
 * first step.  0 for an invalid config. */
size_t ncgpt_optim_state_size(const ncgpt_config* cfg);

/* One optimizer step, in place on params (fp32 [P]) and state (fp32 [ncgpt_optim_state_size]), from grads
 * (fp32 [P], e.g. those of ncgpt_backward).  step counts from 1 (AdamW's bias correction).  Runs on the bound
 * stream; its Newton-Schulz scratch overlays the workspace's saved activations, so the next call on the
 * context must be ncgpt_forward (probes of the last forward are lost).  ESTATE between ncgpt_forward and
 * ncgpt_backward; EINVAL for null pointers, step < 1, ns_steps outside [0, 20] or a momentum / beta outside
 * [0, 1). */
ncgpt_status ncgpt_optim_step(ncgpt_ctx* ctx, float* params, const float* grads, float* state, int64_t step,
                              const ncgpt_optim_config* oc);

/* KV-cache decode ("nanochat 项目深度分析", engine section: a preallocated cache (layers, 2, B, H, T, D) with
 * a position pointer).  The cache is caller-owned device memory in the compute dtype, laid out
 * [n_layer][2 (k, v)][batch][n_kv_head][seq_len][head_dim]; k is stored after RoPE and QK-norm, as attention
 * reads it.  seq_len is the cache capacity. */
size_t ncgpt_kv_cache_bytes(const ncgpt_ctx* ctx);

/* Prefill: copy k and v of positions [0, n) of every sequence from the last ncgpt_forward into the cache
 * (a prompt of n tokens run through ncgpt_forward; the forward's positions >= n do not affect positions < n).
 * ESTATE before ncgpt_forward or after ncgpt_optim_step; EINVAL for n outside [0, seq_len]. */
ncgpt_status ncgpt_kv_fill(ncgpt_ctx* ctx, void* kv_cache, int32_t n);

/* One decode step: ids int32 [batch] are the tokens at position pos (0 <= pos < seq_len) of each sequence;
 * positions < pos must already be in the cache (ncgpt_kv_fill or earlier steps).  Runs the block stack on
 * these batch tokens, stores their k and v at pos, and writes the next-token logits, fp32 [batch, vocab],
 * to logits.  It equals the causal forward of the sequences at their last position.  recast = 1 casts params
 * to the bf16 weight copy first (NCGPT_BF16); 0 reuses the copy of the last ncgpt_forward or recasting step
 * (ESTATE if there is none; params changed since make it stale).  Uses its own scratch: a pending
 * ncgpt_loss / ncgpt_backward of the last forward is not disturbed. */
ncgpt_status ncgpt_decode_step(ncgpt_ctx* ctx, const int32_t* ids, const float* params, void* kv_cache, int32_t pos,
                               float* logits, int recast);

/* Synchronise the bound stream and report device-side errors: EDEVICE if the flag is set (the flag is then
 * cleared), EHIP on an asynchronous HIP error, OK otherwise. */
ncgpt_status ncgpt_check(ncgpt_ctx* ctx);

/* Loss-scaling check (the GradScaler step of the fp16 setting): *ok (device int32) = 1 when all n values of x
 * (device fp32, e.g. the gradients of a scaled backward) are finite, else 0.  Enqueued on the bound stream; no
 * synchronisation.  EINVAL for null pointers. */
ncgpt_status ncgpt_grads_finite(ncgpt_ctx* ctx, const float* x, size_t n, int32_t* ok);

/* Saved-activation readout (for tests).  Copies one activation of the last forward, converted to fp32,
 * into dst (device, fp32, ncgpt_probe_numel elements) and synchronises the stream.  what:
 *   0 x0 [N,C] the first block's input   1 xn1 [N,C] pre-attention norm (layer)
 *   2 qkv [N,(H+2Hkv)D] after RoPE/QK-norm (layer)   3 y [N,H*D] attention output (layer)
 *   4 lse_att [B,H,T] attention log-sum-exp (layer)  5 xn2 [N,C] pre-MLP norm (layer)
 *   6 act [N,F] relu(xn2 Wfc^T)^2 (layer)  7 xf [N,C] final norm    8 lse [N] logits log-sum-exp
 *   9 loss_rows [N] per-token loss (0 when ignored)
 *  10 demb [N,C] gradient w.r.t. the embedding rows wte[ids] (after backward; x0's gradient taken back
 *     through the embedding norm when embed_norm = 1)
 * EINVAL for an unknown what or layer, ESTATE before the forward that produces it. */
ncgpt_status ncgpt_probe_numel(const ncgpt_ctx* ctx, int what, size_t* numel);
ncgpt_status ncgpt_probe(ncgpt_ctx* ctx, int what, int layer, float* dst);

/* Per-kernel timing.  When enabled, every launch is bracketed by HIP events on the bound stream; the
 * readout synchronises and aggregates by kernel name since the last reset: launch count, total ms, and
 * the algorithmic FLOPs and HBM bytes of those launches (FLOPs = 2*M*N*K for a GEMM, causal pairs only for
 * attention; bytes = compulsory reads + writes of the bandwidth-bound kernels). */
ncgpt_status ncgpt_timing_enable(ncgpt_ctx* ctx, int enable);
ncgpt_status ncgpt_timing_reset(ncgpt_ctx* ctx);
/* Number of distinct kernel names recorded (synchronises and folds pending events). */
ncgpt_status ncgpt_timing_count(ncgpt_ctx* ctx, int* count);
ncgpt_status ncgpt_timing_get(ncgpt_ctx* ctx, int index, char* name, size_t name_len, int64_t* launches,
                              double* total_ms, double* flops, double* bytes);

/* Message of the last error on this context ("" if none).  Owned by the context. */
const char* ncgpt_last_error(const ncgpt_ctx* ctx);

/* Free the context (host memory only; the caller frees the workspace).  NULL is ignored. */
void ncgpt_destroy(ncgpt_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* NCGPT_H */
