/*
 * ncgpt.h -- C ABI of the MI355X (gfx950) forward / loss / backward of a
 * nanochat-style decoder-only GPT stack.
 *
 * What is computed (sources by page and section):
 *   x0 = wte[ids]                                   untied embedding ("nanochat 项目深度分析" §2.1 item 3)
 *   per layer l:                                    pre-norm block (devpress.csdn.net guide §4.1)
 *     u   = rmsnorm(x)                              parameter-free RMSNorm (§2.1 item 5)
 *     q,k,v = u Wq^T, u Wk^T, u Wv^T                bias-free linears, n_head / n_kv_head (§2.1 items 5, 6)
 *     q,k = rmsnorm_D(rope_t(q)), rmsnorm_D(rope_t(k))   RoPE then QK-norm (§2.1 items 1, 2; §5.3)
 *     y   = causal_softmax(q k^T / sqrt(D)) v       query head h reads kv head h / (n_head/n_kv_head)
 *     x   = x + y Wo^T
 *     x   = x + relu(rmsnorm(x) Wfc^T)^2 Wproj^T    ReLU^2 MLP of width 4 n_embd (§2.1 item 4; woshipm.com §五.1)
 *   z = rmsnorm(x) Wlm^T                            untied lm_head
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

/* Compute dtype: mirrors COMPUTE_DTYPE (fp32, or bf16 with fp32 master weights). */
typedef enum { NCGPT_F32 = 0, NCGPT_BF16 = 1 } ncgpt_dtype;

typedef struct {
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, mlp_dim, vocab_size, batch, seq_len;
    float rope_base; /* 10000 */
    float norm_eps;  /* 2^-23, the epsilon F.rms_norm uses when none is given */
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
 * (128 for NCGPT_BF16), n_head % n_kv_head == 0, n_embd, mlp_dim and vocab_size are multiples of 64,
 * vocab_size <= 65536, seq_len is a multiple of 128 for NCGPT_BF16 (of 64 for NCGPT_F32), and
 * batch*seq_len*vocab fits the workspace plan.  *out receives the context; free it with ncgpt_destroy. */
ncgpt_status ncgpt_create(const ncgpt_config* cfg, ncgpt_dtype dtype, ncgpt_ctx** out);

/* Bytes of device workspace the context needs (saved activations, cast weights, logits, scratch). */
ncgpt_status ncgpt_workspace_size(const ncgpt_ctx* ctx, size_t* bytes);

/* Attach a caller-owned device workspace of at least ncgpt_workspace_size bytes (256-byte aligned) and the
 * HIP stream (hipStream_t, may be NULL for the null stream) every later call enqueues on.  Uploads the RoPE
 * tables and clears the device error flag (asynchronously on that stream).  May be called again to rebind. */
ncgpt_status ncgpt_bind(ncgpt_ctx* ctx, void* workspace, size_t bytes, void* hip_stream);

/* Forward pass.  ids: int32 [batch*seq_len] (row b*seq_len + t).  params: fp32 [P] packed as above.
 * Both must stay valid and unmodified until ncgpt_backward has been enqueued: the context remembers them. */
ncgpt_status ncgpt_forward(ncgpt_ctx* ctx, const int32_t* ids, const float* params);

/* Cross-entropy of the last forward's logits.  targets: int32 [batch*seq_len]; a negative target is
 * ignored.  loss: fp32 [1], receives the mean over valid targets (NaN if none, with the device flag set).
 * targets must stay valid until ncgpt_backward has been enqueued.  ESTATE before ncgpt_forward. */
ncgpt_status ncgpt_loss(ncgpt_ctx* ctx, const int32_t* targets, float* loss);

/* Backward of the last loss.  grads: fp32 [P] receives grad_scale * d loss / d params (accumulate = 0) or
 * has it added (accumulate = 1).  For k micro-batches of gradient accumulation pass grad_scale = 1/k and
 * accumulate = 1 after the first ("nanochat 项目深度分析" §4.3).  The logits in the workspace are consumed.
 * ESTATE unless ncgpt_loss followed the last ncgpt_forward. */
ncgpt_status ncgpt_backward(ncgpt_ctx* ctx, float* grads, int accumulate, float grad_scale);

/* Synchronise the bound stream and report device-side errors: EDEVICE if the flag is set (the flag is then
 * cleared), EHIP on an asynchronous HIP error, OK otherwise. */
ncgpt_status ncgpt_check(ncgpt_ctx* ctx);

/* Saved-activation readout (for tests).  Copies one activation of the last forward, converted to fp32,
 * into dst (device, fp32, ncgpt_probe_numel elements) and synchronises the stream.  what:
 *   0 x0 [N,C] embedding output          1 xn1 [N,C] pre-attention norm (layer)
 *   2 qkv [N,(H+2Hkv)D] after RoPE/QK-norm (layer)   3 y [N,H*D] attention output (layer)
 *   4 lse_att [B,H,T] attention log-sum-exp (layer)  5 xn2 [N,C] pre-MLP norm (layer)
 *   6 act [N,F] relu(xn2 Wfc^T)^2 (layer)  7 xf [N,C] final norm    8 lse [N] logits log-sum-exp
 *   9 loss_rows [N] per-token loss (0 when ignored)  10 dx0 [N,C] gradient w.r.t. x0 (after backward)
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
