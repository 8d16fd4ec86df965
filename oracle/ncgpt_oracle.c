/*
 * ncgpt_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, fp64 CPU statement of what one nanochat-style GPT training
 * step computes (forward, token cross-entropy, backward).  Only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the HIP library: it has its
 * own config struct, its own parameter packing arithmetic and its own RoPE
 * angles, and it is built by gcc, not hipcc.
 *
 * Every floating-point value is carried in double.  Parameters arrive as the
 * fp32 master weights (that is what the model stores, per the precision
 * paragraph of "nanochat：低成本跑通大模型训练全流程" and §4.2 of the
 * devpress.csdn.net nanochat guide) and are widened to double on entry.
 *
 * Sources, by page and section:
 *  - RoPE, split-half pairing and its signs: "nanochat 项目深度分析" §2.1
 *    item 1 and the annotated apply_rotary_emb in §5.3.
 *  - RoPE first, then RMSNorm on q and k: same page, §2.1 item 2.
 *  - ReLU² MLP: same page, §2.1 item 4; hidden width 4·C: woshipm.com §五.1.
 *  - parameter-free RMSNorm, bias-free linears: same page, §2.1 item 5.
 *  - n_head / n_kv_head (grouped-query attention): same page, §2.1 item 6.
 *  - untied wte / lm_head: same page, §2.1 item 3.
 *  - block = norm + causal self-attention + MLP with residuals:
 *    devpress.csdn.net guide §4.1.
 *  - loss = cross-entropy of logits against the shifted targets: "nanochat
 *    项目深度分析" §2.3 (loader yields inputs, targets) and §6.2 snippet.
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *  - RMSNorm epsilon: F.rms_norm with no eps uses 2^-23 (probed behaviour).
 *  - pre-norm on both sublayers and one final norm before lm_head; no norm
 *    right after the embedding.
 *  - RoPE angle for pair i at position t: t * base^(-2i/D), base 10000,
 *    positions restart at 0 in every sequence.
 *  - attention scale 1/sqrt(D); kv head of query head h is h / (H/Hkv);
 *    causal mask j <= t inside one sequence.
 *  - loss is the mean over targets >= 0; negative targets are ignored.
 *  - block variants (off by default): the "logit stabilisation" woshipm.com
 *    §三 item 1 names without a formula is read as the tanh soft-cap
 *    z <- c tanh(z / c); an RMSNorm of the embedding output is the
 *    embedding-norm variant.
 *
 * Parity: every function here is pinned by tests/test_oracle_*.py (closed
 * forms, invariants, special cases that reduce to library routines, and
 * central finite differences of the whole model).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, mlp_dim, vocab_size, batch, seq_len;
    double rope_base, norm_eps;
    double logit_softcap;  /* > 0: logits z become c tanh(z / c) before the loss (a block variant) */
    int32_t embed_norm;    /* 1: RMSNorm right after the embedding (a block variant) */
} orc_config;

/* ------------------------------------------------------------------ */
/* parameter packing: wte, then per layer Wq Wk Wv Wo Wfc Wproj, then lm_head.
 * Every matrix is [out, in], row-major (the F.linear convention).       */

enum { ORC_WQ = 0, ORC_WK = 1, ORC_WV = 2, ORC_WO = 3, ORC_WFC = 4, ORC_WPROJ = 5 };

static int64_t layer_params(const orc_config* c)
{
    int64_t C = c->n_embd, HD = (int64_t)c->n_head * c->head_dim, KD = (int64_t)c->n_kv_head * c->head_dim;
    int64_t F = c->mlp_dim;
    return HD * C + KD * C + KD * C + C * HD + F * C + C * F;
}

int64_t orc_num_params(const orc_config* c)
{
    int64_t VC = (int64_t)c->vocab_size * c->n_embd;
    return VC + (int64_t)c->n_layer * layer_params(c) + VC;
}

/* layer = -1: which 0 = wte, 1 = lm_head.  layer >= 0: which = ORC_W*. */
int orc_param_slice(const orc_config* c, int layer, int which, int64_t* offset, int64_t* rows, int64_t* cols)
{
    int64_t C = c->n_embd, V = c->vocab_size, F = c->mlp_dim;
    int64_t HD = (int64_t)c->n_head * c->head_dim, KD = (int64_t)c->n_kv_head * c->head_dim;
    if (layer < 0) {
        if (which == 0) { *offset = 0; *rows = V; *cols = C; return 0; }
        if (which == 1) { *offset = V * C + (int64_t)c->n_layer * layer_params(c); *rows = V; *cols = C; return 0; }
        return -1;
    }
    if (layer >= c->n_layer) return -1;
    int64_t base = V * C + (int64_t)layer * layer_params(c);
    int64_t r[6] = {HD, KD, KD, C, F, C};
    int64_t k[6] = {C, C, C, HD, C, F};
    if (which < 0 || which > 5) return -1;
    int64_t off = base;
    for (int i = 0; i < which; ++i) off += r[i] * k[i];
    *offset = off; *rows = r[which]; *cols = k[which];
    return 0;
}

/* ------------------------------------------------------------------ */
/* primitives                                                          */

/* y = x W^T for x [rows, in], W [out, in].  Each output is one dot product
 * summed over i in increasing order; four outputs are formed side by side
 * only to keep the CPU's adders busy (the sum order of each is unchanged). */
void orc_linear_fwd(const double* x, const double* W, int64_t rows, int64_t in, int64_t out, double* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < rows; ++n) {
        const double* xr = x + n * in;
        int64_t o = 0;
        for (; o + 4 <= out; o += 4) {
            const double *w0 = W + o * in, *w1 = w0 + in, *w2 = w1 + in, *w3 = w2 + in;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int64_t i = 0; i < in; ++i) {
                s0 += xr[i] * w0[i];
                s1 += xr[i] * w1[i];
                s2 += xr[i] * w2[i];
                s3 += xr[i] * w3[i];
            }
            y[n * out + o] = s0; y[n * out + o + 1] = s1; y[n * out + o + 2] = s2; y[n * out + o + 3] = s3;
        }
        for (; o < out; ++o) {
            double s = 0.0;
            for (int64_t i = 0; i < in; ++i) s += xr[i] * W[o * in + i];
            y[n * out + o] = s;
        }
    }
}

/* dx = dy W  (dx [rows,in], overwritten);  dW (+)= dy^T x  (dW [out,in], added to
 * when acc_dw = 1, overwritten when 0).  Either output may be NULL.
 * dx[n,i] sums over o in increasing order, dW[o,i] over n in increasing
 * order; the partial sums run along rows of W and x so memory is read
 * contiguously. */
void orc_linear_bwd(const double* x, const double* W, const double* dy, int64_t rows, int64_t in, int64_t out,
                    double* dx, double* dW, int acc_dw)
{
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < rows; ++n) {
            double* d = dx + n * in;
            for (int64_t i = 0; i < in; ++i) d[i] = 0.0;
            for (int64_t o = 0; o < out; ++o) {
                const double a = dy[n * out + o];
                const double* w = W + o * in;
                for (int64_t i = 0; i < in; ++i) d[i] += a * w[i];
            }
        }
    }
    if (dW) {
        const int64_t OB = 8;
#pragma omp parallel
        {
            double* acc = (double*)malloc(sizeof(double) * (size_t)(OB * in));
#pragma omp for schedule(static)
            for (int64_t o0 = 0; o0 < out; o0 += OB) {
                const int64_t ob = out - o0 < OB ? out - o0 : OB;
                for (int64_t k = 0; k < ob * in; ++k) acc[k] = 0.0;
                for (int64_t n = 0; n < rows; ++n) {
                    const double* xr = x + n * in;
                    for (int64_t k = 0; k < ob; ++k) {
                        const double a = dy[n * out + o0 + k];
                        double* t = acc + k * in;
                        for (int64_t i = 0; i < in; ++i) t[i] += a * xr[i];
                    }
                }
                for (int64_t k = 0; k < ob; ++k)
                    for (int64_t i = 0; i < in; ++i) {
                        double* g = dW + (o0 + k) * in + i;
                        *g = acc_dw ? *g + acc[k * in + i] : acc[k * in + i];
                    }
            }
            free(acc);
        }
    }
}

/* Parameter-free RMSNorm over the last dim of n: y = x / sqrt(mean(x^2) + eps).
 * rstd[r] = 1/sqrt(mean(x^2)+eps) is returned for the backward. */
void orc_rmsnorm_fwd(const double* x, int64_t rows, int64_t n, double eps, double* y, double* rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t i = 0; i < n; ++i) ss += x[r * n + i] * x[r * n + i];
        double rs = 1.0 / sqrt(ss / (double)n + eps);
        if (rstd) rstd[r] = rs;
        for (int64_t i = 0; i < n; ++i) y[r * n + i] = x[r * n + i] * rs;
    }
}

/* Derivative of the map above: with y the forward output and rstd its scale,
 * dx = rstd * (dy - y * mean(dy * y)).  accumulate = 1 adds into dx. */
void orc_rmsnorm_bwd(const double* y, const double* rstd, const double* dy, int64_t rows, int64_t n, double* dx,
                     int accumulate)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double dot = 0.0;
        for (int64_t i = 0; i < n; ++i) dot += dy[r * n + i] * y[r * n + i];
        dot /= (double)n;
        for (int64_t i = 0; i < n; ++i) {
            double g = rstd[r] * (dy[r * n + i] - y[r * n + i] * dot);
            dx[r * n + i] = accumulate ? dx[r * n + i] + g : g;
        }
    }
}

/* Angle of pair i (i < D/2) at position t. */
static double rope_angle(int64_t t, int64_t i, int64_t D, double base)
{
    return (double)t * pow(base, -2.0 * (double)i / (double)D);
}

/* RoPE on x laid out [B, T, nh, D] (the 4-D head layout the pages assert).
 * Pair (i, i + D/2) at position t is rotated as
 *   y_i       =  x_i cos + x_{i+D/2} sin
 *   y_{i+D/2} = -x_i sin + x_{i+D/2} cos
 * (split halves, not interleaved).  inverse = 1 applies the transpose, which
 * is both the inverse rotation and the backward of the map. */
void orc_rope(double* x, int64_t B, int64_t T, int64_t nh, int64_t D, double base, int inverse)
{
    int64_t half = D / 2;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < B * T; ++bt) {
        int64_t t = bt % T;
        for (int64_t h = 0; h < nh; ++h) {
            double* v = x + (bt * nh + h) * D;
            for (int64_t i = 0; i < half; ++i) {
                double a = rope_angle(t, i, D, base);
                double cs = cos(a), sn = sin(a);
                double x1 = v[i], x2 = v[i + half];
                if (!inverse) {
                    v[i] = x1 * cs + x2 * sn;
                    v[i + half] = -x1 * sn + x2 * cs;
                } else {
                    v[i] = x1 * cs - x2 * sn;
                    v[i + half] = x1 * sn + x2 * cs;
                }
            }
        }
    }
}

/* Causal grouped-query attention.  q [B,T,H,D], k and v [B,T,Hkv,D].
 * For query head h the kv head is g = h / (H/Hkv).
 *   o[b,t,h] = sum_{j<=t} softmax_j(q[b,t,h].k[b,j,g] / sqrt(D)) v[b,j,g]
 * The full score row is materialised; lse[b,h,t] is its log-sum-exp
 * (of the scaled scores).  Keys after t are never read. */
void orc_attention_fwd(const double* q, const double* k, const double* v, int64_t B, int64_t T, int64_t H,
                       int64_t Hkv, int64_t D, double* o, double* lse)
{
    int64_t r = H / Hkv;
    double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic)
    for (int64_t bht = 0; bht < B * H * T; ++bht) {
        int64_t b = bht / (H * T), h = (bht / T) % H, t = bht % T, g = h / r;
        double* s = (double*)malloc(sizeof(double) * (size_t)(t + 1));
        const double* qv = q + ((b * T + t) * H + h) * D;
        double m = -INFINITY;
        for (int64_t j = 0; j <= t; ++j) {
            const double* kv = k + ((b * T + j) * Hkv + g) * D;
            double d = 0.0;
            for (int64_t i = 0; i < D; ++i) d += qv[i] * kv[i];
            s[j] = d * scale;
            if (s[j] > m) m = s[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j <= t; ++j) { s[j] = exp(s[j] - m); z += s[j]; }
        double* ov = o + ((b * T + t) * H + h) * D;
        for (int64_t i = 0; i < D; ++i) ov[i] = 0.0;
        for (int64_t j = 0; j <= t; ++j) {
            const double* vv = v + ((b * T + j) * Hkv + g) * D;
            double p = s[j] / z;
            for (int64_t i = 0; i < D; ++i) ov[i] += p * vv[i];
        }
        if (lse) lse[(b * H + h) * T + t] = m + log(z);
        free(s);
    }
}

/* Backward of the attention above, written from its definition:
 *   P = softmax(S), S = q k^T / sqrt(D) on j <= t
 *   dv_j  = sum_{h in group, t >= j} P_tj do_t
 *   dP_tj = do_t . v_j
 *   dS_tj = P_tj (dP_tj - sum_j' P_tj' dP_tj')
 *   dq_t  = sum_j dS_tj k_j / sqrt(D);   dk_j = sum_{h in group, t} dS_tj q_t / sqrt(D)
 * Outputs are overwritten. */
void orc_attention_bwd(const double* q, const double* k, const double* v, const double* dout, int64_t B, int64_t T,
                       int64_t H, int64_t Hkv, int64_t D, double* dq, double* dk, double* dv)
{
    int64_t r = H / Hkv;
    double scale = 1.0 / sqrt((double)D);
    memset(dk, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    /* one task per (b, g): owns dk, dv of that kv head, so no write races */
#pragma omp parallel for schedule(dynamic)
    for (int64_t bg = 0; bg < B * Hkv; ++bg) {
        int64_t b = bg / Hkv, g = bg % Hkv;
        double* P = (double*)malloc(sizeof(double) * (size_t)T);
        double* dP = (double*)malloc(sizeof(double) * (size_t)T);
        for (int64_t h = g * r; h < (g + 1) * r; ++h)
            for (int64_t t = 0; t < T; ++t) {
                const double* qv = q + ((b * T + t) * H + h) * D;
                const double* dov = dout + ((b * T + t) * H + h) * D;
                double m = -INFINITY;
                for (int64_t j = 0; j <= t; ++j) {
                    const double* kv = k + ((b * T + j) * Hkv + g) * D;
                    double d = 0.0;
                    for (int64_t i = 0; i < D; ++i) d += qv[i] * kv[i];
                    P[j] = d * scale;
                    if (P[j] > m) m = P[j];
                }
                double z = 0.0;
                for (int64_t j = 0; j <= t; ++j) { P[j] = exp(P[j] - m); z += P[j]; }
                double rowdot = 0.0;
                for (int64_t j = 0; j <= t; ++j) {
                    P[j] /= z;
                    const double* vv = v + ((b * T + j) * Hkv + g) * D;
                    double d = 0.0;
                    for (int64_t i = 0; i < D; ++i) d += dov[i] * vv[i];
                    dP[j] = d;
                    rowdot += P[j] * d;
                }
                double* dqv = dq + ((b * T + t) * H + h) * D;
                for (int64_t i = 0; i < D; ++i) dqv[i] = 0.0;
                for (int64_t j = 0; j <= t; ++j) {
                    double ds = P[j] * (dP[j] - rowdot) * scale;
                    const double* kv = k + ((b * T + j) * Hkv + g) * D;
                    double* dkv = dk + ((b * T + j) * Hkv + g) * D;
                    double* dvv = dv + ((b * T + j) * Hkv + g) * D;
                    for (int64_t i = 0; i < D; ++i) {
                        dqv[i] += ds * kv[i];
                        dkv[i] += ds * qv[i];
                        dvv[i] += P[j] * dov[i];
                    }
                }
            }
        free(P);
        free(dP);
    }
}

/* Token cross-entropy of logits z [rows, V] against targets (negative =
 * ignored).  lse[n] = log sum_j exp z[n,j]; loss_rows[n] = lse - z[n, target]
 * (0 for ignored rows).  Returns the number of valid rows; *loss is the mean
 * over valid rows (NaN when there are none). */
int64_t orc_cross_entropy_fwd(const double* z, const int32_t* targets, int64_t rows, int64_t V, double* lse,
                              double* loss_rows, double* loss)
{
    int64_t valid = 0;
    double total = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : valid, total)
    for (int64_t n = 0; n < rows; ++n) {
        const double* zr = z + n * V;
        double m = -INFINITY;
        for (int64_t j = 0; j < V; ++j) if (zr[j] > m) m = zr[j];
        double s = 0.0;
        for (int64_t j = 0; j < V; ++j) s += exp(zr[j] - m);
        double l = m + log(s);
        if (lse) lse[n] = l;
        double ln = 0.0;
        if (targets[n] >= 0) { ln = l - zr[targets[n]]; valid += 1; total += ln; }
        if (loss_rows) loss_rows[n] = ln;
    }
    if (loss) *loss = valid > 0 ? total / (double)valid : NAN;
    return valid;
}

/* dz = grad_scale * (softmax(z) - onehot(target)) / valid on valid rows, 0 on ignored rows. */
void orc_cross_entropy_bwd(const double* z, const int32_t* targets, int64_t rows, int64_t V, int64_t valid,
                           double grad_scale, double* dz)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < rows; ++n) {
        const double* zr = z + n * V;
        double* d = dz + n * V;
        if (targets[n] < 0 || valid == 0) { for (int64_t j = 0; j < V; ++j) d[j] = 0.0; continue; }
        double m = -INFINITY;
        for (int64_t j = 0; j < V; ++j) if (zr[j] > m) m = zr[j];
        double s = 0.0;
        for (int64_t j = 0; j < V; ++j) s += exp(zr[j] - m);
        double c = grad_scale / (double)valid;
        for (int64_t j = 0; j < V; ++j) d[j] = c * exp(zr[j] - m) / s;
        d[targets[n]] -= c;
    }
}

/* Soft-cap of the logits, z <- c tanh(z / c) (c > 0; c <= 0 leaves z alone), and its backward: with the
 * uncapped z, dz <- dz (1 - tanh(z / c)^2). */
void orc_softcap_fwd(double* z, int64_t n, double c)
{
    if (c <= 0.0) return;
    for (int64_t i = 0; i < n; ++i) z[i] = c * tanh(z[i] / c);
}

void orc_softcap_bwd(const double* z, double* dz, int64_t n, double c)
{
    if (c <= 0.0) return;
    for (int64_t i = 0; i < n; ++i) {
        const double t = tanh(z[i] / c);
        dz[i] *= 1.0 - t * t;
    }
}

/* ------------------------------------------------------------------ */
/* the whole model                                                     */

/* Saved activations, one flat double buffer, in this order:
 *   x0 [N,C]
 *   per layer l: xn1 [N,C], rstd1 [N], qkv [N,(H+2Hkv)D] (q,k after RoPE and
 *                QK-norm, v as projected), rstdq [N,H], rstdk [N,Hkv],
 *                y [N,HD], lse_att [B,H,T], xmid [N,C], xn2 [N,C], rstd2 [N],
 *                a [N,F] (= max(0, xn2 Wfc^T)), xout [N,C]
 *   xf [N,C], rstdf [N], lse [N], loss_rows [N], x0n [N,C], rstd0 [N]
 * orc_acts_layout fills the element offsets of each piece. */
enum {
    ORC_A_XN1 = 0, ORC_A_RSTD1, ORC_A_QKV, ORC_A_RSTDQ, ORC_A_RSTDK, ORC_A_Y, ORC_A_LSEATT,
    ORC_A_XMID, ORC_A_XN2, ORC_A_RSTD2, ORC_A_A, ORC_A_XOUT, ORC_A_NLAYER
};

typedef struct {
    int64_t x0, layer0, layer_stride, per_layer[ORC_A_NLAYER], xf, rstdf, lse, loss_rows, x0n, rstd0, total;
} orc_acts_layout;

void orc_get_acts_layout(const orc_config* c, orc_acts_layout* o)
{
    int64_t N = (int64_t)c->batch * c->seq_len, C = c->n_embd, H = c->n_head, Hkv = c->n_kv_head;
    int64_t D = c->head_dim, F = c->mlp_dim, QKV = (H + 2 * Hkv) * D;
    int64_t sz[ORC_A_NLAYER] = {N * C, N, N * QKV, N * H, N * Hkv, N * H * D, (int64_t)c->batch * H * c->seq_len,
                                N * C, N * C, N, N * F, N * C};
    o->x0 = 0;
    o->layer0 = N * C;
    int64_t off = 0;
    for (int i = 0; i < ORC_A_NLAYER; ++i) { o->per_layer[i] = off; off += sz[i]; }
    o->layer_stride = off;
    int64_t end = o->layer0 + (int64_t)c->n_layer * off;
    o->xf = end;
    o->rstdf = end + N * C;
    o->lse = o->rstdf + N;
    o->loss_rows = o->lse + N;
    o->x0n = o->loss_rows + N;        /* the residual stream's start: x0, or rms(x0) with embed_norm */
    o->rstd0 = o->x0n + N * C;
    o->total = o->rstd0 + N;
}

static int check_config(const orc_config* c)
{
    if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_kv_head < 1 || c->head_dim < 2 ||
        (c->head_dim & 1) || c->mlp_dim < 1 || c->vocab_size < 1 || c->batch < 1 || c->seq_len < 1)
        return -1;
    if (c->n_head % c->n_kv_head) return -1;
    return 0;
}

/* Copy q or k heads out of the packed [N, (H+2Hkv)D] row into [N, nh, D]. */
static void unpack_cols(const double* qkv, int64_t N, int64_t QKV, int64_t col0, int64_t width, double* out)
{
    for (int64_t n = 0; n < N; ++n) memcpy(out + n * width, qkv + n * QKV + col0, sizeof(double) * (size_t)width);
}

static void pack_cols(const double* in, int64_t N, int64_t QKV, int64_t col0, int64_t width, double* qkv)
{
    for (int64_t n = 0; n < N; ++n) memcpy(qkv + n * QKV + col0, in + n * width, sizeof(double) * (size_t)width);
}

/* Forward of the whole stack and the loss, saving every activation into
 * acts (laid out by orc_get_acts_layout).  Returns the number of valid
 * targets, or -1 on a bad config / token id. */
static int64_t model_forward(const orc_config* c, const int32_t* ids, const int32_t* targets, const double* p,
                             double* acts, double* loss)
{
    orc_acts_layout lay;
    orc_get_acts_layout(c, &lay);
    int64_t B = c->batch, T = c->seq_len, N = B * T, C = c->n_embd, H = c->n_head, Hkv = c->n_kv_head;
    int64_t D = c->head_dim, F = c->mlp_dim, V = c->vocab_size, HD = H * D, KD = Hkv * D, QKV = HD + 2 * KD;
    double eps = c->norm_eps;
    int64_t off, rr, cc;

    double* x = (double*)malloc(sizeof(double) * (size_t)(N * C));
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(N * (F > QKV ? F : QKV)));
    double* qh = (double*)malloc(sizeof(double) * (size_t)(N * HD));
    double* kh = (double*)malloc(sizeof(double) * (size_t)(N * KD));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(N * KD));

    /* embedding: x0[n] = wte[ids[n]] */
    orc_param_slice(c, -1, 0, &off, &rr, &cc);
    for (int64_t n = 0; n < N; ++n) {
        if (ids[n] < 0 || ids[n] >= V) { free(x); free(tmp); free(qh); free(kh); free(vh); return -1; }
        memcpy(x + n * C, p + off + (int64_t)ids[n] * C, sizeof(double) * (size_t)C);
    }
    memcpy(acts + lay.x0, x, sizeof(double) * (size_t)(N * C));
    if (c->embed_norm) orc_rmsnorm_fwd(acts + lay.x0, N, C, eps, x, acts + lay.rstd0);
    memcpy(acts + lay.x0n, x, sizeof(double) * (size_t)(N * C));

    for (int l = 0; l < c->n_layer; ++l) {
        double* A = acts + lay.layer0 + (int64_t)l * lay.layer_stride;
        double* xn1 = A + lay.per_layer[ORC_A_XN1];
        double* qkv = A + lay.per_layer[ORC_A_QKV];
        double* y = A + lay.per_layer[ORC_A_Y];
        /* attention sublayer */
        orc_rmsnorm_fwd(x, N, C, eps, xn1, A + lay.per_layer[ORC_A_RSTD1]);
        orc_param_slice(c, l, ORC_WQ, &off, &rr, &cc);
        orc_linear_fwd(xn1, p + off, N, C, HD, qh);
        orc_param_slice(c, l, ORC_WK, &off, &rr, &cc);
        orc_linear_fwd(xn1, p + off, N, C, KD, kh);
        orc_param_slice(c, l, ORC_WV, &off, &rr, &cc);
        orc_linear_fwd(xn1, p + off, N, C, KD, vh);
        orc_rope(qh, B, T, H, D, c->rope_base, 0);
        orc_rope(kh, B, T, Hkv, D, c->rope_base, 0);
        orc_rmsnorm_fwd(qh, N * H, D, eps, qh, A + lay.per_layer[ORC_A_RSTDQ]);
        orc_rmsnorm_fwd(kh, N * Hkv, D, eps, kh, A + lay.per_layer[ORC_A_RSTDK]);
        pack_cols(qh, N, QKV, 0, HD, qkv);
        pack_cols(kh, N, QKV, HD, KD, qkv);
        pack_cols(vh, N, QKV, HD + KD, KD, qkv);
        orc_attention_fwd(qh, kh, vh, B, T, H, Hkv, D, y, A + lay.per_layer[ORC_A_LSEATT]);
        orc_param_slice(c, l, ORC_WO, &off, &rr, &cc);
        orc_linear_fwd(y, p + off, N, HD, C, tmp);
        for (int64_t i = 0; i < N * C; ++i) x[i] += tmp[i];
        memcpy(A + lay.per_layer[ORC_A_XMID], x, sizeof(double) * (size_t)(N * C));
        /* MLP sublayer */
        double* xn2 = A + lay.per_layer[ORC_A_XN2];
        double* a = A + lay.per_layer[ORC_A_A];
        orc_rmsnorm_fwd(x, N, C, eps, xn2, A + lay.per_layer[ORC_A_RSTD2]);
        orc_param_slice(c, l, ORC_WFC, &off, &rr, &cc);
        orc_linear_fwd(xn2, p + off, N, C, F, a);
        for (int64_t i = 0; i < N * F; ++i) { a[i] = a[i] > 0.0 ? a[i] : 0.0; tmp[i] = a[i] * a[i]; }
        orc_param_slice(c, l, ORC_WPROJ, &off, &rr, &cc);
        double* proj = (double*)malloc(sizeof(double) * (size_t)(N * C));
        orc_linear_fwd(tmp, p + off, N, F, C, proj);
        for (int64_t i = 0; i < N * C; ++i) x[i] += proj[i];
        free(proj);
        memcpy(A + lay.per_layer[ORC_A_XOUT], x, sizeof(double) * (size_t)(N * C));
    }
    double* xf = acts + lay.xf;
    orc_rmsnorm_fwd(x, N, C, eps, xf, acts + lay.rstdf);
    free(x); free(tmp); free(qh); free(kh); free(vh);

    /* lm_head and loss, one row block at a time so the logits never exceed ~64 MB */
    orc_param_slice(c, -1, 1, &off, &rr, &cc);
    int64_t blk = (int64_t)(8 * 1024 * 1024) / V;
    if (blk < 1) blk = 1;
    double* z = (double*)malloc(sizeof(double) * (size_t)(blk * V));
    int64_t valid = 0;
    double total = 0.0;
    for (int64_t n0 = 0; n0 < N; n0 += blk) {
        int64_t nb = N - n0 < blk ? N - n0 : blk;
        double part;
        orc_linear_fwd(xf + n0 * C, p + off, nb, C, V, z);
        orc_softcap_fwd(z, nb * V, c->logit_softcap);
        int64_t vb = orc_cross_entropy_fwd(z, targets + n0, nb, V, acts + lay.lse + n0, acts + lay.loss_rows + n0, &part);
        if (vb > 0) total += part * (double)vb;
        valid += vb;
    }
    free(z);
    *loss = valid > 0 ? total / (double)valid : NAN;
    return valid;
}

int64_t orc_acts_size(const orc_config* c)
{
    orc_acts_layout lay;
    orc_get_acts_layout(c, &lay);
    return lay.total;
}

static double* widen(const float* p, int64_t P)
{
    double* d = (double*)malloc(sizeof(double) * (size_t)P);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < P; ++i) d[i] = (double)p[i];
    return d;
}

/* Forward + loss with fp64 parameters.  acts may be NULL (then an internal
 * buffer is used).  Returns valid-target count, -1 on error. */
int64_t orc_forward_f64(const orc_config* c, const int32_t* ids, const int32_t* targets, const double* p,
                        double* acts, double* loss)
{
    if (check_config(c)) return -1;
    double* own = NULL;
    if (!acts) { own = (double*)malloc(sizeof(double) * (size_t)orc_acts_size(c)); acts = own; }
    int64_t v = model_forward(c, ids, targets, p, acts, loss);
    free(own);
    return v;
}

/* Same, with the fp32 master weights the model stores (widened exactly). */
int64_t orc_forward(const orc_config* c, const int32_t* ids, const int32_t* targets, const float* params,
                    double* acts, double* loss)
{
    if (check_config(c)) return -1;
    double* p = widen(params, orc_num_params(c));
    int64_t v = orc_forward_f64(c, ids, targets, p, acts, loss);
    free(p);
    return v;
}

/* grads[P] = grad_scale * d loss / d params, for the mean loss over valid
 * targets, with fp64 parameters.  Runs the forward itself.  Returns the
 * valid-target count, -1 on error. */
int64_t orc_grad_f64(const orc_config* c, const int32_t* ids, const int32_t* targets, const double* p,
                     double grad_scale, double* grads, double* loss)
{
    if (check_config(c)) return -1;
    int64_t P = orc_num_params(c);
    orc_acts_layout lay;
    orc_get_acts_layout(c, &lay);
    double* acts = (double*)malloc(sizeof(double) * (size_t)lay.total);
    int64_t valid = model_forward(c, ids, targets, p, acts, loss);
    if (valid < 0) { free(acts); return -1; }
    memset(grads, 0, sizeof(double) * (size_t)P);

    int64_t B = c->batch, T = c->seq_len, N = B * T, C = c->n_embd, H = c->n_head, Hkv = c->n_kv_head;
    int64_t D = c->head_dim, F = c->mlp_dim, V = c->vocab_size, HD = H * D, KD = Hkv * D, QKV = HD + 2 * KD;
    int64_t off, rr, cc;

    /* lm_head + cross-entropy: recompute logits in row blocks */
    double* xf = acts + lay.xf;
    double* dxf = (double*)malloc(sizeof(double) * (size_t)(N * C));
    orc_param_slice(c, -1, 1, &off, &rr, &cc);
    int64_t blk = (int64_t)(8 * 1024 * 1024) / V;
    if (blk < 1) blk = 1;
    double* z = (double*)malloc(sizeof(double) * (size_t)(blk * V));
    double* dz = (double*)malloc(sizeof(double) * (size_t)(blk * V));
    for (int64_t n0 = 0; n0 < N; n0 += blk) {
        int64_t nb = N - n0 < blk ? N - n0 : blk;
        orc_linear_fwd(xf + n0 * C, p + off, nb, C, V, z);
        if (c->logit_softcap > 0.0) {
            double* zc = (double*)malloc(sizeof(double) * (size_t)(nb * V));
            memcpy(zc, z, sizeof(double) * (size_t)(nb * V));
            orc_softcap_fwd(zc, nb * V, c->logit_softcap);
            orc_cross_entropy_bwd(zc, targets + n0, nb, V, valid, grad_scale, dz);
            orc_softcap_bwd(z, dz, nb * V, c->logit_softcap);
            free(zc);
        } else {
            orc_cross_entropy_bwd(z, targets + n0, nb, V, valid, grad_scale, dz);
        }
        orc_linear_bwd(xf + n0 * C, p + off, dz, nb, C, V, dxf + n0 * C, grads + off, 1);
    }
    free(z);
    free(dz);

    /* final norm */
    double* dx = (double*)malloc(sizeof(double) * (size_t)(N * C));
    orc_rmsnorm_bwd(xf, acts + lay.rstdf, dxf, N, C, dx, 0);
    free(dxf);

    double* dbuf = (double*)malloc(sizeof(double) * (size_t)(N * (F > QKV ? F : QKV)));
    double* act = (double*)malloc(sizeof(double) * (size_t)(N * F));
    double* dnrm = (double*)malloc(sizeof(double) * (size_t)(N * C));
    double* qh = (double*)malloc(sizeof(double) * (size_t)(N * HD));
    double* kh = (double*)malloc(sizeof(double) * (size_t)(N * KD));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(N * KD));
    double* dq = (double*)malloc(sizeof(double) * (size_t)(N * HD));
    double* dk = (double*)malloc(sizeof(double) * (size_t)(N * KD));
    double* dv = (double*)malloc(sizeof(double) * (size_t)(N * KD));
    double* dyb = (double*)malloc(sizeof(double) * (size_t)(N * HD));

    for (int l = c->n_layer - 1; l >= 0; --l) {
        double* A = acts + lay.layer0 + (int64_t)l * lay.layer_stride;
        /* MLP: xout = xmid + (a*a) Wproj^T, a = relu(xn2 Wfc^T) */
        double* a = A + lay.per_layer[ORC_A_A];
        for (int64_t i = 0; i < N * F; ++i) act[i] = a[i] * a[i];
        orc_param_slice(c, l, ORC_WPROJ, &off, &rr, &cc);
        orc_linear_bwd(act, p + off, dx, N, F, C, dbuf, grads + off, 1); /* dbuf = dact */
        for (int64_t i = 0; i < N * F; ++i) dbuf[i] *= 2.0 * a[i];        /* dh = dact * 2 max(0,h) */
        orc_param_slice(c, l, ORC_WFC, &off, &rr, &cc);
        orc_linear_bwd(A + lay.per_layer[ORC_A_XN2], p + off, dbuf, N, C, F, dnrm, grads + off, 1);
        orc_rmsnorm_bwd(A + lay.per_layer[ORC_A_XN2], A + lay.per_layer[ORC_A_RSTD2], dnrm, N, C, dx, 1);

        /* attention: xmid = xin + y Wo^T */
        orc_param_slice(c, l, ORC_WO, &off, &rr, &cc);
        orc_linear_bwd(A + lay.per_layer[ORC_A_Y], p + off, dx, N, HD, C, dyb, grads + off, 1);
        double* qkv = A + lay.per_layer[ORC_A_QKV];
        unpack_cols(qkv, N, QKV, 0, HD, qh);
        unpack_cols(qkv, N, QKV, HD, KD, kh);
        unpack_cols(qkv, N, QKV, HD + KD, KD, vh);
        orc_attention_bwd(qh, kh, vh, dyb, B, T, H, Hkv, D, dq, dk, dv);
        /* QK-norm backward (qh, kh hold the normalised outputs), then RoPE transpose */
        orc_rmsnorm_bwd(qh, A + lay.per_layer[ORC_A_RSTDQ], dq, N * H, D, dq, 0);
        orc_rmsnorm_bwd(kh, A + lay.per_layer[ORC_A_RSTDK], dk, N * Hkv, D, dk, 0);
        orc_rope(dq, B, T, H, D, c->rope_base, 1);
        orc_rope(dk, B, T, Hkv, D, c->rope_base, 1);
        double* xn1 = A + lay.per_layer[ORC_A_XN1];
        orc_param_slice(c, l, ORC_WQ, &off, &rr, &cc);
        orc_linear_bwd(xn1, p + off, dq, N, C, HD, dnrm, grads + off, 1);
        orc_param_slice(c, l, ORC_WK, &off, &rr, &cc);
        orc_linear_bwd(xn1, p + off, dk, N, C, KD, dbuf, grads + off, 1);
        for (int64_t i = 0; i < N * C; ++i) dnrm[i] += dbuf[i];
        orc_param_slice(c, l, ORC_WV, &off, &rr, &cc);
        orc_linear_bwd(xn1, p + off, dv, N, C, KD, dbuf, grads + off, 1);
        for (int64_t i = 0; i < N * C; ++i) dnrm[i] += dbuf[i];
        orc_rmsnorm_bwd(xn1, A + lay.per_layer[ORC_A_RSTD1], dnrm, N, C, dx, 1);
    }

    /* embedding norm, then the embedding: dwte[ids[n]] += dx0[n] */
    if (c->embed_norm) orc_rmsnorm_bwd(acts + lay.x0n, acts + lay.rstd0, dx, N, C, dx, 0);
    orc_param_slice(c, -1, 0, &off, &rr, &cc);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < C; ++i) grads[off + (int64_t)ids[n] * C + i] += dx[n * C + i];

    free(dx); free(dbuf); free(act); free(dnrm); free(qh); free(kh); free(vh); free(dq); free(dk); free(dv);
    free(dyb); free(acts);
    return valid;
}

/* Same, with the fp32 master weights the model stores (widened exactly). */
int64_t orc_grad(const orc_config* c, const int32_t* ids, const int32_t* targets, const float* params,
                 double grad_scale, double* grads, double* loss)
{
    if (check_config(c)) return -1;
    double* p = widen(params, orc_num_params(c));
    int64_t v = orc_grad_f64(c, ids, targets, p, grad_scale, grads, loss);
    free(p);
    return v;
}
