/*
 * optim_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain fp64 CPU statement of the optimizer step that follows the backward
 * pass in the nanochat pretraining loop: Muon for the Transformer matrices and
 * AdamW for the embedding and the unembedding ("nanochat 项目深度分析" §2.2 and
 * §4.2: learning rates 0.2 for the embedding, 0.004 for the unembedding and
 * 0.02 for the matrices; Muon = SGD-momentum, then an orthogonalisation of
 * the update by a Newton-Schulz iteration, then a step scale from the matrix
 * aspect ratio).  Built into liboracle.so with ncgpt_oracle.c; shares nothing
 * with the HIP library.
 *
 * The pages name the iteration but leave its details out.  It is taken from the
 * published Muon description (K. Jordan et al., "Muon: an optimizer for the
 * hidden layers of neural networks", 2024), which also fixes the momentum form:
 *   buf = mu buf + (1 - mu) g,   u = (1 - mu) g + mu buf  (Nesterov; else u = buf),
 *   X0 = u / max(||u||_F, eps) taken wide (a tall matrix is transposed),
 *   five steps of  A = X X^T,  X <- a X + (b A + c A A) X  with (a, b, c) =
 *   (3.4445, -4.7750, 2.0315),
 *   p <- p (1 - lr wd) - lr sqrt(max(1, rows / cols)) X.
 * AdamW is Loshchilov and Hutter's decoupled-weight-decay Adam with bias
 * correction.  The constants arrive as arguments.
 *
 * Pins (tests/test_oracle_optim.py): the iteration equals the closed form
 * U p5(S / ||G||_F) V^T from an SVD (p5 = the quintic applied five times);
 * AdamW equals torch.optim.AdamW in fp64; the composed Muon step agrees with
 * torch.optim.Muon to the precision of that routine's bf16 iteration.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {   /* the layout of ncgpt_oracle.c's config */
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, mlp_dim, vocab_size, batch, seq_len;
    double rope_base, norm_eps;
    double logit_softcap;
    int32_t embed_norm;
} orc_config;

int orc_param_slice(const orc_config* c, int layer, int which, int64_t* offset, int64_t* rows, int64_t* cols);
int64_t orc_num_params(const orc_config* c);

typedef struct {
    double matrix_lr, embedding_lr, unembedding_lr;
    double muon_momentum;
    int32_t muon_nesterov, ns_steps;
    double ns_a, ns_b, ns_c, ns_eps;
    double adam_beta1, adam_beta2, adam_eps;
    double weight_decay;
} orc_optim;

/* C [m, n] = A [m, k] B^T with B [n, k]: each entry one dot product summed over k in increasing order. */
static void matmul_abt(const double* A, const double* B, int64_t m, int64_t n, int64_t k, double* C)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t q = 0; q < k; ++q) s += A[i * k + q] * B[j * k + q];
            C[i * n + j] = s;
        }
}

/* C [m, n] = A [m, k] B with B [k, n]. */
static void matmul_ab(const double* A, const double* B, int64_t m, int64_t n, int64_t k, double* C)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) C[i * n + j] = 0.0;
        for (int64_t q = 0; q < k; ++q) {
            const double a = A[i * k + q];
            for (int64_t j = 0; j < n; ++j) C[i * n + j] += a * B[q * n + j];
        }
    }
}

/* The Newton-Schulz iteration of the published Muon description on G [rows, cols]; out [rows, cols]. */
void orc_newton_schulz(const double* G, int64_t rows, int64_t cols, int steps, double a, double b, double c,
                       double eps, double* out)
{
    const int tall = rows > cols;
    const int64_t m = tall ? cols : rows, n = tall ? rows : cols;   /* X is m x n with m <= n */
    double* X = malloc(sizeof(double) * m * n);
    double* Y = malloc(sizeof(double) * m * n);
    double* A = malloc(sizeof(double) * m * m);
    double* AA = malloc(sizeof(double) * m * m);
    double* Bm = malloc(sizeof(double) * m * m);
    double ss = 0.0;
    for (int64_t i = 0; i < rows * cols; ++i) ss += G[i] * G[i];
    double nrm = sqrt(ss);
    if (nrm < eps) nrm = eps;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t q = 0; q < cols; ++q) {
            const double v = G[r * cols + q] / nrm;
            if (tall) X[q * n + r] = v;
            else X[r * n + q] = v;
        }
    for (int s = 0; s < steps; ++s) {
        matmul_abt(X, X, m, m, n, A);      /* A = X X^T */
        matmul_ab(A, A, m, m, m, AA);      /* A A */
        for (int64_t i = 0; i < m * m; ++i) Bm[i] = b * A[i] + c * AA[i];
        matmul_ab(Bm, X, m, n, m, Y);      /* B X */
        for (int64_t i = 0; i < m * n; ++i) X[i] = a * X[i] + Y[i];
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t q = 0; q < cols; ++q) out[r * cols + q] = tall ? X[q * n + r] : X[r * n + q];
    free(X); free(Y); free(A); free(AA); free(Bm);
}

/* One Muon update of the matrix p [rows, cols] with gradient g and momentum buffer buf (both updated). */
void orc_muon_update(double* p, const double* g, double* buf, int64_t rows, int64_t cols, double lr, double mu,
                     int nesterov, double wd, int steps, double a, double b, double c, double eps)
{
    const int64_t n = rows * cols;
    double* u = malloc(sizeof(double) * n);
    double* O = malloc(sizeof(double) * n);
    for (int64_t i = 0; i < n; ++i) {
        buf[i] = mu * buf[i] + (1.0 - mu) * g[i];
        u[i] = nesterov ? (1.0 - mu) * g[i] + mu * buf[i] : buf[i];
    }
    orc_newton_schulz(u, rows, cols, steps, a, b, c, eps, O);
    const double scale = lr * sqrt(rows > cols ? (double)rows / (double)cols : 1.0);
    for (int64_t i = 0; i < n; ++i) p[i] = p[i] * (1.0 - lr * wd) - scale * O[i];
    free(u); free(O);
}

/* One AdamW update (step t >= 1) of n parameters with moments m and v (both updated). */
void orc_adamw_update(double* p, const double* g, double* m, double* v, int64_t n, int64_t t, double lr, double b1,
                      double b2, double eps, double wd)
{
    const double bc1 = 1.0 - pow(b1, (double)t), bc2 = 1.0 - pow(b2, (double)t);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = b1 * m[i] + (1.0 - b1) * g[i];
        v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        const double mh = m[i] / bc1, vh = v[i] / bc2;
        p[i] = p[i] * (1.0 - lr * wd) - lr * mh / (sqrt(vh) + eps);
    }
}

/* Optimizer state, fp64 elements: a momentum buffer for every layer matrix (the packed matrix range, in
 * packing order), then the AdamW moments m and v of wte and then of lm_head. */
int64_t orc_optim_state_size(const orc_config* c)
{
    const int64_t VC = (int64_t)c->vocab_size * c->n_embd;
    return orc_num_params(c) - 2 * VC + 4 * VC;
}

/* The whole step over the packed parameters: Muon for each layer matrix, AdamW for wte and lm_head. */
void orc_optim_step(const orc_config* c, double* params, const double* grads, double* state, int64_t t,
                    const orc_optim* o)
{
    const int64_t VC = (int64_t)c->vocab_size * c->n_embd, P = orc_num_params(c);
    const int64_t nmat = P - 2 * VC;
    for (int l = 0; l < c->n_layer; ++l)
        for (int w = 0; w < 6; ++w) {
            int64_t off, r, k;
            orc_param_slice(c, l, w, &off, &r, &k);
            orc_muon_update(params + off, grads + off, state + (off - VC), r, k, o->matrix_lr, o->muon_momentum,
                            o->muon_nesterov, o->weight_decay, o->ns_steps, o->ns_a, o->ns_b, o->ns_c, o->ns_eps);
        }
    int64_t off, r, k;
    orc_param_slice(c, -1, 0, &off, &r, &k);
    orc_adamw_update(params + off, grads + off, state + nmat, state + nmat + VC, VC, t, o->embedding_lr,
                     o->adam_beta1, o->adam_beta2, o->adam_eps, o->weight_decay);
    orc_param_slice(c, -1, 1, &off, &r, &k);
    orc_adamw_update(params + off, grads + off, state + nmat + 2 * VC, state + nmat + 3 * VC, VC, t,
                     o->unembedding_lr, o->adam_beta1, o->adam_beta2, o->adam_eps, o->weight_decay);
}
