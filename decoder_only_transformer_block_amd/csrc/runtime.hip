// Host runtime behind include/ncgpt.h: shape validation, the workspace plan,
// and the launch sequence of one forward / loss / backward on the bound stream.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/ncgpt.h"
#include "kernels.h"

using namespace ncgpt;

namespace {

constexpr int kCUs = 256;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    size_t flag, cosv, sinv, wcast, x0, x, layer0, layer_stride;
    size_t l_xn1, l_rstd1, l_qkv, l_rstdq, l_rstdk, l_y, l_lse, l_xn2, l_rstd2, l_act;
    size_t xf, rstdf, logits, lse, loss_rows, dxn, dx, dx_cd, dh, dy, dqkv, delta, splitk, iscr, total;
};

struct Timed {
    const char* name;
    hipEvent_t a, b;
    double flops, bytes;
};
struct Agg {
    std::string name;
    int64_t launches = 0;
    double ms = 0, flops = 0, bytes = 0;
};

struct WGrad {  // choice for one weight-gradient GEMM
    int tile, splits, k_split;
};

}  // namespace

struct ncgpt_ctx {
    ncgpt_config cfg;
    ncgpt_dtype dtype;
    Dt dt;
    int64_t L, C, H, Hkv, D, F, V, B, T, N, HD, KD, QKV, P, VC;
    size_t esz;
    Plan pl;
    std::vector<float> cos_host, sin_host;
    uint8_t* ws = nullptr;
    size_t ws_bytes = 0;
    hipStream_t stream = nullptr;
    bool bound = false;
    const int32_t* ids = nullptr;
    const float* params = nullptr;
    const int32_t* targets = nullptr;
    int state = 0;  // 0: nothing, 1: forward done, 2: loss done, 3: backward done
    std::string err;
    bool timing = false;
    std::vector<Timed> pending;
    std::vector<hipEvent_t> pool;
    std::vector<Agg> agg;
    bool attrs_done = false;

    template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
    size_t lay(int l, size_t o) const { return pl.layer0 + (size_t)l * pl.layer_stride + o; }
};

namespace {

ncgpt_status fail(ncgpt_ctx* c, ncgpt_status st, const std::string& msg) {
    if (c) c->err = msg;
    return st;
}

ncgpt_status hip_fail(ncgpt_ctx* c, hipError_t e, const char* what) {
    return fail(c, NCGPT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool valid_cfg(const ncgpt_config* g) {
    return g && g->n_layer > 0 && g->n_embd > 0 && g->n_head > 0 && g->n_kv_head > 0 && g->head_dim > 0 &&
           g->mlp_dim > 0 && g->vocab_size > 0 && g->batch > 0 && g->seq_len > 0;
}

int64_t layer_params(const ncgpt_config* g) {
    int64_t C = g->n_embd, HD = (int64_t)g->n_head * g->head_dim, KD = (int64_t)g->n_kv_head * g->head_dim;
    return HD * C + 2 * KD * C + C * HD + 2 * (int64_t)g->mlp_dim * C;
}

// GEMM tile for an output of M x N: the largest tile whose workgroup count
// fills whole rounds of the 256 CUs well (>= 85 %), else the best filling one.
int pick_tile(int64_t M, int64_t N) {
    static const int bm[3] = {256, 256, 128}, bn[3] = {256, 128, 128};
    int best = 2;
    double best_eff = -1;
    for (int t = 0; t < 3; ++t) {
        int64_t tiles = ((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]);
        double eff = (double)tiles / (double)(((tiles + kCUs - 1) / kCUs) * kCUs);
        if (tiles >= kCUs && eff >= 0.85) return t;
        if (eff > best_eff + 1e-9) { best_eff = eff; best = t; }
    }
    return best;
}

// Weight gradient dW[M,N] = sum over K tokens.  The output alone has few
// tiles (e.g. 9 for 768 x 768) while K is the whole batch of tokens, so K is
// split until one round of workgroups covers the CUs; large outputs use the
// forward tile rule.
WGrad pick_wgrad(Dt dt, int64_t M, int64_t N, int64_t K) {
    WGrad w;
    if (dt == Dt::F32) {
        w.tile = 0;
        int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
        int64_t s = std::max<int64_t>(1, (4 * kCUs) / tiles);
        s = std::min<int64_t>(s, K / 256);
        w.splits = (int)std::max<int64_t>(1, s);
    } else {
        static const int bm[3] = {256, 256, 128}, bn[3] = {256, 128, 128};
        const int64_t tiles0 = ((M + 255) / 256) * ((N + 255) / 256);
        if (tiles0 < kCUs) {
            w.tile = (M >= 256 && N >= 256) ? 0 : 2;
        } else {
            w.tile = pick_tile(M, N);
        }
        int64_t tiles = ((M + bm[w.tile] - 1) / bm[w.tile]) * ((N + bn[w.tile] - 1) / bn[w.tile]);
        int64_t s = tiles >= kCUs ? 1 : kCUs / tiles;
        s = std::min<int64_t>(s, K / 512);
        w.splits = (int)std::max<int64_t>(1, s);
    }
    int64_t kb = K / 64;
    int64_t per = (kb + w.splits - 1) / w.splits;
    w.k_split = (int)(per * 64);
    w.splits = (int)((K + w.k_split - 1) / w.k_split);
    return w;
}

void make_plan(ncgpt_ctx* c) {
    Plan& p = c->pl;
    size_t off = 0;
    auto A = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t e = c->esz, N = c->N;
    p.flag = A(256);
    p.cosv = A((size_t)c->T * (c->D / 2) * 4);
    p.sinv = A((size_t)c->T * (c->D / 2) * 4);
    p.wcast = A(c->dt == Dt::BF16 ? (size_t)(c->P - c->VC) * 2 : 0);
    p.x0 = A(N * c->C * e);
    p.x = A(N * c->C * e);
    // one layer's saved activations
    size_t lo = 0;
    auto LA = [&](size_t bytes) { size_t o = lo; lo += align256(bytes); return o; };
    p.l_xn1 = LA(N * c->C * e);
    p.l_rstd1 = LA(N * 4);
    p.l_qkv = LA(N * c->QKV * e);
    p.l_rstdq = LA(N * c->H * 4);
    p.l_rstdk = LA(N * c->Hkv * 4);
    p.l_y = LA(N * c->HD * e);
    p.l_lse = LA((size_t)c->B * c->H * c->T * 4);
    p.l_xn2 = LA(N * c->C * e);
    p.l_rstd2 = LA(N * 4);
    p.l_act = LA(N * c->F * e);
    p.layer_stride = lo;
    p.layer0 = A(lo * c->L);
    p.xf = A(N * c->C * e);
    p.rstdf = A(N * 4);
    p.logits = A(N * c->V * e);
    p.lse = A(N * 4);
    p.loss_rows = A(N * 4);
    p.dxn = A(N * c->C * 4);
    p.dx = A(N * c->C * 4);
    p.dx_cd = A(c->dt == Dt::BF16 ? N * c->C * 2 : 0);
    p.dh = A(N * c->F * e);
    p.dy = A(N * c->HD * e);
    p.dqkv = A(N * c->QKV * e);
    p.delta = A((size_t)2 * c->B * c->H * c->T * 4);
    // split-K partials: the largest splits * M * N over the weight gradients
    size_t sk = 0;
    const int64_t shapes[5][2] = {{c->QKV, c->C}, {c->C, c->HD}, {c->F, c->C}, {c->C, c->F}, {c->V, c->C}};
    for (auto& s : shapes) {
        WGrad w = pick_wgrad(c->dt, s[0], s[1], (int64_t)N);
        if (w.splits > 1) sk = std::max(sk, (size_t)w.splits * s[0] * s[1] * 4);
    }
    p.splitk = A(sk);
    p.iscr = A(embed_bwd_scratch_ints((int)N, (int)c->V) * 4);
    p.total = off;
}

// ---------------------------------------------------------------- launch wrapper with optional timing
template <class F>
ncgpt_status launch(ncgpt_ctx* c, const char* name, double flops, double bytes, F&& fn) {
    hipEvent_t a = nullptr, b = nullptr;
    if (c->timing) {
        for (hipEvent_t* ev : {&a, &b}) {
            if (!c->pool.empty()) {
                *ev = c->pool.back();
                c->pool.pop_back();
            } else if (hipEventCreate(ev) != hipSuccess) {
                return fail(c, NCGPT_EHIP, "hipEventCreate failed");
            }
        }
        (void)hipEventRecord(a, c->stream);
    }
    hipError_t e = fn();
    if (e != hipSuccess) return hip_fail(c, e, name);
    if (c->timing) {
        (void)hipEventRecord(b, c->stream);
        c->pending.push_back({name, a, b, flops, bytes});
    }
    return NCGPT_OK;
}

#define TRY(x)                                   \
    do {                                         \
        ncgpt_status _s = (x);                   \
        if (_s != NCGPT_OK) return _s;           \
    } while (0)

ncgpt_status fold_timing(ncgpt_ctx* c) {
    if (c->pending.empty()) return NCGPT_OK;
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
    for (auto& t : c->pending) {
        float ms = 0;
        (void)hipEventElapsedTime(&ms, t.a, t.b);
        auto it = std::find_if(c->agg.begin(), c->agg.end(), [&](const Agg& g) { return g.name == t.name; });
        if (it == c->agg.end()) {
            c->agg.push_back(Agg{t.name});
            it = c->agg.end() - 1;
        }
        it->launches += 1;
        it->ms += ms;
        it->flops += t.flops;
        it->bytes += t.bytes;
        c->pool.push_back(t.a);
        c->pool.push_back(t.b);
    }
    c->pending.clear();
    return NCGPT_OK;
}

const char* epi_name(Epi e) {
    switch (e) {
    case Epi::StoreCd: return "store";
    case Epi::StoreF32: return "store_f32";
    case Epi::ResidualCd: return "residual";
    case Epi::ReluSq: return "relusq";
    case Epi::ReluSqBwd: return "relusq_bwd";
    case Epi::Grad: return "grad";
    case Epi::SplitK: return "splitk";
    }
    return "?";
}

// Names must outlive the pending list: intern them.
const char* intern(const std::string& s) {
    static std::vector<std::string*> names;
    for (auto* p : names)
        if (*p == s) return p->c_str();
    names.push_back(new std::string(s));
    return names.back()->c_str();
}

// tag: the call site (qkv, lm_head, dWfc, ...), so every timing row is one shape
ncgpt_status gemm(ncgpt_ctx* c, GemmDesc d, const char* tag) {
    d.dt = c->dt;
    if (d.tile < 0) d.tile = pick_tile(d.M, d.N);
    const char* nm = intern(std::string(gemm_kernel_name(d)) + ":" + epi_name(d.epi) + ":" + tag);
    const double fl = 2.0 * d.M * d.N * d.K;
    // algorithmic bytes: both operands once, the output (and what the epilogue reads) once
    const double e = d.dt == Dt::BF16 ? 2.0 : 4.0, mn = (double)d.M * d.N;
    double out = e;
    switch (d.epi) {
    case Epi::StoreF32: out = 4.0; break;
    case Epi::ResidualCd: case Epi::ReluSqBwd: out = 2.0 * e; break;
    case Epi::Grad: out = d.accumulate ? 8.0 : 4.0; break;
    case Epi::SplitK: out = 4.0 * std::max(1, d.splits); break;
    default: break;
    }
    const double by = ((double)d.M * d.K + (double)d.N * d.K) * e + mn * out;
    return launch(c, nm, fl, by, [&] { return launch_gemm(d, c->stream); });
}

// weight gradient: out(f32 grads slice [M,N]) (+)= A^T-layout x B^T-layout over K tokens
ncgpt_status wgrad(ncgpt_ctx* c, const char* tag, const void* dY, int ldy, const void* X, int ldx, int M, int N,
                   float* g, int accumulate, int tile = -1, int variant = -1) {
    const int K = (int)c->N;
    WGrad w = pick_wgrad(c->dt, M, N, K);
    if (tile >= 0 && w.splits == 1) w.tile = tile;
    GemmDesc d;
    // both operands are read through transposing LDS reads (half rate): the four-wave persistent
    // ring, which reads fewer fragments per MFMA, measured fastest
    d.variant = variant >= 0 ? variant : 8;
    d.A = dY; d.lda = ldy; d.a_kcontig = false;
    d.B = X; d.ldb = ldx; d.b_kcontig = false;
    d.M = M; d.N = N; d.K = K;
    d.tile = w.tile;
    d.ldo = N;
    if (w.splits == 1) {
        d.epi = Epi::Grad;
        d.out = g;
        d.accumulate = accumulate;
        return gemm(c, d, tag);
    }
    d.epi = Epi::SplitK;
    d.splits = w.splits;
    d.k_split = w.k_split;
    d.out = c->at<float>(c->pl.splitk);
    d.split_stride = (size_t)M * N;
    TRY(gemm(c, d, tag));
    const size_t n = (size_t)M * N;
    return launch(c, intern(std::string("splitk_reduce:") + tag), 0.0, (double)n * 4 * (w.splits + 1 + accumulate), [&] {
        return launch_splitk_reduce(c->at<float>(c->pl.splitk), w.splits, (size_t)M * N, g, n, accumulate, c->stream);
    });
}

const void* weight(ncgpt_ctx* c, int layer, int which) {
    size_t off;
    int64_t r, cc;
    ncgpt_param_slice(&c->cfg, layer, which, &off, &r, &cc);
    if (c->dt == Dt::BF16) return c->at<uint8_t>(c->pl.wcast) + (off - c->VC) * 2;
    return c->params + off;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

size_t ncgpt_num_params(const ncgpt_config* g) {
    if (!valid_cfg(g)) return 0;
    int64_t VC = (int64_t)g->vocab_size * g->n_embd;
    return (size_t)(2 * VC + (int64_t)g->n_layer * layer_params(g));
}

ncgpt_status ncgpt_param_slice(const ncgpt_config* g, int layer, int which, size_t* offset, int64_t* rows,
                               int64_t* cols) {
    if (!valid_cfg(g) || !offset || !rows || !cols) return NCGPT_EINVAL;
    int64_t C = g->n_embd, V = g->vocab_size, F = g->mlp_dim;
    int64_t HD = (int64_t)g->n_head * g->head_dim, KD = (int64_t)g->n_kv_head * g->head_dim;
    if (layer == -1) {
        if (which == 0) { *offset = 0; *rows = V; *cols = C; return NCGPT_OK; }
        if (which == 1) {
            *offset = (size_t)(V * C + (int64_t)g->n_layer * layer_params(g));
            *rows = V; *cols = C;
            return NCGPT_OK;
        }
        return NCGPT_EINVAL;
    }
    if (layer < 0 || layer >= g->n_layer || which < 0 || which > 5) return NCGPT_EINVAL;
    const int64_t r[6] = {HD, KD, KD, C, F, C}, k[6] = {C, C, C, HD, C, F};
    int64_t off = V * C + (int64_t)layer * layer_params(g);
    for (int i = 0; i < which; ++i) off += r[i] * k[i];
    *offset = (size_t)off;
    *rows = r[which];
    *cols = k[which];
    return NCGPT_OK;
}

ncgpt_status ncgpt_create(const ncgpt_config* g, ncgpt_dtype dtype, ncgpt_ctx** out) {
    if (!out) return NCGPT_EINVAL;
    *out = nullptr;
    if (!valid_cfg(g) || (dtype != NCGPT_F32 && dtype != NCGPT_BF16)) return NCGPT_EINVAL;
    const bool bf = dtype == NCGPT_BF16;
    if (g->n_head % g->n_kv_head) return NCGPT_EUNSUPPORTED;
    if (bf ? g->head_dim != 128 : (g->head_dim != 64 && g->head_dim != 128)) return NCGPT_EUNSUPPORTED;
    if (g->n_embd % 64 || g->mlp_dim % 64 || g->vocab_size % 64) return NCGPT_EUNSUPPORTED;
    if (g->vocab_size > 65536) return NCGPT_EUNSUPPORTED;  // the embedding-gradient counting sort
    if (bf ? g->seq_len % 128 : g->seq_len % 64) return NCGPT_EUNSUPPORTED;
    if ((double)g->batch * g->seq_len * g->vocab_size > 4.0e12) return NCGPT_EUNSUPPORTED;
    if (!(g->norm_eps >= 0.0f) || !(g->rope_base > 0.0f)) return NCGPT_EINVAL;
    ncgpt_ctx* c = new (std::nothrow) ncgpt_ctx();
    if (!c) return NCGPT_ENOMEM;
    c->cfg = *g;
    c->dtype = dtype;
    c->dt = bf ? Dt::BF16 : Dt::F32;
    c->L = g->n_layer; c->C = g->n_embd; c->H = g->n_head; c->Hkv = g->n_kv_head; c->D = g->head_dim;
    c->F = g->mlp_dim; c->V = g->vocab_size; c->B = g->batch; c->T = g->seq_len;
    c->N = c->B * c->T; c->HD = c->H * c->D; c->KD = c->Hkv * c->D; c->QKV = c->HD + 2 * c->KD;
    c->P = (int64_t)ncgpt_num_params(g);
    c->VC = c->V * c->C;
    c->esz = bf ? 2 : 4;
    make_plan(c);
    // RoPE tables: angle t * base^(-2i/D), evaluated in double, stored fp32
    const int half = (int)(c->D / 2);
    c->cos_host.resize((size_t)c->T * half);
    c->sin_host.resize((size_t)c->T * half);
    for (int64_t t = 0; t < c->T; ++t)
        for (int i = 0; i < half; ++i) {
            double ang = (double)t * std::pow((double)g->rope_base, -2.0 * i / (double)c->D);
            c->cos_host[(size_t)t * half + i] = (float)std::cos(ang);
            c->sin_host[(size_t)t * half + i] = (float)std::sin(ang);
        }
    *out = c;
    return NCGPT_OK;
}

ncgpt_status ncgpt_workspace_size(const ncgpt_ctx* c, size_t* bytes) {
    if (!c || !bytes) return NCGPT_EINVAL;
    *bytes = c->pl.total;
    return NCGPT_OK;
}

ncgpt_status ncgpt_bind(ncgpt_ctx* c, void* workspace, size_t bytes, void* stream) {
    if (!c) return NCGPT_EINVAL;
    if (!workspace) return fail(c, NCGPT_EINVAL, "null workspace");
    if (bytes < c->pl.total) return fail(c, NCGPT_ENOMEM, "workspace smaller than ncgpt_workspace_size");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(c, NCGPT_EINVAL, "workspace not 256-byte aligned");
    if (!c->attrs_done) {
        hipError_t e = attn_init_attributes();
        if (e != hipSuccess) return hip_fail(c, e, "attention kernel attributes");
        e = gemm_init_attributes();
        if (e != hipSuccess) return hip_fail(c, e, "gemm kernel attributes");
        c->attrs_done = true;
    }
    c->ws = static_cast<uint8_t*>(workspace);
    c->ws_bytes = bytes;
    c->stream = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(c->ws + c->pl.cosv, c->cos_host.data(), c->cos_host.size() * 4,
                                  hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->ws + c->pl.sinv, c->sin_host.data(), c->sin_host.size() * 4, hipMemcpyHostToDevice,
                           c->stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->ws + c->pl.flag, 0, 256, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "bind uploads");
    c->bound = true;
    c->state = 0;
    return NCGPT_OK;
}

ncgpt_status ncgpt_forward(ncgpt_ctx* c, const int32_t* ids, const float* params) {
    if (!c) return NCGPT_EINVAL;
    if (!c->bound) return fail(c, NCGPT_ESTATE, "ncgpt_bind has not been called");
    if (!ids || !params) return fail(c, NCGPT_EINVAL, "null ids or params");
    c->ids = ids;
    c->params = params;
    c->state = 0;
    const Plan& p = c->pl;
    const Dt dt = c->dt;
    const int N = (int)c->N, C = (int)c->C, F = (int)c->F, QKV = (int)c->QKV, HD = (int)c->HD, V = (int)c->V;
    const float eps = c->cfg.norm_eps;
    const size_t e = c->esz;
    uint32_t* flag = c->at<uint32_t>(p.flag);

    if (dt == Dt::BF16) {
        const size_t n = (size_t)(c->P - c->VC);
        TRY(launch(c, "cast_bf16", 0.0, (double)n * 6,
                   [&] { return launch_cast_bf16(params + c->VC, c->ws + p.wcast, n, c->stream); }));
    }
    TRY(launch(c, "embed_fwd", 0.0, (double)N * C * (4 + e) + N * 4.0, [&] {
        return launch_embed_fwd(dt, ids, params, c->ws + p.x0, N, C, V, flag, c->stream);
    }));
    const double norm_bytes = (double)N * C * 2 * e + N * 4.0;
    for (int l = 0; l < c->L; ++l) {
        uint8_t* xin = c->ws + (l == 0 ? p.x0 : p.x);
        uint8_t* xn1 = c->ws + c->lay(l, p.l_xn1);
        uint8_t* qkv = c->ws + c->lay(l, p.l_qkv);
        uint8_t* y = c->ws + c->lay(l, p.l_y);
        uint8_t* xn2 = c->ws + c->lay(l, p.l_xn2);
        uint8_t* act = c->ws + c->lay(l, p.l_act);
        TRY(launch(c, "rmsnorm_fwd", 0.0, norm_bytes, [&] {
            return launch_rmsnorm_fwd(dt, xin, xn1, c->at<float>(c->lay(l, p.l_rstd1)), N, C, eps, c->stream);
        }));
        {
            GemmDesc d;
            d.A = xn1; d.lda = C; d.B = weight(c, l, 0); d.ldb = C;
            d.M = N; d.N = QKV; d.K = C;
            d.epi = Epi::StoreCd; d.out = qkv; d.ldo = QKV;
            d.variant = 9;  // the persistent eight-wave ring measured fastest for this shape
            d.group_m = 8;  // bands of 8 tile-rows measured faster than bands of 4 for this shape
            TRY(gemm(c, d, "qkv"));
        }
        TRY(launch(c, "rope_qknorm_fwd", 0.0, (double)N * (c->H + c->Hkv) * c->D * 2 * e, [&] {
            return launch_rope_qknorm_fwd(dt, qkv, c->at<float>(c->lay(l, p.l_rstdq)), c->at<float>(c->lay(l, p.l_rstdk)),
                                          c->at<float>(p.cosv), c->at<float>(p.sinv), N, (int)c->T, (int)c->H,
                                          (int)c->Hkv, (int)c->D, eps, c->stream);
        }));
        {
            AttnDesc ad;
            ad.dt = dt; ad.B = (int)c->B; ad.T = (int)c->T; ad.H = (int)c->H; ad.Hkv = (int)c->Hkv; ad.D = (int)c->D;
            ad.qkv = qkv; ad.y = y; ad.lse = c->at<float>(c->lay(l, p.l_lse));
            const double pairs = (double)c->B * c->H * c->T * (c->T + 1) / 2.0;
            // algorithmic bytes: read q, k, v; write y and the row log-sum-exp
            const double qb = (double)N * c->H * c->D * e, kb = (double)N * c->Hkv * c->D * e;
            TRY(launch(c, dt == Dt::BF16 ? "attn_fwd_bf16" : "attn_fwd_f32", 4.0 * c->D * pairs,
                       2 * qb + 2 * kb + (double)N * c->H * 4, [&] { return launch_attn_fwd(ad, c->stream); }));
        }
        {
            GemmDesc d;
            d.A = y; d.lda = HD; d.B = weight(c, l, 3); d.ldb = HD;
            d.M = N; d.N = C; d.K = HD;
            d.epi = Epi::ResidualCd; d.out = c->ws + p.x; d.in = xin; d.ldo = C;
            d.variant = 7;  // epilogue reads the residual: the eight-wave ring without spills
            d.group_m = 8;
            TRY(gemm(c, d, "attn_out"));
        }
        TRY(launch(c, "rmsnorm_fwd", 0.0, norm_bytes, [&] {
            return launch_rmsnorm_fwd(dt, c->ws + p.x, xn2, c->at<float>(c->lay(l, p.l_rstd2)), N, C, eps, c->stream);
        }));
        {
            GemmDesc d;
            d.A = xn2; d.lda = C; d.B = weight(c, l, 4); d.ldb = C;
            d.M = N; d.N = F; d.K = C;
            d.epi = Epi::ReluSq; d.out = act; d.ldo = F;
            d.variant = 7;  // the non-persistent eight-wave ring measured fastest for this shape
            TRY(gemm(c, d, "fc"));
        }
        {
            GemmDesc d;
            d.A = act; d.lda = F; d.B = weight(c, l, 5); d.ldb = F;
            d.M = N; d.N = C; d.K = F;
            d.epi = Epi::ResidualCd; d.out = c->ws + p.x; d.in = c->ws + p.x; d.ldo = C;
            d.variant = 9;  // measured faster than the non-persistent ring despite a small spill
            TRY(gemm(c, d, "proj"));
        }
    }
    TRY(launch(c, "rmsnorm_fwd", 0.0, norm_bytes, [&] {
        return launch_rmsnorm_fwd(dt, c->ws + p.x, c->ws + p.xf, c->at<float>(p.rstdf), N, C, eps, c->stream);
    }));
    {
        GemmDesc d;
        d.A = c->ws + p.xf; d.lda = C; d.B = weight(c, -1, 1); d.ldb = C;
        d.M = N; d.N = V; d.K = C;
        d.epi = Epi::StoreCd; d.out = c->ws + p.logits; d.ldo = V;
        d.group_m = 8;
        TRY(gemm(c, d, "lm_head"));
    }
    c->state = 1;
    return NCGPT_OK;
}

ncgpt_status ncgpt_loss(ncgpt_ctx* c, const int32_t* targets, float* loss) {
    if (!c) return NCGPT_EINVAL;
    if (c->state < 1) return fail(c, NCGPT_ESTATE, "ncgpt_loss before ncgpt_forward");
    if (!targets || !loss) return fail(c, NCGPT_EINVAL, "null targets or loss");
    const Plan& p = c->pl;
    const int N = (int)c->N, V = (int)c->V;
    uint32_t* flag = c->at<uint32_t>(p.flag);
    c->targets = targets;
    TRY(launch(c, "ce_fwd_rows", 0.0, (double)N * V * c->esz + N * 12.0, [&] {
        return launch_ce_fwd_rows(c->dt, c->ws + p.logits, targets, c->at<float>(p.lse), c->at<float>(p.loss_rows), N,
                                  V, flag, c->stream);
    }));
    TRY(launch(c, "loss_reduce", 0.0, N * 8.0, [&] {
        return launch_loss_reduce(c->at<float>(p.loss_rows), targets, N, V, loss, c->at<float>(p.flag + 4), flag,
                                  c->stream);
    }));
    c->state = 2;
    return NCGPT_OK;
}

ncgpt_status ncgpt_backward(ncgpt_ctx* c, float* grads, int accumulate, float grad_scale) {
    if (!c) return NCGPT_EINVAL;
    if (c->state != 2) return fail(c, NCGPT_ESTATE, "ncgpt_backward needs ncgpt_loss after the last ncgpt_forward");
    if (!grads) return fail(c, NCGPT_EINVAL, "null grads");
    const Plan& p = c->pl;
    const Dt dt = c->dt;
    const int N = (int)c->N, C = (int)c->C, F = (int)c->F, QKV = (int)c->QKV, HD = (int)c->HD, V = (int)c->V;
    const size_t e = c->esz;
    const int acc = accumulate ? 1 : 0;
    uint8_t* logits = c->ws + p.logits;
    float* dxn = c->at<float>(p.dxn);
    float* dx = c->at<float>(p.dx);
    uint8_t* dxg = dt == Dt::BF16 ? c->ws + p.dx_cd : c->ws + p.dx;  // GEMM operand copy of dx
    void* dx_cd = dt == Dt::BF16 ? (void*)(c->ws + p.dx_cd) : nullptr;

    auto gslice = [&](int layer, int which) {
        size_t off;
        int64_t r, cc;
        ncgpt_param_slice(&c->cfg, layer, which, &off, &r, &cc);
        return grads + off;
    };

    // cross-entropy -> dz (in place over the logits)
    TRY(launch(c, "ce_bwd", 0.0, (double)N * V * 2 * e, [&] {
        return launch_ce_bwd(dt, logits, c->at<float>(p.lse), c->targets, c->at<float>(p.flag + 4), grad_scale, N, V,
                             c->stream);
    }));
    {   // dxf = dz Wlm
        GemmDesc d;
        d.A = logits; d.lda = V; d.B = weight(c, -1, 1); d.ldb = C; d.b_kcontig = false;
        d.M = N; d.N = C; d.K = V;
        d.epi = Epi::StoreCd; d.out = dxn; d.ldo = C;  // compute dtype
        d.variant = 7;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
        TRY(gemm(c, d, "dxf"));
    }
    // dWlm = dz^T xf: vocab x n_embd output over all tokens; 256 x 128 tiles, the four-wave persistent ring
    // measured fastest
    TRY(wgrad(c, "dWlm", logits, V, c->ws + p.xf, C, V, C, gslice(-1, 1), acc, 1, 8));
    const double nb = (double)N * C * (e + e + 4 + (dt == Dt::BF16 ? 2 : 0)) + N * 4.0;
    TRY(launch(c, "rmsnorm_bwd", 0.0, nb, [&] {
        return launch_rmsnorm_bwd(dt, c->ws + p.xf, c->at<float>(p.rstdf), dxn, dx, dx_cd, N, C, 0, c->stream);
    }));
    for (int l = (int)c->L - 1; l >= 0; --l) {
        uint8_t* xn1 = c->ws + c->lay(l, p.l_xn1);
        uint8_t* qkv = c->ws + c->lay(l, p.l_qkv);
        uint8_t* y = c->ws + c->lay(l, p.l_y);
        uint8_t* xn2 = c->ws + c->lay(l, p.l_xn2);
        uint8_t* act = c->ws + c->lay(l, p.l_act);
        {   // dh = (dx Wproj) * 2 relu(h), relu(h) = sqrt(act)
            GemmDesc d;
            d.A = dxg; d.lda = C; d.B = weight(c, l, 5); d.ldb = F; d.b_kcontig = false;
            d.M = N; d.N = F; d.K = C;
            d.epi = Epi::ReluSqBwd; d.out = c->ws + p.dh; d.in = act; d.ldo = F;
            d.variant = 7;  // epilogue reads act: the eight-wave ring without spills
            TRY(gemm(c, d, "dh"));
        }
        TRY(wgrad(c, "dWproj", dxg, C, act, F, C, F, gslice(l, 5), acc));  // dWproj = dx^T act
        {   // dxn2 = dh Wfc
            GemmDesc d;
            d.A = c->ws + p.dh; d.lda = F; d.B = weight(c, l, 4); d.ldb = C; d.b_kcontig = false;
            d.M = N; d.N = C; d.K = F;
            d.epi = Epi::StoreCd; d.out = dxn; d.ldo = C;  // compute dtype
            d.variant = 7;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
            TRY(gemm(c, d, "dxn2"));
        }
        TRY(wgrad(c, "dWfc", c->ws + p.dh, F, xn2, C, F, C, gslice(l, 4), acc));  // dWfc = dh^T xn2
        TRY(launch(c, "rmsnorm_bwd", 0.0, nb + (double)N * C * 4, [&] {
            return launch_rmsnorm_bwd(dt, xn2, c->at<float>(c->lay(l, p.l_rstd2)), dxn, dx, dx_cd, N, C, 1, c->stream);
        }));
        {   // dy = dx Wo
            GemmDesc d;
            d.A = dxg; d.lda = C; d.B = weight(c, l, 3); d.ldb = HD; d.b_kcontig = false;
            d.M = N; d.N = HD; d.K = C;
            d.epi = Epi::StoreCd; d.out = c->ws + p.dy; d.ldo = HD;
            TRY(gemm(c, d, "dy"));
        }
        TRY(wgrad(c, "dWo", dxg, C, y, HD, C, HD, gslice(l, 3), acc));  // dWo = dx^T y
        {
            AttnDesc ad;
            ad.dt = dt; ad.B = (int)c->B; ad.T = (int)c->T; ad.H = (int)c->H; ad.Hkv = (int)c->Hkv; ad.D = (int)c->D;
            ad.qkv = qkv; ad.y = y; ad.lse = c->at<float>(c->lay(l, p.l_lse));
            ad.dy = c->ws + p.dy; ad.dqkv = c->ws + p.dqkv; ad.delta = c->at<float>(p.delta);
            ad.rstdq = c->at<float>(c->lay(l, p.l_rstdq)); ad.rstdk = c->at<float>(c->lay(l, p.l_rstdk));
            ad.cosv = c->at<float>(p.cosv); ad.sinv = c->at<float>(p.sinv);
            const double pairs = (double)c->B * c->H * c->T * (c->T + 1) / 2.0;
            const bool bf = dt == Dt::BF16;
            // algorithmic backward FLOPs: dV, dK and the dP product (6 D per pair) in the key-outer kernel,
            // dQ (2 D per pair) in the query-outer one; the recomputed S and dP products are not counted
            // algorithmic bytes: dQ reads q, k, v, y, dy and lse, writes dq and delta; dK/dV reads q, k, v,
            // dy, lse and delta, writes dk and dv
            const double qb = (double)N * c->H * c->D * e, kb = (double)N * c->Hkv * c->D * e;
            const double rows = (double)N * c->H * 4;
            TRY(launch(c, bf ? "attn_bwd_dq_bf16" : "attn_bwd_dq_f32", 2.0 * c->D * pairs, 4 * qb + 2 * kb + 2 * rows,
                       [&] { return launch_attn_bwd(ad, c->stream, 0); }));
            TRY(launch(c, bf ? "attn_bwd_dkdv_bf16" : "attn_bwd_dkdv_f32", 6.0 * c->D * pairs,
                       2 * qb + 4 * kb + 2 * rows, [&] { return launch_attn_bwd(ad, c->stream, 1); }));
        }
        if (dt != Dt::BF16) {  // the bf16 attention backward applies it in its epilogues
            TRY(launch(c, "rope_qknorm_bwd", 0.0, (double)N * (c->H + c->Hkv) * c->D * 3 * e, [&] {
                return launch_rope_qknorm_bwd(dt, c->ws + p.dqkv, qkv, c->at<float>(c->lay(l, p.l_rstdq)),
                                              c->at<float>(c->lay(l, p.l_rstdk)), c->at<float>(p.cosv),
                                              c->at<float>(p.sinv), N, (int)c->T, (int)c->H, (int)c->Hkv, (int)c->D,
                                              c->stream);
            }));
        }
        {   // dxn1 = dqkv Wqkv
            GemmDesc d;
            d.A = c->ws + p.dqkv; d.lda = QKV; d.B = weight(c, l, 0); d.ldb = C; d.b_kcontig = false;
            d.M = N; d.N = C; d.K = QKV;
            d.epi = Epi::StoreCd; d.out = dxn; d.ldo = C;  // compute dtype
            d.variant = 7;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
            TRY(gemm(c, d, "dxn1"));
        }
        TRY(wgrad(c, "dWqkv", c->ws + p.dqkv, QKV, xn1, C, QKV, C, gslice(l, 0), acc));  // dWqkv = dqkv^T xn1
        TRY(launch(c, "rmsnorm_bwd", 0.0, nb + (double)N * C * 4, [&] {
            return launch_rmsnorm_bwd(dt, xn1, c->at<float>(c->lay(l, p.l_rstd1)), dxn, dx, dx_cd, N, C, 1, c->stream);
        }));
    }
    TRY(launch(c, "embed_bwd", 0.0, (double)N * C * 8 + (double)V * C * (4 + 4 * acc), [&] {
        return launch_embed_bwd(c->ids, dx, gslice(-1, 0), N, C, V, acc, c->at<int32_t>(p.iscr), dxn, c->stream);
    }));
    c->state = 3;
    return NCGPT_OK;
}

ncgpt_status ncgpt_check(ncgpt_ctx* c) {
    if (!c) return NCGPT_EINVAL;
    if (!c->bound) return fail(c, NCGPT_ESTATE, "ncgpt_bind has not been called");
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
    uint32_t flag = 0;
    e = hipMemcpy(&flag, c->ws + c->pl.flag, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(c, e, "reading the device error flag");
    if (flag) {
        (void)hipMemset(c->ws + c->pl.flag, 0, 4);
        std::string m = "device error:";
        if (flag & kErrBadToken) m += " token id outside [0, vocab);";
        if (flag & kErrBadTarget) m += " target >= vocab;";
        if (flag & kErrNoTargets) m += " no valid target;";
        return fail(c, NCGPT_EDEVICE, m);
    }
    return NCGPT_OK;
}

ncgpt_status ncgpt_probe_numel(const ncgpt_ctx* c, int what, size_t* numel) {
    if (!c || !numel) return NCGPT_EINVAL;
    const size_t N = (size_t)c->N;
    switch (what) {
    case 0: case 1: case 5: case 7: case 10: *numel = N * c->C; return NCGPT_OK;
    case 2: *numel = N * c->QKV; return NCGPT_OK;
    case 3: *numel = N * c->HD; return NCGPT_OK;
    case 4: *numel = (size_t)c->B * c->H * c->T; return NCGPT_OK;
    case 6: *numel = N * c->F; return NCGPT_OK;
    case 8: case 9: *numel = N; return NCGPT_OK;
    }
    return NCGPT_EINVAL;
}

ncgpt_status ncgpt_probe(ncgpt_ctx* c, int what, int layer, float* dst) {
    if (!c || !dst) return NCGPT_EINVAL;
    size_t n;
    if (ncgpt_probe_numel(c, what, &n) != NCGPT_OK) return fail(c, NCGPT_EINVAL, "unknown probe");
    const bool per_layer = what >= 1 && what <= 6;
    if (per_layer && (layer < 0 || layer >= c->L)) return fail(c, NCGPT_EINVAL, "probe layer out of range");
    if (what == 10 ? c->state < 3 : (what == 8 || what == 9 ? c->state < 2 : c->state < 1))
        return fail(c, NCGPT_ESTATE, "probe before the call that produces it");
    const Plan& p = c->pl;
    const uint8_t* src = nullptr;
    Dt dt = c->dt;
    switch (what) {
    case 0: src = c->ws + p.x0; break;
    case 1: src = c->ws + c->lay(layer, p.l_xn1); break;
    case 2: src = c->ws + c->lay(layer, p.l_qkv); break;
    case 3: src = c->ws + c->lay(layer, p.l_y); break;
    case 4: src = c->ws + c->lay(layer, p.l_lse); dt = Dt::F32; break;
    case 5: src = c->ws + c->lay(layer, p.l_xn2); break;
    case 6: src = c->ws + c->lay(layer, p.l_act); break;
    case 7: src = c->ws + p.xf; break;
    case 8: src = c->ws + p.lse; dt = Dt::F32; break;
    case 9: src = c->ws + p.loss_rows; dt = Dt::F32; break;
    case 10: src = c->ws + p.dx; dt = Dt::F32; break;
    }
    hipError_t e = launch_to_f32(dt, src, dst, n, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "probe");
    return NCGPT_OK;
}

ncgpt_status ncgpt_timing_enable(ncgpt_ctx* c, int enable) {
    if (!c) return NCGPT_EINVAL;
    c->timing = enable != 0;
    return NCGPT_OK;
}

ncgpt_status ncgpt_timing_reset(ncgpt_ctx* c) {
    if (!c) return NCGPT_EINVAL;
    TRY(fold_timing(c));
    c->agg.clear();
    return NCGPT_OK;
}

ncgpt_status ncgpt_timing_count(ncgpt_ctx* c, int* count) {
    if (!c || !count) return NCGPT_EINVAL;
    TRY(fold_timing(c));
    *count = (int)c->agg.size();
    return NCGPT_OK;
}

ncgpt_status ncgpt_timing_get(ncgpt_ctx* c, int index, char* name, size_t name_len, int64_t* launches,
                              double* total_ms, double* flops, double* bytes) {
    if (!c || !name || name_len == 0 || !launches || !total_ms || !flops || !bytes) return NCGPT_EINVAL;
    TRY(fold_timing(c));
    if (index < 0 || index >= (int)c->agg.size()) return NCGPT_EINVAL;
    const Agg& g = c->agg[index];
    std::snprintf(name, name_len, "%s", g.name.c_str());
    *launches = g.launches;
    *total_ms = g.ms;
    *flops = g.flops;
    *bytes = g.bytes;
    return NCGPT_OK;
}

const char* ncgpt_last_error(const ncgpt_ctx* c) { return c ? c->err.c_str() : "null context"; }

void ncgpt_destroy(ncgpt_ctx* c) {
    if (!c) return;
    for (auto& t : c->pending) {
        (void)hipEventDestroy(t.a);
        (void)hipEventDestroy(t.b);
    }
    for (auto ev : c->pool) (void)hipEventDestroy(ev);
    delete c;
}

}  // extern "C"
