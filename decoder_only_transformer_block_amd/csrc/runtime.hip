// Host runtime behind include/ncgpt.h: shape validation, the workspace plan,
// and the launch sequence of one forward / loss / backward on the bound stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/ncgpt.h"
#include "kernels.h"

using namespace ncgpt;

namespace {

constexpr int kCUs = 256;
// dWlm = dz^T xf reads the [tokens, vocab] dz once per column tile of its n_embd-wide output: 256 x 256 tiles
// (split-K where the tile rounds come out uneven) measured faster than 256 x 128 ones, which read dz twice as
// often (d12: 2.52 against 3.15 ms per step)
constexpr int kDWlmTile = 0;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    size_t flag, cosv, sinv, wcast, w8, w8s, a8, a8s, x0, rstd0, x, layer0, layer_stride;
    size_t l_xn1, l_rstd1, l_qkv, l_rstdq, l_rstdk, l_y, l_lse, l_xn2, l_rstd2, l_act;
    size_t xf, rstdf, logits, cepart, zt, lse, loss_rows, dxn, dx, dx_cd, dh, dy, dqkv, delta, splitk, iscr, total;
    int ce_nblk;
    // optimizer step scratch (overlays the saved activations from layer0 on)
    size_t o_part, o_inv;
    int n_groups;
    int64_t g_rows[6], g_cols[6];
    int g_count[6];
    size_t g_x0[6], g_x1[6], g_a[6], g_b[6];
    int w_group[6];
    MuonShapes shapes;
    // KV-cache decode buffers (their own region: a decode may follow a forward used as prefill)
    int Bp;
    size_t d_x, d_xn, d_rstd, d_qkv, d_rq, d_rk, d_y, d_act, d_part, d_attn;
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
    int static_dev = -1;  // device whose static scratch holds the workspace (ncgpt_bind_static), else -1
    int lm_mode = NCGPT_LOGITS_STORED;  // ncgpt_set_lm_head_mode
    bool fp8 = false;                   // ncgpt_set_fp8: forward linears on E4M3 operands
    bool loss_fp8 = false;              // the last ncgpt_loss ran its LM head on E4M3 operands
    SoftCap cap;                        // the logit soft-cap of cfg (off when cfg.logit_softcap == 0)
    bool cast_valid = false;  // the workspace holds a 16-bit copy of the weights (a forward or a recasting decode)
    int loss_mode = NCGPT_LOGITS_STORED;  // the mode the last ncgpt_loss ran in
    const int32_t* ids = nullptr;
    const float* params = nullptr;
    const int32_t* targets = nullptr;
    int state = 0;  // 0: nothing, 1: forward done, 2: loss done, 3: backward done
    std::string err;
    bool timing = false;
    std::vector<Timed> pending;
    std::vector<hipEvent_t> pool;
    std::vector<Agg> agg;

    template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
    size_t lay(int l, size_t o) const { return pl.layer0 + (size_t)l * pl.layer_stride + o; }
};

// ---------------------------------------------------------------- static scratch (ncgpt_bind_static)
// A workspace that lives in the library itself, for callers that cannot allocate device memory.  Each GPU
// the library runs on holds its own copy of the array until the process ends.  In host code `scratch` is
// only a host-side stand-in for the symbol: its device address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is used.
static constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];                        // device address of `scratch`, per device
std::atomic<const ncgpt_ctx*> g_scratch_owner[kMaxDevices];  // context last bound to that device's array
}  // namespace

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

// Tile for the ring and persistent GEMMs: fewest rounds of the 256 CUs weighted by each tile's time, with the
// tiles' measured relative rates -- a 256 x 128 tile loads 50 % more operand bytes per FLOP and runs at about
// 0.75 of the 256 x 256 rate, a 128 x 128 one at about 0.5 -- so a half-empty last round of large tiles can still
// beat full rounds of smaller ones.  Ties go to the larger tile.  A batched product counts the tiles of all items.
int pick_tile_rounds(int64_t M, int64_t N, int64_t batch) {
    static const int bm[3] = {256, 256, 128}, bn[3] = {256, 128, 128};
    static const double cost[3] = {1.0, 0.5 / 0.75, 0.25 / 0.5};   // time of one tile, 256 x 256 = 1
    int best = 0;
    double best_t = 1e300;
    for (int t = 0; t < 3; ++t) {
        const int64_t tiles = ((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]) * batch;
        const double time = (double)((tiles + kCUs - 1) / kCUs) * cost[t];
        if (time < best_t - 1e-9) { best_t = time; best = t; }
    }
    return best;
}

// Weight gradient dW[M,N] = sum over K tokens.  The output alone has few
// tiles (e.g. 9 for 768 x 768) while K is the whole batch of tokens, so K is
// split until one round of workgroups covers the CUs; large outputs use the
// forward tile rule.
// tile >= 0 (16-bit): that tile, with the split count from the same model
WGrad pick_wgrad(Dt dt, int64_t M, int64_t N, int64_t K, int tile = -1) {
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
        if (tile >= 0) {
            w.tile = tile;
        } else if (tiles0 < kCUs) {
            w.tile = (M >= 256 && N >= 256) ? 0 : 2;
        } else {
            w.tile = pick_tile(M, N);
        }
        int64_t tiles = ((M + bm[w.tile] - 1) / bm[w.tile]) * ((N + bn[w.tile] - 1) / bn[w.tile]);
        // splits s: rounds of the (split, tile) items times the time of a 1/s-deep tile, plus the fixed-order
        // reduce of s fp32 partials; the rates are the measured ones of these kernels (about 4.7 TFLOP/s per CU
        // for the split-K GEMMs, 6 TB/s for the reduce)
        const double tile_s = 2.0 * bm[w.tile] * bn[w.tile] * (double)K / 4.7e12, out_bytes = 4.0 * M * N;
        int64_t best = 1;
        double best_t = 1e300;
        const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(K / 512, 64));
        for (int64_t s = 1; s <= smax; ++s) {
            const double t = (double)((tiles * s + kCUs - 1) / kCUs) / (double)s * tile_s +
                             (s > 1 ? (double)(s + 1) * out_bytes / 6.0e12 : 0.0);
            if (t < best_t * 0.999) { best_t = t; best = s; }
        }
        w.splits = (int)best;
    }
    int64_t kb = K / 64;
    int64_t per = (kb + w.splits - 1) / w.splits;
    w.k_split = (int)(per * 64);
    w.splits = (int)((K + w.k_split - 1) / w.k_split);
    return w;
}

// The 16-bit LM-head GEMM z = xf Wlm^T (tokens x vocab, K = n_embd): its tile, loop and band height are
// fixed here so that the workspace plan (the CeStats column blocks) and the launches agree.
GemmDesc lm_head_desc(const ncgpt_ctx* c) {
    GemmDesc d;
    d.dt = c->dt;
    d.lda = (int)c->C; d.ldb = (int)c->C;
    d.M = (int)c->N; d.N = (int)c->V; d.K = (int)c->C;
    d.ldo = (int)c->V;
    d.tile = pick_tile(d.M, d.N);
    d.group_m = 8;
    // 32768 tiles at depth 12: the persistent ring measured 0.8 ms faster than one workgroup per tile
    d.loop = GemmLoop::Persist8;
    return d;
}

// Split-K of a decode GEMM (B rows x N, reduction K): enough workgroups of 128 x 128 tiles to cover the CUs.
struct DecSplit {
    int splits, k_split;
};
DecSplit decode_split(int N, int K) {
    const int tiles = (N + 127) / 128;
    int s = std::max(1, std::min(K / 64, (2 * kCUs + tiles - 1) / tiles));
    const int per = (K / 64 + s - 1) / s;
    DecSplit d;
    d.k_split = per * 64;
    d.splits = (K + d.k_split - 1) / d.k_split;
    return d;
}

void make_plan(ncgpt_ctx* c) {
    Plan& p = c->pl;
    size_t off = 0;
    auto A = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t e = c->esz, N = c->N;
    p.flag = A(256);
    p.cosv = A((size_t)c->T * (c->D / 2) * 4);
    p.sinv = A((size_t)c->T * (c->D / 2) * 4);
    p.wcast = A(mfma_dt(c->dt) ? (size_t)(c->P - c->VC) * 2 : 0);
    // fp8 forward linears (bf16 mode): E4M3 weights at the bf16 copy's element offsets, their per-row scales
    // (layer-major rows: qkv, Wo, Wfc, Wproj; then lm_head), and one activation's rows with their scales
    {
        const bool bf = c->dt == Dt::BF16;
        const size_t rows = (size_t)c->L * (c->QKV + 2 * c->C + c->F) + c->V;
        const size_t widest = (size_t)std::max(c->C, std::max(c->HD, c->F));
        p.w8 = A(bf ? (size_t)(c->P - c->VC) : 0);
        p.w8s = A(bf ? rows * 4 : 0);
        p.a8 = A(bf ? N * widest : 0);
        p.a8s = A(bf ? N * 4 : 0);
    }
    p.x0 = A(N * c->C * e);      // the residual stream's start: the embedding, or its RMS norm (embed_norm)
    p.rstd0 = A(c->cfg.embed_norm ? N * 4 : 0);
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
    const GemmDesc lm = lm_head_desc(c);
    p.ce_nblk = (int)((c->V + gemm_wave_cols(lm) - 1) / gemm_wave_cols(lm));
    p.cepart = A(mfma_dt(c->dt) ? N * p.ce_nblk * 8 : 0);
    p.zt = A(N * 4);
    p.lse = A(N * 4);
    p.loss_rows = A(N * 4);
    p.dxn = A(N * c->C * 4);
    p.dx = A(N * c->C * 4);
    p.dx_cd = A(mfma_dt(c->dt) ? N * c->C * 2 : 0);
    p.dh = A(N * c->F * e);
    p.dy = A(N * c->HD * e);
    p.dqkv = A(N * c->QKV * e);
    p.delta = A((size_t)2 * c->B * c->H * c->T * 4);
    // split-K partials: the largest splits * M * N over the weight gradients
    size_t sk = 0;
    const int64_t shapes[5][3] = {{c->QKV, c->C, -1}, {c->C, c->HD, -1}, {c->F, c->C, -1}, {c->C, c->F, -1},
                                  {c->V, c->C, kDWlmTile}};
    for (auto& s : shapes) {
        WGrad w = pick_wgrad(c->dt, s[0], s[1], (int64_t)N, (int)s[2]);
        if (w.splits > 1) sk = std::max(sk, (size_t)w.splits * s[0] * s[1] * 4);
    }
    p.splitk = A(sk);
    p.iscr = A(embed_bwd_scratch_ints((int)N, (int)c->V) * 4);
    p.total = off;

    // optimizer step: Newton-Schulz buffers per shape group, laid over the saved activations
    const int64_t r6[6] = {c->HD, c->KD, c->KD, c->C, c->F, c->C}, k6[6] = {c->C, c->C, c->C, c->HD, c->C, c->F};
    MuonShapes& sh = p.shapes;
    int64_t o = 0;
    for (int w = 0; w < 6; ++w) {
        sh.off[w] = o;
        sh.size[w] = r6[w] * k6[w];
        o += sh.size[w];
    }
    sh.layer = o;
    p.n_groups = 0;
    for (int w = 0; w < 6; ++w) {
        int g = 0;
        while (g < p.n_groups && !(p.g_rows[g] == r6[w] && p.g_cols[g] == k6[w])) ++g;
        if (g == p.n_groups) {
            p.g_rows[g] = r6[w];
            p.g_cols[g] = k6[w];
            p.g_count[g] = 0;
            ++p.n_groups;
        }
        p.w_group[w] = g;
        sh.group_slot[w] = p.g_count[g]++;
    }
    for (int w = 0; w < 6; ++w) sh.group_count[w] = p.g_count[p.w_group[w]];
    off = p.layer0;
    p.o_part = A((size_t)(c->L * sh.layer / 4096) * 4);
    p.o_inv = A((size_t)c->L * 6 * 4);
    for (int g = 0; g < p.n_groups; ++g) {
        const size_t items = (size_t)c->L * p.g_count[g], mm = (size_t)std::min(p.g_rows[g], p.g_cols[g]);
        p.g_x0[g] = A(items * p.g_rows[g] * p.g_cols[g] * 2);
        p.g_x1[g] = A(items * p.g_rows[g] * p.g_cols[g] * 2);
        p.g_a[g] = A(items * mm * mm * 2);
        p.g_b[g] = A(items * mm * mm * 2);
    }
    p.total = std::max(p.total, off);

    // decode: B rows padded to a multiple of 8 (the GEMMs' row granularity)
    off = p.total;
    const size_t Bp = (size_t)((c->B + 7) / 8 * 8);
    p.Bp = (int)Bp;
    p.d_x = A(Bp * c->C * e);
    p.d_xn = A(Bp * c->C * e);
    p.d_rstd = A(Bp * 4);
    p.d_qkv = A(Bp * c->QKV * e);
    p.d_rq = A(Bp * c->H * 4);
    p.d_rk = A(Bp * c->Hkv * 4);
    p.d_y = A(Bp * c->HD * e);
    p.d_act = A(Bp * c->F * e);
    size_t dp = 0;
    const int64_t dshape[5][2] = {{c->QKV, c->C}, {c->C, c->HD}, {c->F, c->C}, {c->C, c->F}, {c->V, c->C}};
    for (auto& d : dshape) {
        const DecSplit sp = decode_split((int)d[0], (int)d[1]);
        dp = std::max(dp, (size_t)sp.splits * Bp * d[0] * 4);
    }
    p.d_part = A(dp);
    p.d_attn = A(decode_attn_part_floats((int)c->B, (int)c->H, (int)c->D, (int)c->T) * 4);
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
    case Epi::ResidualCd: return "residual";
    case Epi::ReluSq: return "relusq";
    case Epi::ReluSqBwd: return "relusq_bwd";
    case Epi::Grad: return "grad";
    case Epi::SplitK: return "splitk";
    case Epi::CeStats: return "ce_stats";
    case Epi::Dz: return "dz";
    case Epi::RopeNorm: return "rope_qknorm";
    case Epi::Axpby: return "axpby";
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
ncgpt_status gemm(ncgpt_ctx* c, GemmDesc d, const char* tag, bool bf16_always = false) {
    d.dt = bf16_always ? Dt::BF16 : c->dt;
    if (d.tile < 0) d.tile = pick_tile_rounds(d.M, d.N, d.batch);
    const char* nm = intern(std::string(gemm_kernel_name(d)) + ":" + epi_name(d.epi) + ":" + tag);
    const double fl = 2.0 * d.M * d.N * d.K * d.batch;
    // algorithmic bytes: both operands once, the output (and what the epilogue reads) once
    const double e = mfma_dt(d.dt) ? 2.0 : 4.0, mn = (double)d.M * d.N;
    double out = e;
    switch (d.epi) {
    case Epi::ResidualCd: case Epi::ReluSqBwd: out = 2.0 * e; break;
    case Epi::CeStats: out = (d.out ? e : 0.0) + 8.0 * d.nblk / d.N; break;
    case Epi::Axpby: out = 4.0; break;
    case Epi::Grad: out = d.accumulate ? 8.0 : 4.0; break;
    case Epi::SplitK: out = 4.0 * std::max(1, d.splits); break;
    default: break;
    }
    const double by = (((double)d.M * d.K + (double)d.N * d.K) * (d.fp8 ? 1.0 : e) + mn * out) * d.batch;
    return launch(c, nm, fl, by, [&] { return launch_gemm(d, c->stream); });
}

// weight gradient: out(f32 grads slice [M,N]) (+)= A^T-layout x B^T-layout over K tokens
ncgpt_status wgrad(ncgpt_ctx* c, const char* tag, const void* dY, int ldy, const void* X, int ldx, int M, int N,
                   float* g, int accumulate, int tile = -1) {
    const int K = (int)c->N;
    const WGrad w = pick_wgrad(c->dt, M, N, K, tile);
    GemmDesc d;
    // both operands are read through transposing LDS reads (half rate): the four-wave persistent
    // ring, which reads fewer fragments per MFMA, measured fastest
    d.loop = GemmLoop::Persist4;
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
    if (mfma_dt(c->dt)) return c->at<uint8_t>(c->pl.wcast) + (off - c->VC) * 2;
    return c->params + off;
}

// fp8 copy of a forward weight (layer -1: lm_head; which 0: the whole qkv weight, 3: Wo, 4: Wfc, 5: Wproj) and
// the scales of its rows
const void* weight8(ncgpt_ctx* c, int layer, int which) {
    size_t off;
    int64_t r, cc;
    ncgpt_param_slice(&c->cfg, layer, which, &off, &r, &cc);
    return c->at<uint8_t>(c->pl.w8) + (off - c->VC);
}
int64_t w8_row(const ncgpt_ctx* c, int layer, int which) {
    const int64_t rpl = c->QKV + 2 * c->C + c->F;
    if (layer < 0) return c->L * rpl;
    const int64_t first[6] = {0, 0, 0, c->QKV, c->QKV + c->C, c->QKV + c->C + c->F};
    return layer * rpl + first[which];
}
const float* wscale8(ncgpt_ctx* c, int layer, int which) { return c->at<float>(c->pl.w8s) + w8_row(c, layer, which); }

// E4M3 copies of every forward weight with their row scales, from the fp32 parameters: one launch per matrix
// kind over all layers, and the lm_head
ncgpt_status quantize_weights(ncgpt_ctx* c) {
    const int64_t lp = layer_params(&c->cfg), rpl = c->QKV + 2 * c->C + c->F;
    struct Kind { int which; int64_t rows, cols; } kinds[4] = {
        {0, c->QKV, c->C}, {3, c->C, c->HD}, {4, c->F, c->C}, {5, c->C, c->F}};
    for (const Kind& k : kinds) {
        size_t off;
        int64_t r, cc;
        ncgpt_param_slice(&c->cfg, 0, k.which, &off, &r, &cc);
        TRY(launch(c, "quant_fp8_w", 0.0, (double)c->L * k.rows * k.cols * 5, [&] {
            return launch_quant_rows_fp8(Dt::F32, c->params + off, (size_t)lp, c->at<uint8_t>(c->pl.w8) + (off - c->VC),
                                         (size_t)lp, c->at<float>(c->pl.w8s) + w8_row(c, 0, k.which), (size_t)rpl,
                                         (int)k.rows, (int)k.cols, (int)c->L, c->stream);
        }));
    }
    size_t off;
    int64_t r, cc;
    ncgpt_param_slice(&c->cfg, -1, 1, &off, &r, &cc);
    return launch(c, "quant_fp8_w", 0.0, (double)c->VC * 5, [&] {
        return launch_quant_rows_fp8(Dt::F32, c->params + off, 0, c->at<uint8_t>(c->pl.w8) + (off - c->VC), 0,
                                     c->at<float>(c->pl.w8s) + w8_row(c, -1, 1), 0, (int)c->V, (int)c->C, 1, c->stream);
    });
}

// E4M3 rows of one [N, cols] activation (compute dtype bf16) into the shared fp8 activation buffer
ncgpt_status quantize_act(ncgpt_ctx* c, const void* x, int cols) {
    return launch(c, "quant_fp8", 0.0, (double)c->N * cols * 3 + c->N * 4.0, [&] {
        return launch_quant_rows_fp8(Dt::BF16, x, 0, c->at<uint8_t>(c->pl.a8), 0, c->at<float>(c->pl.a8s), 0,
                                     (int)c->N, cols, 1, c->stream);
    });
}

// the RMSNorm kernel that holds rows in registers also writes the E4M3 copy (n_embd = 256 k, k in 1..6 or 8)
bool norm_writes_fp8(const ncgpt_ctx* c) {
    const int64_t k = c->C / 256;
    return c->C % 256 == 0 && k >= 1 && k <= 8 && k != 7;
}

// RMSNorm of [N, C] rows; in fp8 mode the E4M3 rows land in the activation buffer (from the norm kernel
// itself when it can, else from the row quantiser)
ncgpt_status norm_fwd(ncgpt_ctx* c, const void* x, void* y, float* rstd, bool to_fp8) {
    const Plan& p = c->pl;
    const bool fused = to_fp8 && norm_writes_fp8(c);
    const double bytes = (double)c->N * c->C * (2 * c->esz + (fused ? 1 : 0)) + c->N * 4.0;
    TRY(launch(c, "rmsnorm_fwd", 0.0, bytes, [&] {
        return launch_rmsnorm_fwd(c->dt, x, y, rstd, (int)c->N, (int)c->C, c->cfg.norm_eps, c->stream,
                                  fused ? (void*)c->at<uint8_t>(p.a8) : nullptr, fused ? c->at<float>(p.a8s) : nullptr);
    }));
    if (to_fp8 && !fused) TRY(quantize_act(c, y, (int)c->C));
    return NCGPT_OK;
}

// turn a forward GEMM (A = the activation last quantised, B = weight (layer, which)) into its fp8 form
void use_fp8(ncgpt_ctx* c, GemmDesc& d, int layer, int which) {
    d.fp8 = true;
    d.A = c->at<uint8_t>(c->pl.a8);
    d.B = weight8(c, layer, which);
    d.rsa = c->at<float>(c->pl.a8s);
    d.rsb = wscale8(c, layer, which);
    d.tile = 0;
    d.loop = GemmLoop::Ring8;
}

// Attach a workspace and stream: upload the RoPE tables, clear the device error flag (a kernel, not a
// memset node), reset the call-order state.
ncgpt_status bind_common(ncgpt_ctx* c, uint8_t* ws, size_t bytes, void* stream) {
    c->ws = ws;
    c->ws_bytes = bytes;
    c->stream = static_cast<hipStream_t>(stream);
    c->bound = false;
    hipError_t e = hipMemcpyAsync(c->ws + c->pl.cosv, c->cos_host.data(), c->cos_host.size() * 4,
                                  hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->ws + c->pl.sinv, c->sin_host.data(), c->sin_host.size() * 4, hipMemcpyHostToDevice,
                           c->stream);
    if (e == hipSuccess) e = launch_zero_u32(c->at<uint32_t>(c->pl.flag), 64, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "bind uploads");
    c->bound = true;
    c->state = 0;
    c->cast_valid = false;
    return NCGPT_OK;
}

// A context bound to a device's static scratch gives the array up (when it still owns it).
void release_static(ncgpt_ctx* c) {
    if (c->static_dev >= 0) {
        const ncgpt_ctx* me = c;
        g_scratch_owner[c->static_dev].compare_exchange_strong(me, nullptr);
        c->static_dev = -1;
    }
}

// Bound, and (for the static scratch) still the array's owner.
ncgpt_status check_bound(ncgpt_ctx* c) {
    if (!c->bound) return fail(c, NCGPT_ESTATE, "ncgpt_bind has not been called");
    if (c->static_dev >= 0 && g_scratch_owner[c->static_dev].load() != c) {
        c->bound = false;
        c->state = 0;
        return fail(c, NCGPT_ESTATE, "another context has been bound to this device's static scratch since");
    }
    return NCGPT_OK;
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
    if (!valid_cfg(g) || (dtype != NCGPT_F32 && dtype != NCGPT_BF16 && dtype != NCGPT_F16)) return NCGPT_EINVAL;
    const bool bf = dtype != NCGPT_F32;   // the 16-bit MFMA path (bf16 or fp16)
    if (g->n_head % g->n_kv_head) return NCGPT_EUNSUPPORTED;
    if (bf ? g->head_dim != 128 : (g->head_dim != 64 && g->head_dim != 128)) return NCGPT_EUNSUPPORTED;
    if (g->n_embd % 64 || g->mlp_dim % 64 || g->vocab_size % 64) return NCGPT_EUNSUPPORTED;
    if (g->vocab_size > 65536) return NCGPT_EUNSUPPORTED;  // the embedding-gradient counting sort
    if (bf ? g->seq_len % 128 : g->seq_len % 64) return NCGPT_EUNSUPPORTED;
    if ((double)g->batch * g->seq_len * g->vocab_size > 4.0e12) return NCGPT_EUNSUPPORTED;
    if (!(g->norm_eps >= 0.0f) || !(g->rope_base > 0.0f)) return NCGPT_EINVAL;
    if (!(g->logit_softcap >= 0.0f) || !std::isfinite(g->logit_softcap)) return NCGPT_EINVAL;
    if (g->embed_norm != 0 && g->embed_norm != 1) return NCGPT_EINVAL;
    ncgpt_ctx* c = new (std::nothrow) ncgpt_ctx();
    if (!c) return NCGPT_ENOMEM;
    c->cfg = *g;
    c->dtype = dtype;
    c->dt = dtype == NCGPT_BF16 ? Dt::BF16 : (dtype == NCGPT_F16 ? Dt::F16 : Dt::F32);
    c->L = g->n_layer; c->C = g->n_embd; c->H = g->n_head; c->Hkv = g->n_kv_head; c->D = g->head_dim;
    c->F = g->mlp_dim; c->V = g->vocab_size; c->B = g->batch; c->T = g->seq_len;
    c->N = c->B * c->T; c->HD = c->H * c->D; c->KD = c->Hkv * c->D; c->QKV = c->HD + 2 * c->KD;
    c->P = (int64_t)ncgpt_num_params(g);
    c->VC = c->V * c->C;
    c->esz = bf ? 2 : 4;
    c->cap = make_softcap(g->logit_softcap);
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
    release_static(c);
    return bind_common(c, static_cast<uint8_t*>(workspace), bytes, stream);
}

ncgpt_status ncgpt_bind_static(ncgpt_ctx* c, void* stream) {
    if (!c) return NCGPT_EINVAL;
    if (c->pl.total > kStaticScratchBytes)
        return fail(c, NCGPT_ENOMEM, "workspace of " + std::to_string(c->pl.total) + " bytes exceeds the " +
                                         std::to_string(kStaticScratchBytes) + "-byte static scratch");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(c, e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(c, NCGPT_EUNSUPPORTED, "device index beyond the static scratch table");
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(c, e, "hipGetSymbolAddress(scratch)");
            if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255))
                return fail(c, NCGPT_EHIP, "static scratch has no 256-byte aligned device address");
            g_scratch_ptr[dev] = ptr;
        }
        ptr = g_scratch_ptr[dev];
    }
    release_static(c);
    ncgpt_status st = bind_common(c, static_cast<uint8_t*>(ptr), kStaticScratchBytes, stream);
    if (st != NCGPT_OK) return st;
    c->static_dev = dev;
    g_scratch_owner[dev].store(c);
    return NCGPT_OK;
}

ncgpt_status ncgpt_forward(ncgpt_ctx* c, const int32_t* ids, const float* params) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
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

    if (mfma_dt(dt)) {
        const size_t n = (size_t)(c->P - c->VC);
        TRY(launch(c, "cast_bf16", 0.0, (double)n * 6,
                   [&] { return launch_cast_bf16(params + c->VC, c->ws + p.wcast, n, c->stream, dt); }));
        c->cast_valid = true;
        if (c->fp8) TRY(quantize_weights(c));
    }
    const double norm_bytes = (double)N * C * 2 * e + N * 4.0;
    // the embedding; with embed_norm it passes through an RMSNorm before it enters the first block (the raw
    // rows go through x, which the first block overwrites)
    uint8_t* emb = c->ws + (c->cfg.embed_norm ? p.x : p.x0);
    TRY(launch(c, "embed_fwd", 0.0, (double)N * C * (4 + e) + N * 4.0, [&] {
        return launch_embed_fwd(dt, ids, params, emb, N, C, V, flag, c->stream);
    }));
    if (c->cfg.embed_norm) {
        TRY(launch(c, "rmsnorm_fwd", 0.0, norm_bytes, [&] {
            return launch_rmsnorm_fwd(dt, emb, c->ws + p.x0, c->at<float>(p.rstd0), N, C, eps, c->stream);
        }));
    }
    for (int l = 0; l < c->L; ++l) {
        uint8_t* xin = c->ws + (l == 0 ? p.x0 : p.x);
        uint8_t* xn1 = c->ws + c->lay(l, p.l_xn1);
        uint8_t* qkv = c->ws + c->lay(l, p.l_qkv);
        uint8_t* y = c->ws + c->lay(l, p.l_y);
        uint8_t* xn2 = c->ws + c->lay(l, p.l_xn2);
        uint8_t* act = c->ws + c->lay(l, p.l_act);
        TRY(norm_fwd(c, xin, xn1, c->at<float>(c->lay(l, p.l_rstd1)), c->fp8));
        {
            GemmDesc d;
            d.A = xn1; d.lda = C; d.B = weight(c, l, 0); d.ldb = C;
            d.M = N; d.N = QKV; d.K = C;
            d.out = qkv; d.ldo = QKV;
            d.group_m = 8;  // bands of 8 tile-rows measured faster than bands of 4 for this shape
            if (mfma_dt(dt)) {
                // RoPE + QK-norm in the epilogue: each wave of the 4 x 2 grid owns one head
                d.epi = Epi::RopeNorm; d.loop = GemmLoop::Persist8Heads; d.tile = 0;
                d.cosv = c->at<float>(p.cosv); d.sinv = c->at<float>(p.sinv);
                d.rstdq = c->at<float>(c->lay(l, p.l_rstdq)); d.rstdk = c->at<float>(c->lay(l, p.l_rstdk));
                d.T = (int)c->T; d.H = (int)c->H; d.Hkv = (int)c->Hkv; d.eps = eps;
                if (c->fp8) use_fp8(c, d, l, 0);   // xn1's E4M3 rows came with the norm
                TRY(gemm(c, d, "qkv"));
            } else {
                d.epi = Epi::StoreCd;
                TRY(gemm(c, d, "qkv"));
                TRY(launch(c, "rope_qknorm_fwd", 0.0, (double)N * (c->H + c->Hkv) * c->D * 2 * e, [&] {
                    return launch_rope_qknorm_fwd(dt, qkv, c->at<float>(c->lay(l, p.l_rstdq)),
                                                  c->at<float>(c->lay(l, p.l_rstdk)), c->at<float>(p.cosv),
                                                  c->at<float>(p.sinv), N, (int)c->T, (int)c->H, (int)c->Hkv,
                                                  (int)c->D, eps, c->stream);
                }));
            }
        }
        {
            AttnDesc ad;
            ad.dt = dt; ad.B = (int)c->B; ad.T = (int)c->T; ad.H = (int)c->H; ad.Hkv = (int)c->Hkv; ad.D = (int)c->D;
            ad.qkv = qkv; ad.y = y; ad.lse = c->at<float>(c->lay(l, p.l_lse));
            const double pairs = (double)c->B * c->H * c->T * (c->T + 1) / 2.0;
            // algorithmic bytes: read q, k, v; write y and the row log-sum-exp
            const double qb = (double)N * c->H * c->D * e, kb = (double)N * c->Hkv * c->D * e;
            TRY(launch(c, mfma_dt(dt) ? "attn_fwd_bf16" : "attn_fwd_f32", 4.0 * c->D * pairs,
                       2 * qb + 2 * kb + (double)N * c->H * 4, [&] { return launch_attn_fwd(ad, c->stream); }));
        }
        {
            GemmDesc d;
            d.A = y; d.lda = HD; d.B = weight(c, l, 3); d.ldb = HD;
            d.M = N; d.N = C; d.K = HD;
            d.epi = Epi::ResidualCd; d.out = c->ws + p.x; d.in = xin; d.ldo = C;
            d.loop = GemmLoop::Ring8;  // epilogue reads the residual: the eight-wave ring without spills
            d.group_m = 8;
            if (c->fp8) {
                TRY(quantize_act(c, y, HD));
                use_fp8(c, d, l, 3);
            }
            TRY(gemm(c, d, "attn_out"));
        }
        TRY(norm_fwd(c, c->ws + p.x, xn2, c->at<float>(c->lay(l, p.l_rstd2)), c->fp8));
        {
            GemmDesc d;
            d.A = xn2; d.lda = C; d.B = weight(c, l, 4); d.ldb = C;
            d.M = N; d.N = F; d.K = C;
            d.epi = Epi::ReluSq; d.out = act; d.ldo = F;
            d.loop = GemmLoop::Ring8;  // the non-persistent eight-wave ring measured fastest for this shape
            if (c->fp8) use_fp8(c, d, l, 4);      // xn2's E4M3 rows came with the norm
            TRY(gemm(c, d, "fc"));
        }
        {
            GemmDesc d;
            d.A = act; d.lda = F; d.B = weight(c, l, 5); d.ldb = F;
            d.M = N; d.N = C; d.K = F;
            d.epi = Epi::ResidualCd; d.out = c->ws + p.x; d.in = c->ws + p.x; d.ldo = C;
            d.loop = GemmLoop::Persist8;  // measured faster than the non-persistent ring despite a small spill
            d.group_m = 2;                // the n_embd-wide outputs: bands of 2 tile-rows measured fastest
            if (c->fp8) {
                TRY(quantize_act(c, act, F));
                use_fp8(c, d, l, 5);
            }
            TRY(gemm(c, d, "proj"));
        }
    }
    TRY(norm_fwd(c, c->ws + p.x, c->ws + p.xf, c->at<float>(p.rstdf), c->fp8));  // xf's E4M3 rows for the LM head
    c->state = 1;
    return NCGPT_OK;
}

ncgpt_status ncgpt_loss(ncgpt_ctx* c, const int32_t* targets, float* loss) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
    if (c->state < 1) return fail(c, NCGPT_ESTATE, "ncgpt_loss before ncgpt_forward");
    if (!targets || !loss) return fail(c, NCGPT_EINVAL, "null targets or loss");
    const Plan& p = c->pl;
    const int N = (int)c->N, V = (int)c->V;
    uint32_t* flag = c->at<uint32_t>(p.flag);
    c->targets = targets;
    c->state = 1;
    GemmDesc d = lm_head_desc(c);
    d.A = c->ws + p.xf; d.B = weight(c, -1, 1);
    if (mfma_dt(c->dt)) {
        // logits, their softmax statistics and the target logit in one pass; the logits are stored for the
        // backward only in the stored-logit mode
        d.epi = Epi::CeStats;
        d.out = c->lm_mode == NCGPT_LOGITS_STORED ? (void*)(c->ws + p.logits) : nullptr;
        d.part = c->ws + p.cepart; d.nblk = p.ce_nblk;
        d.zt = c->at<float>(p.zt); d.targets = targets;
        d.cap = c->cap;
        if (c->fp8) use_fp8(c, d, -1, 1);   // the forward's final norm left xf's E4M3 rows
        const int nblk = (int)((V + gemm_wave_cols(d) - 1) / gemm_wave_cols(d));  // <= p.ce_nblk
        d.nblk = nblk;
        TRY(gemm(c, d, c->lm_mode == NCGPT_LOGITS_STORED ? "lm_head" : "lm_head_nostore"));
        TRY(launch(c, "ce_merge", 0.0, (double)N * nblk * 8 + N * 16.0, [&] {
            return launch_ce_merge(c->ws + p.cepart, nblk, c->at<float>(p.zt), targets, c->at<float>(p.lse),
                                   c->at<float>(p.loss_rows), N, V, flag, c->stream);
        }));
    } else {
        d.epi = Epi::StoreCd; d.out = c->ws + p.logits;
        TRY(gemm(c, d, "lm_head"));
        if (c->cap.c > 0.0f) {
            TRY(launch(c, "softcap", 0.0, (double)N * V * c->esz * 2, [&] {
                return launch_softcap(c->dt, c->ws + p.logits, (size_t)N * V, c->cap, c->stream);
            }));
        }
        TRY(launch(c, "ce_fwd_rows", 0.0, (double)N * V * c->esz + N * 12.0, [&] {
            return launch_ce_fwd_rows(c->dt, c->ws + p.logits, targets, c->at<float>(p.lse), c->at<float>(p.loss_rows),
                                      N, V, flag, c->stream);
        }));
    }
    TRY(launch(c, "loss_reduce", 0.0, N * 8.0, [&] {
        return launch_loss_reduce(c->at<float>(p.loss_rows), targets, N, V, loss, c->at<float>(p.flag + 4), flag,
                                  c->stream);
    }));
    c->loss_mode = mfma_dt(c->dt) ? c->lm_mode : NCGPT_LOGITS_STORED;
    c->loss_fp8 = c->fp8;
    c->state = 2;
    return NCGPT_OK;
}

ncgpt_status ncgpt_set_fp8(ncgpt_ctx* c, int on) {
    if (!c) return NCGPT_EINVAL;
    if (on != 0 && on != 1) return fail(c, NCGPT_EINVAL, "fp8 switch is 0 or 1");
    if (on && c->dt != Dt::BF16) return fail(c, NCGPT_EUNSUPPORTED, "fp8 linears are built for the bf16 compute dtype");
    if (on && (c->C % 128 || c->HD % 128 || c->F % 128))
        return fail(c, NCGPT_EUNSUPPORTED, "fp8 linears need n_embd, n_head * head_dim and mlp_dim multiples of 128");
    c->fp8 = on != 0;
    c->state = 0;  // the saved activations of an earlier forward do not match the new setting
    return NCGPT_OK;
}

ncgpt_status ncgpt_set_lm_head_mode(ncgpt_ctx* c, int mode) {
    if (!c) return NCGPT_EINVAL;
    if (mode != NCGPT_LOGITS_STORED && mode != NCGPT_LOGITS_RECOMPUTED) return fail(c, NCGPT_EINVAL, "unknown mode");
    if (mode == NCGPT_LOGITS_RECOMPUTED && !mfma_dt(c->dt))
        return fail(c, NCGPT_EUNSUPPORTED, "the recomputed-logit mode is built for the 16-bit compute dtypes");
    c->lm_mode = mode;
    return NCGPT_OK;
}

ncgpt_status ncgpt_backward(ncgpt_ctx* c, float* grads, int accumulate, float grad_scale) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
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
    uint8_t* dxg = mfma_dt(dt) ? c->ws + p.dx_cd : c->ws + p.dx;  // GEMM operand copy of dx
    void* dx_cd = mfma_dt(dt) ? (void*)(c->ws + p.dx_cd) : nullptr;

    auto gslice = [&](int layer, int which) {
        size_t off;
        int64_t r, cc;
        ncgpt_param_slice(&c->cfg, layer, which, &off, &r, &cc);
        return grads + off;
    };

    if (c->loss_mode == NCGPT_LOGITS_RECOMPUTED) {
        // the logits again, turned into dz by the GEMM's epilogue (nothing was stored by ncgpt_loss)
        GemmDesc d = lm_head_desc(c);
        d.A = c->ws + p.xf; d.B = weight(c, -1, 1);
        d.epi = Epi::Dz; d.out = logits;
        d.lse = c->at<float>(p.lse); d.targets = c->targets; d.inv_valid = c->at<float>(p.flag + 4);
        d.grad_scale = grad_scale;
        d.cap = c->cap;
        if (c->loss_fp8) use_fp8(c, d, -1, 1);  // the loss left xf's E4M3 rows in the activation buffer
        TRY(gemm(c, d, "lm_head_dz"));
    } else {
        // cross-entropy -> dz (in place over the logits)
        TRY(launch(c, "ce_bwd", 0.0, (double)N * V * 2 * e, [&] {
            return launch_ce_bwd(dt, logits, c->at<float>(p.lse), c->targets, c->at<float>(p.flag + 4), grad_scale,
                                 c->cap, N, V, c->stream);
        }));
    }
    {   // dxf = dz Wlm
        GemmDesc d;
        d.A = logits; d.lda = V; d.B = weight(c, -1, 1); d.ldb = C; d.b_kcontig = false;
        d.M = N; d.N = C; d.K = V;
        d.epi = Epi::StoreCd; d.out = dxn; d.ldo = C;  // compute dtype
        d.loop = GemmLoop::Ring8;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
        d.group_m = 2;             // the n_embd-wide outputs: bands of 2 tile-rows measured fastest
        TRY(gemm(c, d, "dxf"));
    }
    // dWlm = dz^T xf: vocab x n_embd output over all tokens (the tile: kDWlmTile)
    TRY(wgrad(c, "dWlm", logits, V, c->ws + p.xf, C, V, C, gslice(-1, 1), acc, kDWlmTile));
    // In the 16-bit modes the residual-stream gradient lives in the compute dtype, as the residual stream itself
    // does (dx_cd, read and written by every norm's backward); only layer 0's also leaves it in fp32 (dx) for the
    // embedding gradient.  fp32 keeps it in dx.
    const bool g16 = mfma_dt(dt);
    float* const dx_acc = g16 ? nullptr : dx;
    const int acc_from = g16 ? 2 : 1;
    auto nb_of = [&](int accumulate, bool f32_out) {   // bytes of one norm backward
        return (double)N * C * (2.0 * e + (accumulate ? e : 0) + (g16 ? 2 : 0) + (f32_out ? 4 : 0)) + N * 4.0;
    };
    TRY(launch(c, "rmsnorm_bwd", 0.0, nb_of(0, !g16), [&] {
        return launch_rmsnorm_bwd(dt, c->ws + p.xf, c->at<float>(p.rstdf), dxn, dx_acc, dx_cd, N, C, 0, c->stream);
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
            d.loop = GemmLoop::Ring8;  // epilogue reads act: the eight-wave ring without spills
            TRY(gemm(c, d, "dh"));
        }
        TRY(wgrad(c, "dWproj", dxg, C, act, F, C, F, gslice(l, 5), acc));  // dWproj = dx^T act
        {   // dxn2 = dh Wfc
            GemmDesc d;
            d.A = c->ws + p.dh; d.lda = F; d.B = weight(c, l, 4); d.ldb = C; d.b_kcontig = false;
            d.M = N; d.N = C; d.K = F;
            d.epi = Epi::StoreCd; d.out = dxn; d.ldo = C;  // compute dtype
            d.loop = GemmLoop::Ring8;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
            d.group_m = 2;             // the n_embd-wide outputs: bands of 2 tile-rows measured fastest
            TRY(gemm(c, d, "dxn2"));
        }
        TRY(wgrad(c, "dWfc", c->ws + p.dh, F, xn2, C, F, C, gslice(l, 4), acc));  // dWfc = dh^T xn2
        TRY(launch(c, "rmsnorm_bwd", 0.0, nb_of(1, !g16), [&] {
            return launch_rmsnorm_bwd(dt, xn2, c->at<float>(c->lay(l, p.l_rstd2)), dxn, dx_acc, dx_cd, N, C, acc_from,
                                      c->stream);
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
            const bool bf = mfma_dt(dt);
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
        if (!mfma_dt(dt)) {  // the 16-bit attention backward applies it in its epilogues
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
            d.loop = GemmLoop::Ring8;  // input gradients (NN): the non-persistent eight-wave ring measured fastest
            d.group_m = 2;             // the n_embd-wide outputs: bands of 2 tile-rows measured fastest
            TRY(gemm(c, d, "dxn1"));
        }
        TRY(wgrad(c, "dWqkv", c->ws + p.dqkv, QKV, xn1, C, QKV, C, gslice(l, 0), acc));  // dWqkv = dqkv^T xn1
        TRY(launch(c, "rmsnorm_bwd", 0.0, nb_of(1, !g16 || l == 0), [&] {
            return launch_rmsnorm_bwd(dt, xn1, c->at<float>(c->lay(l, p.l_rstd1)), dxn, l == 0 ? dx : dx_acc, dx_cd,
                                      N, C, acc_from, c->stream);
        }));
    }
    float* demb = dx;    // the gradient at the embedding's output
    float* escr = dxn;   // embed_bwd's [N, C] scratch
    if (c->cfg.embed_norm) {
        // through the embedding norm: its input gradient into dxn (from dx in the compute dtype, as every norm's
        // backward takes it), then dx serves as the scratch
        const void* dy = mfma_dt(dt) ? (const void*)(c->ws + p.dx_cd) : (const void*)dx;
        TRY(launch(c, "rmsnorm_bwd", 0.0, (double)N * C * (2.0 * e + 4) + N * 4.0, [&] {
            return launch_rmsnorm_bwd(dt, c->ws + p.x0, c->at<float>(p.rstd0), dy, dxn, nullptr, N, C, 0, c->stream);
        }));
        demb = dxn;
        escr = dx;
    }
    TRY(launch(c, "embed_bwd", 0.0, (double)N * C * 8 + (double)V * C * (4 + 4 * acc), [&] {
        return launch_embed_bwd(c->ids, demb, gslice(-1, 0), N, C, V, acc, c->at<int32_t>(p.iscr), escr, c->stream);
    }));
    c->state = 3;
    return NCGPT_OK;
}

size_t ncgpt_optim_state_size(const ncgpt_config* g) {
    if (!valid_cfg(g)) return 0;
    const int64_t VC = (int64_t)g->vocab_size * g->n_embd;
    return (size_t)((int64_t)g->n_layer * layer_params(g) + 4 * VC);
}

ncgpt_status ncgpt_optim_step(ncgpt_ctx* c, float* params, const float* grads, float* state, int64_t step,
                              const ncgpt_optim_config* oc) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
    if (c->state == 1 || c->state == 2)
        return fail(c, NCGPT_ESTATE, "ncgpt_optim_step between ncgpt_forward and ncgpt_backward");
    if (!params || !grads || !state || !oc) return fail(c, NCGPT_EINVAL, "null params, grads, state or config");
    if (step < 1 || oc->ns_steps < 0 || oc->ns_steps > 20 || !(oc->muon_momentum >= 0.0f && oc->muon_momentum < 1.0f) ||
        !(oc->adam_beta1 >= 0.0f && oc->adam_beta1 < 1.0f) || !(oc->adam_beta2 >= 0.0f && oc->adam_beta2 < 1.0f) ||
        !(oc->ns_eps > 0.0f))
        return fail(c, NCGPT_EINVAL, "optimizer step or constants out of range");
    const Plan& p = c->pl;
    const MuonShapes& sh = p.shapes;
    const int L = (int)c->L;
    const int64_t VC = c->VC, nmat = (int64_t)L * sh.layer;
    const float mu = oc->muon_momentum;
    const int nest = oc->muon_nesterov ? 1 : 0;
    c->state = 0;   // the Newton-Schulz scratch overwrites the saved activations
    float* gm = const_cast<float*>(grads) + VC;   // the packed matrix range
    float* pm = params + VC;
    float* part = c->at<float>(p.o_part);
    float* inv = c->at<float>(p.o_inv);
    TRY(launch(c, "muon_momentum", 0.0, (double)nmat * 12, [&] {
        return launch_muon_momentum(gm, state, part, (size_t)nmat, mu, nest, c->stream);
    }));
    TRY(launch(c, "muon_norm", 0.0, (double)nmat / 4096 * 4, [&] {
        return launch_muon_norm(part, inv, sh, L, oc->ns_eps, c->stream);
    }));
    for (int w = 0; w < 6; ++w) {
        const int g = p.w_group[w];
        TRY(launch(c, "muon_init", 0.0, (double)L * sh.size[w] * 10, [&] {
            return launch_muon_init(gm, state, inv, c->ws + p.g_x0[g], sh, w, L, mu, nest, c->stream);
        }));
    }
    // Newton-Schulz on each shape group, batched over its L * count matrices
    for (int g = 0; g < p.n_groups; ++g) {
        const int R = (int)p.g_rows[g], Cc = (int)p.g_cols[g], batch = L * p.g_count[g];
        const bool tall = R > Cc;
        const int m = tall ? Cc : R;
        uint8_t* X[2] = {c->ws + p.g_x0[g], c->ws + p.g_x1[g]};
        uint8_t* Am = c->ws + p.g_a[g];
        uint8_t* Bm = c->ws + p.g_b[g];
        const int64_t sx = (int64_t)R * Cc, sm = (int64_t)m * m;
        for (int it = 0; it < oc->ns_steps; ++it) {
            uint8_t* x = X[it & 1];
            uint8_t* xn = X[(it + 1) & 1];
            {   // A = X X^T (wide) or X^T X (tall)
                GemmDesc d;
                d.A = x; d.B = x; d.lda = Cc; d.ldb = Cc;
                d.a_kcontig = !tall; d.b_kcontig = !tall;
                d.M = m; d.N = m; d.K = tall ? R : Cc;
                d.epi = Epi::StoreCd; d.out = Am; d.ldo = m;
                d.loop = GemmLoop::Ring8;
                d.batch = batch; d.sA = sx; d.sB = sx; d.sOut = sm;
                TRY(gemm(c, d, "ns_gram", true));
            }
            {   // B = b A + c A A
                GemmDesc d;
                d.A = Am; d.B = Am; d.lda = m; d.ldb = m; d.b_kcontig = false;
                d.M = m; d.N = m; d.K = m;
                d.epi = Epi::Axpby; d.out = Bm; d.in = Am; d.ldo = m; d.alpha = oc->ns_b; d.beta = oc->ns_c;
                d.loop = GemmLoop::Ring8;
                d.batch = batch; d.sA = sm; d.sB = sm; d.sOut = sm; d.sIn = sm;
                TRY(gemm(c, d, "ns_poly", true));
            }
            {   // X = a X + B X (wide) or a X + X B (tall)
                GemmDesc d;
                if (tall) { d.A = x; d.lda = Cc; d.B = Bm; d.ldb = m; d.sA = sx; d.sB = sm; d.K = Cc; }
                else { d.A = Bm; d.lda = m; d.B = x; d.ldb = Cc; d.sA = sm; d.sB = sx; d.K = R; }
                d.b_kcontig = false;
                d.M = R; d.N = Cc;
                d.epi = Epi::Axpby; d.out = xn; d.in = x; d.ldo = Cc; d.alpha = oc->ns_a; d.beta = 1.0f;
                d.loop = GemmLoop::Ring8;
                d.batch = batch; d.sOut = sx; d.sIn = sx;
                TRY(gemm(c, d, "ns_update", true));
            }
        }
    }
    const float decay = 1.0f - oc->matrix_lr * oc->weight_decay;
    for (int w = 0; w < 6; ++w) {
        const int g = p.w_group[w];
        const double ratio = (double)p.g_rows[g] / (double)p.g_cols[g];
        const float scaled = (float)(oc->matrix_lr * std::sqrt(std::max(1.0, ratio)));
        TRY(launch(c, "muon_apply", 0.0, (double)L * sh.size[w] * 10, [&] {
            return launch_muon_apply(pm, c->ws + (oc->ns_steps & 1 ? p.g_x1[g] : p.g_x0[g]), sh, w, L, decay, scaled,
                                     c->stream);
        }));
    }
    // AdamW on wte and lm_head
    const double bc1 = 1.0 - std::pow((double)oc->adam_beta1, (double)step);
    const double bc2 = 1.0 - std::pow((double)oc->adam_beta2, (double)step);
    for (int which = 0; which < 2; ++which) {
        size_t off;
        int64_t r, k;
        ncgpt_param_slice(&c->cfg, -1, which, &off, &r, &k);
        const float lr = which == 0 ? oc->embedding_lr : oc->unembedding_lr;
        AdamArgs a{lr, oc->adam_beta1, oc->adam_beta2, oc->adam_eps, (float)bc1, (float)bc2,
                   1.0f - lr * oc->weight_decay};
        float* mo = state + nmat + (size_t)which * 2 * VC;
        TRY(launch(c, "adamw", 0.0, (double)VC * 28, [&] {
            return launch_adamw(params + off, grads + off, mo, mo + VC, (size_t)VC, a, c->stream);
        }));
    }
    return NCGPT_OK;
}

size_t ncgpt_kv_cache_bytes(const ncgpt_ctx* c) {
    if (!c) return 0;
    return (size_t)c->L * 2 * c->B * c->Hkv * c->T * c->D * c->esz;
}

ncgpt_status ncgpt_kv_fill(ncgpt_ctx* c, void* kv_cache, int32_t n) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
    if (c->state < 1) return fail(c, NCGPT_ESTATE, "ncgpt_kv_fill needs the k and v of an ncgpt_forward");
    if (!kv_cache || n < 0 || n > c->T) return fail(c, NCGPT_EINVAL, "null cache or position count outside [0, seq_len]");
    const Plan& p = c->pl;
    const size_t per_layer = (size_t)2 * c->B * c->Hkv * c->T * c->D * c->esz;
    for (int l = 0; l < c->L; ++l) {
        TRY(launch(c, "kv_fill", 0.0, (double)per_layer * n / c->T * 2, [&] {
            return launch_kv_store(c->dt, c->ws + c->lay(l, p.l_qkv), static_cast<uint8_t*>(kv_cache) + l * per_layer,
                                   (int)c->B, (int)c->H, (int)c->Hkv, (int)c->D, (int)c->T, 0, n, (int)c->T, c->stream);
        }));
    }
    return NCGPT_OK;
}

ncgpt_status ncgpt_decode_step(ncgpt_ctx* c, const int32_t* ids, const float* params, void* kv_cache, int32_t pos,
                               float* logits, int recast) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
    if (!ids || !params || !kv_cache || !logits) return fail(c, NCGPT_EINVAL, "null ids, params, cache or logits");
    if (pos < 0 || pos >= c->T) return fail(c, NCGPT_EINVAL, "position outside [0, seq_len)");
    const Plan& p = c->pl;
    const Dt dt = c->dt;
    const int B = (int)c->B, Bp = p.Bp, C = (int)c->C, F = (int)c->F, QKV = (int)c->QKV, HD = (int)c->HD;
    const int V = (int)c->V;
    const float eps = c->cfg.norm_eps;
    const size_t e = c->esz;
    // the fp32 weights of this call (weight() reads them); the forward's pointer is restored on return, so a
    // pending backward still sees its own parameters
    struct Restore {
        ncgpt_ctx* c;
        const float* saved;
        ~Restore() { c->params = saved; }
    } restore{c, c->params};
    c->params = params;
    if (mfma_dt(dt)) {
        if (recast) {
            const size_t n = (size_t)(c->P - c->VC);
            TRY(launch(c, "cast_bf16", 0.0, (double)n * 6,
                       [&] { return launch_cast_bf16(params + c->VC, c->ws + p.wcast, n, c->stream, dt); }));
            c->cast_valid = true;
        } else if (!c->cast_valid) {
            return fail(c, NCGPT_ESTATE, "no 16-bit weight copy yet: pass recast = 1");
        }
    }
    uint8_t* x = c->ws + p.d_x;
    uint8_t* xn = c->ws + p.d_xn;
    uint8_t* qkv = c->ws + p.d_qkv;
    uint8_t* y = c->ws + p.d_y;
    uint8_t* act = c->ws + p.d_act;
    float* part = c->at<float>(p.d_part);
    uint32_t* flag = c->at<uint32_t>(p.flag);
    // padding rows stay zero: every row is independent, the padded ones are never read back
    TRY(launch(c, "decode_zero", 0.0, 0.0, [&] {
        hipError_t st = launch_zero_u32(reinterpret_cast<uint32_t*>(x), (size_t)Bp * C * e / 4, c->stream);
        return st == hipSuccess ? launch_zero_u32(reinterpret_cast<uint32_t*>(y), (size_t)Bp * HD * e / 4, c->stream) : st;
    }));
    TRY(launch(c, "embed_fwd", 0.0, (double)B * C * (4 + e), [&] {
        return launch_embed_fwd(dt, ids, params, c->cfg.embed_norm ? xn : x, B, C, V, flag, c->stream);
    }));
    if (c->cfg.embed_norm) {
        TRY(launch(c, "rmsnorm_fwd", 0.0, (double)B * C * 2 * e, [&] {
            return launch_rmsnorm_fwd(dt, xn, x, c->at<float>(p.d_rstd), B, C, eps, c->stream);
        }));
    }
    // one B-row GEMM: split-K partials, then the finish (mode as launch_decode_finish)
    auto dgemm = [&](const char* tag, const void* A, int lda, const void* W, int N, int K, int mode, void* out,
                     const void* in, int rows) -> ncgpt_status {
        const DecSplit sp = decode_split(N, K);
        GemmDesc d;
        d.A = A; d.lda = lda; d.B = W; d.ldb = K;
        d.M = Bp; d.N = N; d.K = K;
        d.epi = Epi::SplitK; d.out = part; d.ldo = N;
        d.splits = sp.splits; d.k_split = sp.k_split; d.split_stride = (size_t)Bp * N;
        d.tile = 2; d.loop = GemmLoop::Ring8;
        TRY(gemm(c, d, tag));
        return launch(c, "decode_finish", 0.0, (double)Bp * N * 4 * (sp.splits + 1), [&] {
            return launch_decode_finish(dt, part, sp.splits, (size_t)Bp * N, rows, N, mode, out, in, c->stream,
                                        mode == 3 ? c->cap : SoftCap());
        });
    };
    const size_t cache_layer = (size_t)2 * B * c->Hkv * c->T * c->D * e;
    for (int l = 0; l < c->L; ++l) {
        uint8_t* cache = static_cast<uint8_t*>(kv_cache) + l * cache_layer;
        TRY(launch(c, "rmsnorm_fwd", 0.0, (double)Bp * C * 2 * e, [&] {
            return launch_rmsnorm_fwd(dt, x, xn, c->at<float>(p.d_rstd), Bp, C, eps, c->stream);
        }));
        TRY(dgemm("dec_qkv", xn, C, weight(c, l, 0), QKV, C, 0, qkv, nullptr, Bp));
        TRY(launch(c, "rope_qknorm_fwd", 0.0, (double)B * (c->H + c->Hkv) * c->D * 2 * e, [&] {
            return launch_rope_qknorm_fwd(dt, qkv, c->at<float>(p.d_rq), c->at<float>(p.d_rk), c->at<float>(p.cosv),
                                          c->at<float>(p.sinv), B, (int)c->T, (int)c->H, (int)c->Hkv, (int)c->D, eps,
                                          c->stream, pos);
        }));
        TRY(launch(c, "kv_store", 0.0, (double)B * 2 * c->KD * e * 2, [&] {
            return launch_kv_store(dt, qkv, cache, B, (int)c->H, (int)c->Hkv, (int)c->D, (int)c->T, pos, 1, 1,
                                   c->stream);
        }));
        TRY(launch(c, "decode_attn", 0.0, (double)B * c->Hkv * (pos + 1) * c->D * 2 * e, [&] {
            return launch_decode_attn(dt, qkv, cache, c->at<float>(p.d_attn), y, B, (int)c->H, (int)c->Hkv,
                                      (int)c->D, (int)c->T, pos, c->stream);
        }));
        TRY(dgemm("dec_attn_out", y, HD, weight(c, l, 3), C, HD, 1, x, x, Bp));
        TRY(launch(c, "rmsnorm_fwd", 0.0, (double)Bp * C * 2 * e, [&] {
            return launch_rmsnorm_fwd(dt, x, xn, c->at<float>(p.d_rstd), Bp, C, eps, c->stream);
        }));
        TRY(dgemm("dec_fc", xn, C, weight(c, l, 4), F, C, 2, act, nullptr, Bp));
        TRY(dgemm("dec_proj", act, F, weight(c, l, 5), C, F, 1, x, x, Bp));
    }
    TRY(launch(c, "rmsnorm_fwd", 0.0, (double)Bp * C * 2 * e, [&] {
        return launch_rmsnorm_fwd(dt, x, xn, c->at<float>(p.d_rstd), Bp, C, eps, c->stream);
    }));
    return dgemm("dec_lm_head", xn, C, weight(c, -1, 1), V, C, 3, logits, nullptr, B);
}

ncgpt_status ncgpt_check(ncgpt_ctx* c) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
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

ncgpt_status ncgpt_grads_finite(ncgpt_ctx* c, const float* x, size_t n, int32_t* ok) {
    if (!c) return NCGPT_EINVAL;
    TRY(check_bound(c));
    if (!x || !ok) return fail(c, NCGPT_EINVAL, "null values or flag");
    return launch(c, "grads_finite", 0.0, (double)n * 4, [&] { return launch_finite(x, n, ok, c->stream); });
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
    TRY(check_bound(c));
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
    case 10: src = c->ws + (c->cfg.embed_norm ? p.dxn : p.dx); dt = Dt::F32; break;
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
    release_static(c);
    for (auto& t : c->pending) {
        (void)hipEventDestroy(t.a);
        (void)hipEventDestroy(t.b);
    }
    for (auto ev : c->pool) (void)hipEventDestroy(ev);
    delete c;
}

}  // extern "C"
