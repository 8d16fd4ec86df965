// Internal launcher interface between the ncgpt runtime (runtime.hip) and the
// HIP kernels.  Not part of the public C ABI (that is include/ncgpt.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ncgpt {

enum class Dt : int { F32 = 0, BF16 = 1, F16 = 2 };
// the 16-bit compute dtypes share the MFMA path (bf16, or fp16 with loss scaling)
inline bool mfma_dt(Dt d) { return d != Dt::F32; }

// Device-side error bits, OR-ed into a flag word in the workspace and read by
// the host in ncgpt_check.
enum : uint32_t { kErrBadToken = 1u, kErrNoTargets = 2u, kErrBadTarget = 4u };

// Logit soft-cap z -> c tanh(z / c) (off when c == 0).  The constants are formed once on the host, so every
// kernel that caps or differentiates a logit uses the same float values: k = 2 log2(e) / c, ic = 1 / c.
struct SoftCap {
    float c = 0.0f, c2 = 0.0f, k = 0.0f, ic = 0.0f;
};
inline SoftCap make_softcap(float c) {
    SoftCap s;
    if (c > 0.0f) {
        s.c = c;
        s.c2 = 2.0f * c;
        s.k = (float)(2.0 * 1.4426950408889634 / (double)c);
        s.ic = (float)(1.0 / (double)c);
    }
    return s;
}

// ---------------------------------------------------------------- GEMM
// C[m][n] = sum_k A(m,k) * B(n,k), fp32 accumulation.
//   a_kcontig: A(m,k) = A[m*lda + k]  else A(m,k) = A[k*lda + m]
//   b_kcontig: B(n,k) = B[n*ldb + k]  else B(n,k) = B[k*ldb + n]
// Operands are bf16 in Dt::BF16 mode (MFMA kernel) and fp32 in Dt::F32 mode
// (SIMT kernel).  K must be a multiple of 64; M and N multiples of 8.
enum class Epi : int {
    StoreCd,     // out[m*ldo+n] = cd(v)
    ResidualCd,  // out[m*ldo+n] = cd(in[m*ldo+n] + v)        (in may equal out)
    ReluSq,      // out[m*ldo+n] = cd(a * a), a = cd(max(v, 0))   (the MLP activation act)
    ReluSqBwd,   // out[m*ldo+n] = cd(v * 2 * sqrt(in[m*ldo+n]))   (in = saved act; sqrt(act) recovers a to bf16 rounding)
    Grad,        // out(f32) = (accumulate ? out : 0) + v
    SplitK,      // out(f32)[split*split_stride + m*ldo + n] = v
    CeStats,     // bf16 LM head: per row and wave column block the (max, sum) of the softmax in the log2
                 // domain (part), the logit at the row's target (zt); the rounded logits too when out != 0;
                 // with a soft-cap every logit is capped first (and stored capped)
    Dz,          // bf16 LM head recomputed in the backward: out = bf16(scale (softmax(z) - onehot(target))),
                 // scale = grad_scale * inv_valid on rows with a valid target, 0 elsewhere; with a soft-cap
                 // z is the capped logit and the result is multiplied by 1 - (z / c)^2
    Axpby,       // bf16: out = cd(alpha in + beta v) (the Newton-Schulz steps); NN layout, batches allowed
    RopeNorm,    // bf16 qkv projection (head_dim 128, Persist8Heads, 256 x 256 tiles): q and k heads rotated
                 // (RoPE) and RMS-normalised over the head, 1/rms saved; v heads stored as they are
};

// MFMA main loop (all three stream 32-deep stages straight into a four-stage LDS ring):
//   Ring8    eight waves, one output tile per workgroup;
//   Persist4 four waves, persistent (the grid is the resident workgroups, walking (split, tile) items);
//   Persist8 eight waves, persistent;
//   Persist8Heads eight waves, persistent, in a 4 x 2 grid: on a 256 x 256 tile each wave owns 64 rows x 128
//            columns, i.e. whole attention heads of the qkv projection (the RopeNorm epilogue needs that).
enum class GemmLoop : int { Ring8 = 0, Persist4 = 1, Persist8 = 2, Persist8Heads = 3 };

struct GemmDesc {
    Dt dt = Dt::BF16;
    const void* A = nullptr;
    const void* B = nullptr;
    int lda = 0, ldb = 0;
    bool a_kcontig = true, b_kcontig = true;
    int M = 0, N = 0, K = 0;
    Epi epi = Epi::StoreCd;
    void* out = nullptr;
    const void* in = nullptr;
    int ldo = 0;
    int accumulate = 0;
    int splits = 1;         // split-K: K is cut into ceil(K / k_split) ranges of k_split (grid.y)
    int k_split = 0;        // multiple of 64; 0 = K / splits
    size_t split_stride = 0;
    // LM-head epilogues (CeStats, Dz)
    void* part = nullptr;            // float2 [nblk][M]
    int nblk = 0;                    // column blocks per row = ceil(N / gemm_wave_cols)
    float* zt = nullptr;             // [M]
    const int32_t* targets = nullptr;
    const float* lse = nullptr;      // [M] natural-log LSE (Dz)
    const float* inv_valid = nullptr;
    float grad_scale = 1.0f;
    SoftCap cap;                     // logit soft-cap (CeStats, Dz)
    // RopeNorm epilogue
    const float* cosv = nullptr;     // [T, 64] rotation tables
    const float* sinv = nullptr;
    float* rstdq = nullptr;          // [M, H]
    float* rstdk = nullptr;          // [M, Hkv]
    int T = 0, H = 0, Hkv = 0;
    float eps = 0.0f;
    // Axpby epilogue
    float alpha = 0.0f, beta = 1.0f;
    // batched GEMM (the Ring8 loop only; StoreCd and Axpby epilogues): item z reads A + z sA and B + z sB and
    // writes out + z sOut (reading in + z sIn); strides in elements
    int batch = 1;
    int64_t sA = 0, sB = 0, sOut = 0, sIn = 0;
    // fp8 operands (bf16 mode, NT layout, the forward epilogues): A [M, K] and B [N, K] hold OCP E4M3 bytes, K,
    // lda and ldb count bytes; the product is multiplied by rsa[m] rsb[n] (per-row scales) before the epilogue
    bool fp8 = false;
    const float* rsa = nullptr;
    const float* rsb = nullptr;
    int tile = -1;    // MFMA tile: 0 = 256x256, 1 = 256x128, 2 = 128x128; -1 = chosen from the shape
    int group_m = 4;  // tiles are walked in bands of group_m tile-rows (L2 reuse of the B tiles)
    GemmLoop loop = GemmLoop::Persist8;
};

const char* gemm_kernel_name(const GemmDesc& d);
// columns of one wave's share of an output tile (the CeStats column block) for d's tile and loop
int gemm_wave_cols(const GemmDesc& d);
hipError_t launch_gemm(const GemmDesc& d, hipStream_t s);
// grads = (accumulate ? grads : 0) + sum_s part[s]   (n elements, n % 4 == 0)
hipError_t launch_splitk_reduce(const float* part, int splits, size_t stride, float* grads, size_t n,
                                int accumulate, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnDesc {
    Dt dt = Dt::BF16;
    int B = 0, T = 0, H = 0, Hkv = 0, D = 0;
    const void* qkv = nullptr;  // [B*T, (H+2Hkv)*D] cd: q | k | v
    void* y = nullptr;          // [B*T, H*D] cd
    float* lse = nullptr;       // [B, H, T] natural-log LSE of the scaled scores
    const void* dy = nullptr;   // [B*T, H*D] cd (backward)
    void* dqkv = nullptr;       // [B*T, (H+2Hkv)*D] cd (backward)
    float* delta = nullptr;     // [2, B, H, T] scratch (backward): delta, then (bf16) the LSE in log2 units
    // bf16 backward only: the RoPE + QK-norm backward is applied to dq and dk before they are stored
    const float* rstdq = nullptr;  // [B*T, H] saved 1/rms of the rotated q heads
    const float* rstdk = nullptr;  // [B*T, Hkv]
    const float* cosv = nullptr;   // [T, D/2] rotation tables
    const float* sinv = nullptr;
};
hipError_t launch_attn_fwd(const AttnDesc& a, hipStream_t s);
// part 0: dQ (and delta = rowsum(dy * y), which part 1 reads); part 1: dK, dV -- in this order.  In bf16
// the q and k gradients leave already taken back through QK-norm and RoPE (rstdq/rstdk/cosv/sinv).
hipError_t launch_attn_bwd(const AttnDesc& a, hipStream_t s, int part);

// ---------------------------------------------------------------- row-wise / elementwise
// fp32 -> the 16-bit compute dtype (bf16, or fp16 for Dt::F16), round to nearest even
hipError_t launch_cast_bf16(const float* src, void* dst, size_t n, hipStream_t s, Dt dt = Dt::BF16);
hipError_t launch_embed_fwd(Dt dt, const int32_t* ids, const float* wte, void* x, int N, int C, int V,
                            uint32_t* err, hipStream_t s);
// q8 non-null (bf16, C a multiple of 256 up to 2048): the stored rows also as E4M3 bytes with scales qs (the
// row quantiser's result for y)
hipError_t launch_rmsnorm_fwd(Dt dt, const void* x, void* y, float* rstd, int rows, int C, float eps,
                              hipStream_t s, void* q8 = nullptr, float* qs = nullptr);
// g = acc + rstd*(dy - y*mean(dy*y)) with acc = 0 (accumulate 0), the fp32 dx (1) or dx_cd (2); g is written
// to dx (fp32) and to dx_cd (compute dtype), each when non-null
hipError_t launch_rmsnorm_bwd(Dt dt, const void* y, const float* rstd, const void* dy, float* dx, void* dx_cd,
                              int rows, int C, int accumulate, hipStream_t s);
// pos >= 0: every row is one token at position pos (decode); else row n is at position n mod T
hipError_t launch_rope_qknorm_fwd(Dt dt, void* qkv, float* rstdq, float* rstdk, const float* cosv,
                                  const float* sinv, int N, int T, int H, int Hkv, int D, float eps, hipStream_t s,
                                  int pos = -1);
hipError_t launch_rope_qknorm_bwd(Dt dt, void* dqkv, const void* qkv, const float* rstdq, const float* rstdk,
                                  const float* cosv, const float* sinv, int N, int T, int H, int Hkv, int D,
                                  hipStream_t s);
hipError_t launch_ce_fwd_rows(Dt dt, const void* logits, const int32_t* targets, float* lse, float* loss_rows,
                              int N, int V, uint32_t* err, hipStream_t s);
// lse and per-row loss from the LM-head epilogue's partials (CeStats)
hipError_t launch_ce_merge(const void* part, int nblk, const float* zt, const int32_t* targets, float* lse,
                           float* loss_rows, int N, int V, uint32_t* err, hipStream_t s);
hipError_t launch_loss_reduce(const float* loss_rows, const int32_t* targets, int N, int V, float* loss,
                              float* inv_valid, uint32_t* err, hipStream_t s);
// logits already capped when cap.c > 0: the gradient is multiplied by 1 - (z / c)^2
hipError_t launch_ce_bwd(Dt dt, void* logits, const float* lse, const int32_t* targets, const float* inv_valid,
                         float grad_scale, const SoftCap& cap, int N, int V, hipStream_t s);
// z = c tanh(z / c) in place (n % 4 == 0)
hipError_t launch_softcap(Dt dt, void* z, size_t n, const SoftCap& cap, hipStream_t s);
// dwte = (accumulate ? dwte : 0) + segment sums of dx rows by token id; deterministic.
// scratch: 4*N int32 + N*C f32 (the latter may alias any free [N,C] f32 buffer)
// iscratch: embed_bwd_scratch_ints(N, V) ints; partial: N x C floats; V <= 65536
size_t embed_bwd_scratch_ints(int N, int V);
hipError_t launch_embed_bwd(const int32_t* ids, const float* dx, float* dwte, int N, int C, int V, int accumulate,
                            int32_t* iscratch, float* partial, hipStream_t s);
hipError_t launch_to_f32(Dt dt, const void* src, float* dst, size_t n, hipStream_t s);
// fp8 (E4M3) rows with per-row scales: q[l][r][:] = x[l][r][:] / s[l][r], s = amax / 448, for `layers` matrices of
// rows x cols at element strides x_layer, q_layer, s_layer; src is the element type of x (BF16 or F32)
hipError_t launch_quant_rows_fp8(Dt src, const void* x, size_t x_layer, void* q, size_t q_layer, float* s,
                                 size_t s_layer, int rows, int cols, int layers, hipStream_t st);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s);
// *ok = 1 if all n values are finite, else 0
hipError_t launch_finite(const float* x, size_t n, int32_t* ok, hipStream_t s);

// ---------------------------------------------------------------- KV-cache decode (decode.hip)
// cache of one layer: [2][B][Hkv][Tc][D]; stores k and v heads of qkv rows b * rb + (t - t0), t in [t0, t0 + nt)
hipError_t launch_kv_store(Dt dt, const void* qkv, void* cache, int B, int H, int Hkv, int D, int Tc, int t0, int nt,
                           int rb, hipStream_t s);
// y [B, H*D] = attention of the q heads of qkv rows b (one token per sequence, at position pos) over cache
// positions 0..pos; part: decode_attn_part_floats(B, H, D, Tc) floats of scratch
size_t decode_attn_part_floats(int B, int H, int D, int Tc);
hipError_t launch_decode_attn(Dt dt, const void* qkv, const void* cache, float* part, void* y, int B, int H, int Hkv,
                              int D, int Tc, int pos, hipStream_t s);
// sum of split-K partials part[s][m][n] (s < splits, stride = elements per split) over rows m < rows:
// mode 0 store, 1 residual add (out = in + v), 2 the MLP activation relu(v)^2, 3 fp32 store (soft-capped
// when cap.c > 0: the logits)
hipError_t launch_decode_finish(Dt dt, const float* part, int splits, size_t stride, int rows, int N, int mode,
                                void* out, const void* in, hipStream_t s, const SoftCap& cap = SoftCap());

// ---------------------------------------------------------------- optimizer step (optim.hip)
// The six matrices of a layer (Wq, Wk, Wv, Wo, Wfc, Wproj) inside the packed matrix range: layer stride,
// offset and size of each, and its place in the Newton-Schulz batch of its shape (matrices of equal shape
// form one batch: layer-major, group_count per layer, this one at group_slot).
struct MuonShapes {
    int64_t layer;
    int64_t off[6], size[6];
    int group_count[6], group_slot[6];
};
struct AdamArgs {
    float lr, b1, b2, eps, bc1, bc2, decay;
};
// buf = mu buf + (1 - mu) g over the n-element matrix range (n % 4096 == 0); part[n / 4096] chunk sums of u^2
hipError_t launch_muon_momentum(const float* g, float* buf, float* part, size_t n, float mu, int nesterov,
                                hipStream_t s);
// inv[layer * 6 + w] = 1 / max(||u||_F, eps)
hipError_t launch_muon_norm(const float* part, float* inv, const MuonShapes& sh, int layers, float eps, hipStream_t s);
// x (bf16, the shape group of matrix w): u * inv for every layer
hipError_t launch_muon_init(const float* g, const float* buf, const float* inv, void* x, const MuonShapes& sh, int w,
                            int layers, float mu, int nesterov, hipStream_t s);
// p = p decay - step x for matrix w of every layer
hipError_t launch_muon_apply(float* p, const void* x, const MuonShapes& sh, int w, int layers, float decay, float step,
                             hipStream_t s);
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, size_t n, const AdamArgs& a, hipStream_t s);

}  // namespace ncgpt
