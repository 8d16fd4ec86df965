// Internal launcher interface between the ncgpt runtime (runtime.hip) and the
// HIP kernels.  Not part of the public C ABI (that is include/ncgpt.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ncgpt {

enum class Dt : int { F32 = 0, BF16 = 1 };

// Device-side error bits, OR-ed into a flag word in the workspace and read by
// the host in ncgpt_check.
enum : uint32_t { kErrBadToken = 1u, kErrNoTargets = 2u, kErrBadTarget = 4u };

// ---------------------------------------------------------------- GEMM
// C[m][n] = sum_k A(m,k) * B(n,k), fp32 accumulation.
//   a_kcontig: A(m,k) = A[m*lda + k]  else A(m,k) = A[k*lda + m]
//   b_kcontig: B(n,k) = B[n*ldb + k]  else B(n,k) = B[k*ldb + n]
// Operands are bf16 in Dt::BF16 mode (MFMA kernel) and fp32 in Dt::F32 mode
// (SIMT kernel).  K must be a multiple of 64; M and N multiples of 8.
enum class Epi : int {
    StoreCd,     // out[m*ldo+n] = cd(v)
    StoreF32,    // out(f32)[m*ldo+n] = v
    ResidualCd,  // out[m*ldo+n] = cd(in[m*ldo+n] + v)        (in may equal out)
    ReluSq,      // out[m*ldo+n] = cd(a * a), a = cd(max(v, 0))   (the MLP activation act)
    ReluSqBwd,   // out[m*ldo+n] = cd(v * 2 * sqrt(in[m*ldo+n]))   (in = saved act; sqrt(act) recovers a to bf16 rounding)
    Grad,        // out(f32) = (accumulate ? out : 0) + v
    SplitK,      // out(f32)[split*split_stride + m*ldo + n] = v
};

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
    int tile = -1;    // MFMA tile: 0 = 256x256, 1 = 256x128, 2 = 128x128; -1 = chosen from the shape
    int group_m = 4;  // tiles are walked in bands of group_m tile-rows (L2 reuse of the B tiles)
    int variant = -1; // MFMA main loop: 0 = plain two-stage, 1 = software-pipelined, 2 = two register stages,
                      // 3 = software-pipelined with 8 waves, 4 = direct-to-LDS loads, 5 = the same with 8 waves,
                      // 6 = four-stage ring of 32-deep direct-to-LDS stages, 7 = the same with 8 waves,
                      // 8 = persistent four-stage ring, 9 = the same with 8 waves;
                      // -1 = the default (gemm_set_variant)
};

const char* gemm_kernel_name(const GemmDesc& d);
hipError_t launch_gemm(const GemmDesc& d, hipStream_t s);
// grads = (accumulate ? grads : 0) + sum_s part[s]   (n elements, n % 4 == 0)
hipError_t launch_splitk_reduce(const float* part, int splits, size_t stride, float* grads, size_t n,
                                int accumulate, hipStream_t s);
// MFMA kernels need more than the default 64 KB of dynamic LDS; call once per device.
hipError_t gemm_init_attributes();
// kernel variant of the bf16 GEMM (numbering as GemmDesc::variant; 9, the persistent 8-wave ring, is the default)
void gemm_set_variant(int v);

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
hipError_t attn_init_attributes();

// ---------------------------------------------------------------- row-wise / elementwise
hipError_t launch_cast_bf16(const float* src, void* dst, size_t n, hipStream_t s);
hipError_t launch_embed_fwd(Dt dt, const int32_t* ids, const float* wte, void* x, int N, int C, int V,
                            uint32_t* err, hipStream_t s);
hipError_t launch_rmsnorm_fwd(Dt dt, const void* x, void* y, float* rstd, int rows, int C, float eps,
                              hipStream_t s);
// dx(f32) = (accumulate ? dx : 0) + rstd*(dy - y*mean(dy*y)); dx_cd = cd(dx) when non-null
hipError_t launch_rmsnorm_bwd(Dt dt, const void* y, const float* rstd, const void* dy, float* dx, void* dx_cd,
                              int rows, int C, int accumulate, hipStream_t s);
hipError_t launch_rope_qknorm_fwd(Dt dt, void* qkv, float* rstdq, float* rstdk, const float* cosv,
                                  const float* sinv, int N, int T, int H, int Hkv, int D, float eps, hipStream_t s);
hipError_t launch_rope_qknorm_bwd(Dt dt, void* dqkv, const void* qkv, const float* rstdq, const float* rstdk,
                                  const float* cosv, const float* sinv, int N, int T, int H, int Hkv, int D,
                                  hipStream_t s);
hipError_t launch_ce_fwd_rows(Dt dt, const void* logits, const int32_t* targets, float* lse, float* loss_rows,
                              int N, int V, uint32_t* err, hipStream_t s);
hipError_t launch_loss_reduce(const float* loss_rows, const int32_t* targets, int N, int V, float* loss,
                              float* inv_valid, uint32_t* err, hipStream_t s);
hipError_t launch_ce_bwd(Dt dt, void* logits, const float* lse, const int32_t* targets, const float* inv_valid,
                         float grad_scale, int N, int V, hipStream_t s);
// dwte = (accumulate ? dwte : 0) + segment sums of dx rows by token id; deterministic.
// scratch: 4*N int32 + N*C f32 (the latter may alias any free [N,C] f32 buffer)
// iscratch: embed_bwd_scratch_ints(N, V) ints; partial: N x C floats; V <= 65536
size_t embed_bwd_scratch_ints(int N, int V);
hipError_t launch_embed_bwd(const int32_t* ids, const float* dx, float* dwte, int N, int C, int V, int accumulate,
                            int32_t* iscratch, float* partial, hipStream_t s);
hipError_t launch_to_f32(Dt dt, const void* src, float* dst, size_t n, hipStream_t s);

}  // namespace ncgpt
