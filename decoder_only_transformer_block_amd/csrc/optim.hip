// The optimizer step after the backward pass ("nanochat 项目深度分析" §2.2, §4.2): Muon for every layer
// matrix, AdamW for the embedding and the unembedding.  The Newton-Schulz iteration runs on the bf16 MFMA
// GEMMs (batched over the matrices of one shape); the element-wise parts are below.
//
// Muon, in the form of the published Muon description (K. Jordan et al., 2024):
//   buf = mu buf + (1 - mu) g,   u = (1 - mu) g + mu buf (Nesterov) or buf,
//   X0 = bf16(u / max(||u||_F, eps)),   5 x { A = X X^T (X^T X for a tall matrix), B = b A + c A A,
//   X = a X + B X (X B) },   p = p (1 - lr wd) - lr sqrt(max(1, rows / cols)) X.
// AdamW: Loshchilov and Hutter's decoupled weight decay with bias-corrected moments.
#include "common.h"
#include "kernels.h"

namespace ncgpt {

// Every layer matrix has a multiple of 4096 elements (each of its dimensions is a multiple of 64), so a
// chunk of 4096 consecutive elements of the packed matrix range lies inside one matrix.
constexpr int kChunk = 4096;

// buf = mu buf + (1 - mu) g over the whole matrix range, and per chunk the sum of u^2 (u the Muon update
// direction), summed in a fixed order.
__global__ void __launch_bounds__(256)
muon_momentum_kernel(const float* __restrict__ g, float* __restrict__ buf, float* __restrict__ part, float mu,
                     int nesterov)
{
    __shared__ float red[4];
    const size_t base = (size_t)blockIdx.x * kChunk;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunk / (256 * 4); ++i) {
        const size_t o = base + (size_t)(i * 256 + threadIdx.x) * 4;
        float gv[4], bv[4];
        Vec4<float>::load(g + o, gv);
        Vec4<float>::load(buf + o, bv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[e] = mu * bv[e] + (1.0f - mu) * gv[e];
            const float u = nesterov ? (1.0f - mu) * gv[e] + mu * bv[e] : bv[e];
            ss += u * u;
        }
        Vec4<float>::store(buf + o, bv);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// inv[m] = 1 / max(||u_m||_F, eps) for matrix m = (layer, which): its chunks' partial sums in order.
__global__ void __launch_bounds__(64)
muon_norm_kernel(const float* __restrict__ part, float* __restrict__ inv, MuonShapes sh, float eps)
{
    const int layer = blockIdx.x / 6, w = blockIdx.x % 6;
    const int64_t first = ((int64_t)layer * sh.layer + sh.off[w]) / kChunk, n = sh.size[w] / kChunk;
    float s = 0.0f;
    for (int64_t c = threadIdx.x; c < n; c += 64) s += part[first + c];
    s = wave_sum(s);
    if (threadIdx.x == 0) inv[blockIdx.x] = 1.0f / fmaxf(sqrtf(s), eps);
}

// X0 of matrix (layer = blockIdx.y, which w): bf16(u * inv), into the batch slot of its shape group.
__global__ void __launch_bounds__(256)
muon_init_kernel(const float* __restrict__ g, const float* __restrict__ buf, const float* __restrict__ inv,
                 bf16* __restrict__ x, MuonShapes sh, int w, float mu, int nesterov)
{
    const int layer = blockIdx.y;
    const size_t src = (size_t)layer * sh.layer + sh.off[w];
    bf16* dst = x + ((size_t)layer * sh.group_count[w] + sh.group_slot[w]) * (size_t)sh.size[w];
    const float k = inv[layer * 6 + w];
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)sh.size[w]) return;
    float gv[4], bv[4], u[4];
    Vec4<float>::load(g + src + i, gv);
    Vec4<float>::load(buf + src + i, bv);
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (nesterov ? (1.0f - mu) * gv[e] + mu * bv[e] : bv[e]) * k;
    Vec4<bf16>::store(dst + i, u);
}

// p = p (1 - lr wd) - lr_scaled X for matrix (layer = blockIdx.y, which w).
__global__ void __launch_bounds__(256)
muon_apply_kernel(float* __restrict__ p, const bf16* __restrict__ x, MuonShapes sh, int w, float decay, float step)
{
    const int layer = blockIdx.y;
    const size_t dst = (size_t)layer * sh.layer + sh.off[w];
    const bf16* src = x + ((size_t)layer * sh.group_count[w] + sh.group_slot[w]) * (size_t)sh.size[w];
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)sh.size[w]) return;
    float pv[4], xv[4];
    Vec4<float>::load(p + dst + i, pv);
    Vec4<bf16>::load(src + i, xv);
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = pv[e] * decay - step * xv[e];
    Vec4<float>::store(p + dst + i, pv);
}

// AdamW on n parameters: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
// p = p (1 - lr wd) - lr (m / bc1) / (sqrt(v / bc2) + eps).
__global__ void __launch_bounds__(256)
adamw_kernel(float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m, float* __restrict__ v,
             size_t n4, AdamArgs a)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) {
        float pv[4], gv[4], mv[4], vv[4];
        Vec4<float>::load(p + 4 * i, pv);
        Vec4<float>::load(g + 4 * i, gv);
        Vec4<float>::load(m + 4 * i, mv);
        Vec4<float>::load(v + 4 * i, vv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mv[e] = a.b1 * mv[e] + (1.0f - a.b1) * gv[e];
            vv[e] = a.b2 * vv[e] + (1.0f - a.b2) * gv[e] * gv[e];
            const float mh = mv[e] / a.bc1, vh = vv[e] / a.bc2;
            pv[e] = pv[e] * a.decay - a.lr * mh / (sqrtf(vh) + a.eps);
        }
        Vec4<float>::store(p + 4 * i, pv);
        Vec4<float>::store(m + 4 * i, mv);
        Vec4<float>::store(v + 4 * i, vv);
    }
}

hipError_t launch_muon_momentum(const float* g, float* buf, float* part, size_t n, float mu, int nesterov,
                                hipStream_t s) {
    if (n % kChunk) return hipErrorInvalidValue;
    hipLaunchKernelGGL(muon_momentum_kernel, dim3((unsigned)(n / kChunk)), dim3(256), 0, s, g, buf, part, mu, nesterov);
    return hipGetLastError();
}

hipError_t launch_muon_norm(const float* part, float* inv, const MuonShapes& sh, int layers, float eps, hipStream_t s) {
    for (int w = 0; w < 6; ++w)
        if (sh.size[w] % kChunk || sh.off[w] % kChunk) return hipErrorInvalidValue;
    if (sh.layer % kChunk) return hipErrorInvalidValue;
    hipLaunchKernelGGL(muon_norm_kernel, dim3(layers * 6), dim3(64), 0, s, part, inv, sh, eps);
    return hipGetLastError();
}

hipError_t launch_muon_init(const float* g, const float* buf, const float* inv, void* x, const MuonShapes& sh, int w,
                            int layers, float mu, int nesterov, hipStream_t s) {
    const dim3 grid((unsigned)((sh.size[w] / 4 + 255) / 256), layers);
    hipLaunchKernelGGL(muon_init_kernel, grid, dim3(256), 0, s, g, buf, inv, (bf16*)x, sh, w, mu, nesterov);
    return hipGetLastError();
}

hipError_t launch_muon_apply(float* p, const void* x, const MuonShapes& sh, int w, int layers, float decay, float step,
                             hipStream_t s) {
    const dim3 grid((unsigned)((sh.size[w] / 4 + 255) / 256), layers);
    hipLaunchKernelGGL(muon_apply_kernel, grid, dim3(256), 0, s, p, (const bf16*)x, sh, w, decay, step);
    return hipGetLastError();
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, size_t n, const AdamArgs& a, hipStream_t s) {
    if (n % 4) return hipErrorInvalidValue;
    const size_t n4 = n / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 256 * 32);
    hipLaunchKernelGGL(adamw_kernel, dim3(blocks), dim3(256), 0, s, p, g, m, v, n4, a);
    return hipGetLastError();
}

}  // namespace ncgpt
