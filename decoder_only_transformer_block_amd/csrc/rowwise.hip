// Bandwidth-bound kernels of the step: weight cast, embedding gather and its
// gradient, parameter-free RMSNorm, RoPE + QK-norm, and the cross-entropy
// pieces.  Storage type T is the compute dtype (float, bf16 or fp16); all
// arithmetic is fp32.
#include "common.h"
#include "kernels.h"

namespace ncgpt {

// ------------------------------------------------------------------ fp32 master -> bf16 (RNE)
// The precision scheme keeps fp32 master weights and casts them to the compute
// dtype inside each linear ("nanochat：低成本跑通大模型训练全流程", precision paragraph).
__global__ void __launch_bounds__(256) cast_bf16_kernel(const float* __restrict__ src, bf16* __restrict__ dst, size_t n4)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) {
        float v[4];
        Vec4<float>::load(src + 4 * i, v);
        Vec4<bf16>::store(dst + 4 * i, v);
    }
}

__global__ void __launch_bounds__(256) cast_f16_kernel(const float* __restrict__ src, f16* __restrict__ dst, size_t n4)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) {
        float v[4];
        Vec4<float>::load(src + 4 * i, v);
        Vec4<f16>::store(dst + 4 * i, v);
    }
}

hipError_t launch_cast_bf16(const float* src, void* dst, size_t n, hipStream_t s, Dt dt) {
    size_t n4 = n / 4;
    unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 256 * 64);
    if (dt == Dt::F16)
        hipLaunchKernelGGL(cast_f16_kernel, dim3(blocks), dim3(256), 0, s, src, (f16*)dst, n4);
    else
        hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, (bf16*)dst, n4);
    return hipGetLastError();
}

// ------------------------------------------------------------------ embedding gather
// x[n] = cd(wte[ids[n]]); an id outside [0, V) raises kErrBadToken and yields a zero row.
template <typename T>
__global__ void __launch_bounds__(256)
embed_fwd_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wte, T* __restrict__ x, int N, int C, int V,
                 uint32_t* err)
{
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (n >= N) return;
    const int id = ids[n];
    const bool ok = id >= 0 && id < V;
    if (!ok && lane == 0) raise_error(err, kErrBadToken);
    for (int c = lane * 4; c < C; c += 256) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) Vec4<float>::load(wte + (size_t)id * C + c, v);
        Vec4<T>::store(x + (size_t)n * C + c, v);
    }
}

hipError_t launch_embed_fwd(Dt dt, const int32_t* ids, const float* wte, void* x, int N, int C, int V, uint32_t* err,
                            hipStream_t s) {
    dim3 grid((N + 3) / 4);
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(embed_fwd_kernel<bf16>, grid, dim3(256), 0, s, ids, wte, (bf16*)x, N, C, V, err);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(embed_fwd_kernel<f16>, grid, dim3(256), 0, s, ids, wte, (f16*)x, N, C, V, err);
    else
        hipLaunchKernelGGL(embed_fwd_kernel<float>, grid, dim3(256), 0, s, ids, wte, (float*)x, N, C, V, err);
    return hipGetLastError();
}

// ---- row helpers: sums over lane groups, 8-element (16-byte in bf16) loads and stores
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// 8 values -> 8 E4M3 bytes (x inv), round to nearest even
__device__ __forceinline__ uint2 fp8x8(const float (&v)[8], float inv) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int t = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h] * inv, v[4 * h + 1] * inv, 0, false);
        t = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h + 2] * inv, v[4 * h + 3] * inv, t, true);
        w[h] = (uint32_t)t;
    }
    return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void load8(const f16* p, float (&v)[8]) {
    const f16x8 a = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}
__device__ __forceinline__ void store8(f16* p, const float (&v)[8]) {
    f16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (f16)v[e];
    *reinterpret_cast<f16x8*>(p) = a;
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(p) = a;
}


// ------------------------------------------------------------------ RMSNorm (one wave per row)
// y = x / sqrt(mean(x^2) + eps), no weight ("nanochat 项目深度分析" §2.1 item 5).
template <typename T>
__global__ void __launch_bounds__(256)
rmsnorm_fwd_kernel(const T* __restrict__ x, T* __restrict__ y, float* __restrict__ rstd, int rows, int C, float eps)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const T* xr = x + (size_t)row * C;
    float ss = 0.0f;
    for (int c = lane * 4; c < C; c += 256) {
        float v[4];
        Vec4<T>::load(xr + c, v);
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)C + eps);
    T* yr = y + (size_t)row * C;
    for (int c = lane * 4; c < C; c += 256) {
        float v[4];
        Vec4<T>::load(xr + c, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= rs;
        Vec4<T>::store(yr + c, v);
    }
    if (lane == 0) rstd[row] = rs;
}

// The same map with each row held in registers (C = 256 NCH): 32 lanes per row, two rows
// per wave; lane j holds the 8-element chunks j, j + 32, ..., j + 32 (NCH - 1), so every
// access is 16 bytes wide in bf16, every load is issued before the reduction, and x is
// read once.  With q non-null the stored row (as rounded to T) also leaves as E4M3 bytes with
// the row scale qs = amax / 448, exactly as the row quantiser below would make them from y.
template <typename T, int NCH>
__global__ void __launch_bounds__(256)
rmsnorm_fwd_rows(const T* __restrict__ x, T* __restrict__ y, float* __restrict__ rstd, int rows, int C, float eps,
                 uint8_t* __restrict__ q, float* __restrict__ qs)
{
    const int row = blockIdx.x * 8 + (threadIdx.x >> 5), j = threadIdx.x & 31;
    const bool live = row < rows;               // no early return: the lane-group sums stay uniform
    const size_t base = (size_t)(live ? row : 0) * C + 8 * j;
    float v[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) load8(x + base + 256 * i, v[i]);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
    ss = group_sum<32>(ss);
    const float rs = 1.0f / sqrtf(ss / (float)C + eps);
    if (q) {                                     // uniform
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[i][e] = to_f32(from_f32<T>(v[i][e] * rs));   // the value y stores
                amax = fmaxf(amax, fabsf(v[i][e]));
            }
        amax = group_max<32>(amax);
        if (!live) return;
        const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            store8(y + base + 256 * i, v[i]);
            *reinterpret_cast<uint2*>(q + base + 256 * i) = fp8x8(v[i], inv);
        }
        if (j == 0) {
            rstd[row] = rs;
            qs[row] = amax > 0.0f ? amax / 448.0f : 1.0f;
        }
        return;
    }
    if (!live) return;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] *= rs;
        store8(y + base + 256 * i, v[i]);
    }
    if (j == 0) rstd[row] = rs;
}

template <typename T>
static bool rmsnorm_fwd_rows_launch(const void* x, void* y, float* rstd, int rows, int C, float eps, uint8_t* q,
                                    float* qs, hipStream_t s) {
    const dim3 grid((rows + 7) / 8);
    switch (C % 256 ? 0 : C / 256) {
#define NCGPT_RMS_F(n)                                                                                              \
    case n:                                                                                                          \
        hipLaunchKernelGGL((rmsnorm_fwd_rows<T, n>), grid, dim3(256), 0, s, (const T*)x, (T*)y, rstd, rows, C, eps,  \
                           q, qs);                                                                                   \
        return true;
    NCGPT_RMS_F(1) NCGPT_RMS_F(2) NCGPT_RMS_F(3) NCGPT_RMS_F(4) NCGPT_RMS_F(5) NCGPT_RMS_F(6) NCGPT_RMS_F(8)
#undef NCGPT_RMS_F
    default: return false;
    }
}

hipError_t launch_rmsnorm_fwd(Dt dt, const void* x, void* y, float* rstd, int rows, int C, float eps, hipStream_t s,
                              void* q8, float* qs) {
    if (q8 && (dt != Dt::BF16 || !qs)) return hipErrorInvalidValue;
    if (dt == Dt::BF16  ? rmsnorm_fwd_rows_launch<bf16>(x, y, rstd, rows, C, eps, (uint8_t*)q8, qs, s)
        : dt == Dt::F16 ? rmsnorm_fwd_rows_launch<f16>(x, y, rstd, rows, C, eps, nullptr, nullptr, s)
                        : rmsnorm_fwd_rows_launch<float>(x, y, rstd, rows, C, eps, nullptr, nullptr, s))
        return hipGetLastError();
    if (q8) return hipErrorInvalidValue;       // the E4M3 copy comes only from the register-row kernel
    dim3 grid((rows + 3) / 4);
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, (bf16*)y, rstd, rows, C, eps);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(rmsnorm_fwd_kernel<f16>, grid, dim3(256), 0, s, (const f16*)x, (f16*)y, rstd, rows, C, eps);
    else
        hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, grid, dim3(256), 0, s, (const float*)x, (float*)y, rstd, rows, C,
                           eps);
    return hipGetLastError();
}

// Derivative of the map above, from its saved output y and scale rstd:
// dx = rstd * (dy - y * mean(dy * y)).
// dy arrives in the compute dtype.  The residual-stream gradient it adds to is read from dx (fp32,
// accumulate = 1) or dx_cd (the compute dtype, accumulate = 2), or starts at 0 (accumulate = 0); the sum is
// written to whichever of dx and dx_cd is given.
template <typename T>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_kernel(const T* __restrict__ y, const float* __restrict__ rstd, const T* __restrict__ dy,
                   float* __restrict__ dx, T* __restrict__ dx_cd, int rows, int C, int accumulate)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const size_t base = (size_t)row * C;
    float dot = 0.0f;
    for (int c = lane * 4; c < C; c += 256) {
        float a[4], b[4];
        Vec4<T>::load(y + base + c, a);
        Vec4<T>::load(dy + base + c, b);
        dot += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
    }
    dot = wave_sum(dot) / (float)C;
    const float rs = rstd[row];
    for (int c = lane * 4; c < C; c += 256) {
        float a[4], b[4], o[4] = {0.f, 0.f, 0.f, 0.f};
        Vec4<T>::load(y + base + c, a);
        Vec4<T>::load(dy + base + c, b);
        if (accumulate == 1) Vec4<float>::load(dx + base + c, o);
        else if (accumulate == 2) Vec4<T>::load(dx_cd + base + c, o);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] += rs * (b[i] - a[i] * dot);
        if (dx) Vec4<float>::store(dx + base + c, o);
        if (dx_cd) Vec4<T>::store(dx_cd + base + c, o);
    }
}

// The same derivative with each row held in registers, laid out as in rmsnorm_fwd_rows.
template <typename T, int NCH>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_rows(const T* __restrict__ y, const float* __restrict__ rstd, const T* __restrict__ dy,
                 float* __restrict__ dx, T* __restrict__ dx_cd, int rows, int C, int accumulate)
{
    const int row = blockIdx.x * 8 + (threadIdx.x >> 5), j = threadIdx.x & 31;
    const bool live = row < rows;
    const int rr = live ? row : 0;
    const size_t base = (size_t)rr * C + 8 * j;
    float a[NCH][8], b[NCH][8], o[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        load8(y + base + 256 * i, a[i]);
        load8(dy + base + 256 * i, b[i]);
        if (accumulate == 1) {
            load8(dx + base + 256 * i, o[i]);
        } else if (accumulate == 2) {
            load8(dx_cd + base + 256 * i, o[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e] = 0.0f;
        }
    }
    const float rs = rstd[rr];
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += a[i][e] * b[i][e];
    dot = group_sum<32>(dot) / (float)C;
    if (!live) return;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] += rs * (b[i][e] - a[i][e] * dot);
        if (dx) store8(dx + base + 256 * i, o[i]);
        if (dx_cd) store8(dx_cd + base + 256 * i, o[i]);
    }
}

template <typename T>
static bool rmsnorm_bwd_rows_launch(const void* y, const float* rstd, const void* dy, float* dx, void* dx_cd,
                                    int rows, int C, int accumulate, hipStream_t s) {
    const dim3 grid((rows + 7) / 8);
    switch (C % 256 ? 0 : C / 256) {
#define NCGPT_RMS_B(n)                                                                                          \
    case n:                                                                                                      \
        hipLaunchKernelGGL((rmsnorm_bwd_rows<T, n>), grid, dim3(256), 0, s, (const T*)y, rstd, (const T*)dy, dx, \
                           (T*)dx_cd, rows, C, accumulate);                                                      \
        return true;
    NCGPT_RMS_B(1) NCGPT_RMS_B(2) NCGPT_RMS_B(3) NCGPT_RMS_B(4) NCGPT_RMS_B(5) NCGPT_RMS_B(6) NCGPT_RMS_B(8)
#undef NCGPT_RMS_B
    default: return false;
    }
}

hipError_t launch_rmsnorm_bwd(Dt dt, const void* y, const float* rstd, const void* dy, float* dx, void* dx_cd,
                              int rows, int C, int accumulate, hipStream_t s) {
    if (dt == Dt::BF16  ? rmsnorm_bwd_rows_launch<bf16>(y, rstd, dy, dx, dx_cd, rows, C, accumulate, s)
        : dt == Dt::F16 ? rmsnorm_bwd_rows_launch<f16>(y, rstd, dy, dx, dx_cd, rows, C, accumulate, s)
                        : rmsnorm_bwd_rows_launch<float>(y, rstd, dy, dx, dx_cd, rows, C, accumulate, s))
        return hipGetLastError();
    dim3 grid((rows + 3) / 4);
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)y, rstd, (const bf16*)dy, dx,
                           (bf16*)dx_cd, rows, C, accumulate);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(rmsnorm_bwd_kernel<f16>, grid, dim3(256), 0, s, (const f16*)y, rstd, (const f16*)dy, dx,
                           (f16*)dx_cd, rows, C, accumulate);
    else
        hipLaunchKernelGGL(rmsnorm_bwd_kernel<float>, grid, dim3(256), 0, s, (const float*)y, rstd, (const float*)dy,
                           dx, (float*)dx_cd, rows, C, accumulate);
    return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE + QK-norm
// For each token n (position t = n mod T) and each q and k head: rotate pair
// (i, i + D/2) as y_i = x_i cos + x_{i+D/2} sin, y_{i+D/2} = -x_i sin +
// x_{i+D/2} cos ("nanochat 项目深度分析" §2.1 item 1, §5.3), then RMS-normalise
// the head (item 2).
// Each head is handled by L = D / 16 lanes; lane j of a head holds the 8
// consecutive elements 8j..8j+7 of the first half and their rotation partners
// D/2 + 8j.. of the second half, so every access is 16 bytes (bf16) wide.
template <typename T, int D>
__global__ void __launch_bounds__(256)
rope_qknorm_fwd_kernel(T* __restrict__ qkv, float* __restrict__ rstdq, float* __restrict__ rstdk,
                       const float* __restrict__ cosv, const float* __restrict__ sinv, int N, int T_, int H, int Hkv,
                       float eps, int pos)
{
    constexpr int G = D / 2, L = D / 16;      // half width, lanes per head
    const int gid = blockIdx.x * (256 / L) + threadIdx.x / L;  // (n, head) with head in [0, H+Hkv)
    const int j = threadIdx.x % L;
    const int nh = H + Hkv;
    if (gid >= N * nh) return;                // whole heads leave together (L divides 64)
    const int n = gid / nh, hd = gid % nh;
    const int t = pos >= 0 ? pos : n % T_;      // pos >= 0: every row is a token at that position (decode)
    const int QKV = (H + 2 * Hkv) * D;
    T* v = qkv + (size_t)n * QKV + hd * D + 8 * j;   // k heads follow the q heads
    float x1[8], x2[8], c[8], sn[8];
    load8(v, x1);
    load8(v + G, x2);
    load8(cosv + t * G + 8 * j, c);
    load8(sinv + t * G + 8 * j, sn);
    float y1[8], y2[8], ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        y1[e] = x1[e] * c[e] + x2[e] * sn[e];
        y2[e] = -x1[e] * sn[e] + x2[e] * c[e];
        ss += y1[e] * y1[e] + y2[e] * y2[e];
    }
    ss = group_sum<L>(ss);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) { y1[e] *= rs; y2[e] *= rs; }
    store8(v, y1);
    store8(v + G, y2);
    if (j == 0) {
        if (hd < H) rstdq[(size_t)n * H + hd] = rs;
        else rstdk[(size_t)n * Hkv + hd - H] = rs;
    }
}

// Backward: QK-norm derivative from the saved normalised output y = qkv and
// rstd, then the transposed rotation.  In place on dqkv's q and k columns.
template <typename T, int D>
__global__ void __launch_bounds__(256)
rope_qknorm_bwd_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv, const float* __restrict__ rstdq,
                       const float* __restrict__ rstdk, const float* __restrict__ cosv, const float* __restrict__ sinv,
                       int N, int T_, int H, int Hkv)
{
    constexpr int G = D / 2, L = D / 16;
    const int gid = blockIdx.x * (256 / L) + threadIdx.x / L;
    const int j = threadIdx.x % L;
    const int nh = H + Hkv;
    if (gid >= N * nh) return;
    const int n = gid / nh, hd = gid % nh;
    const int t = n % T_;
    const int QKV = (H + 2 * Hkv) * D;
    const size_t o = (size_t)n * QKV + hd * D + 8 * j;
    float y1[8], y2[8], g1[8], g2[8], c[8], sn[8];
    load8(qkv + o, y1);
    load8(qkv + o + G, y2);
    load8(dqkv + o, g1);
    load8(dqkv + o + G, g2);
    load8(cosv + t * G + 8 * j, c);
    load8(sinv + t * G + 8 * j, sn);
    const float rs = hd < H ? rstdq[(size_t)n * H + hd] : rstdk[(size_t)n * Hkv + hd - H];
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += g1[e] * y1[e] + g2[e] * y2[e];
    dot = group_sum<L>(dot) / (float)D;
    float o1[8], o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float r1 = rs * (g1[e] - y1[e] * dot), r2 = rs * (g2[e] - y2[e] * dot);
        o1[e] = r1 * c[e] - r2 * sn[e];
        o2[e] = r1 * sn[e] + r2 * c[e];
    }
    store8(dqkv + o, o1);
    store8(dqkv + o + G, o2);
}

template <typename T>
static hipError_t rope_fwd_t(T* qkv, float* rq, float* rk, const float* c, const float* sn, int N, int T_, int H,
                             int Hkv, int D, float eps, int pos, hipStream_t s) {
    const size_t heads = (size_t)N * (H + Hkv);
    if (D == 128) {
        hipLaunchKernelGGL((rope_qknorm_fwd_kernel<T, 128>), dim3((unsigned)((heads + 31) / 32)), dim3(256), 0, s, qkv,
                           rq, rk, c, sn, N, T_, H, Hkv, eps, pos);
    } else if (D == 64) {
        hipLaunchKernelGGL((rope_qknorm_fwd_kernel<T, 64>), dim3((unsigned)((heads + 63) / 64)), dim3(256), 0, s, qkv,
                           rq, rk, c, sn, N, T_, H, Hkv, eps, pos);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t rope_bwd_t(T* dqkv, const T* qkv, const float* rq, const float* rk, const float* c, const float* sn,
                             int N, int T_, int H, int Hkv, int D, hipStream_t s) {
    const size_t heads = (size_t)N * (H + Hkv);
    if (D == 128) {
        hipLaunchKernelGGL((rope_qknorm_bwd_kernel<T, 128>), dim3((unsigned)((heads + 31) / 32)), dim3(256), 0, s, dqkv,
                           qkv, rq, rk, c, sn, N, T_, H, Hkv);
    } else if (D == 64) {
        hipLaunchKernelGGL((rope_qknorm_bwd_kernel<T, 64>), dim3((unsigned)((heads + 63) / 64)), dim3(256), 0, s, dqkv,
                           qkv, rq, rk, c, sn, N, T_, H, Hkv);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rope_qknorm_fwd(Dt dt, void* qkv, float* rstdq, float* rstdk, const float* cosv, const float* sinv,
                                  int N, int T, int H, int Hkv, int D, float eps, hipStream_t s, int pos) {
    if (dt == Dt::BF16) return rope_fwd_t((bf16*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, eps, pos, s);
    if (dt == Dt::F16) return rope_fwd_t((f16*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, eps, pos, s);
    return rope_fwd_t((float*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, eps, pos, s);
}

hipError_t launch_rope_qknorm_bwd(Dt dt, void* dqkv, const void* qkv, const float* rstdq, const float* rstdk,
                                  const float* cosv, const float* sinv, int N, int T, int H, int Hkv, int D,
                                  hipStream_t s) {
    if (dt == Dt::BF16)
        return rope_bwd_t((bf16*)dqkv, (const bf16*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, s);
    if (dt == Dt::F16)
        return rope_bwd_t((f16*)dqkv, (const f16*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, s);
    return rope_bwd_t((float*)dqkv, (const float*)qkv, rstdq, rstdk, cosv, sinv, N, T, H, Hkv, D, s);
}

// ------------------------------------------------------------------ cross-entropy
// Per row of logits z: lse = log sum exp z, loss_row = lse - z[target] (0
// when target < 0, i.e. ignored).  One workgroup per row; each thread reads 8
// consecutive logits per step (16 bytes in bf16) and keeps a running (max,
// sum of exp) pair in the base-2 domain.
template <typename T>
__global__ void __launch_bounds__(256)
ce_fwd_rows_kernel(const T* __restrict__ z, const int32_t* __restrict__ targets, float* __restrict__ lse,
                   float* __restrict__ loss_rows, int V, uint32_t* err)
{
    constexpr float kL2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
    __shared__ float red_m[4], red_s[4];
    const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const T* zr = z + (size_t)n * V;
    float m = -INFINITY, s = 0.0f;               // max of z log2(e), sum of 2^(z log2 e - m)
    for (int c = tid * 8; c < V; c += 2048) {
        float v[8];
        load8(zr + c, v);
        float mx = v[0] * kL2e;
#pragma unroll
        for (int e = 0; e < 8; ++e) { v[e] *= kL2e; mx = fmaxf(mx, v[e]); }
        if (mx > m) {
            s *= __builtin_amdgcn_exp2f(m - mx);
            m = mx;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(v[e] - m);
    }
    // combine (m, s) across the wave, then across the 4 waves
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float mo = __shfl_xor(m, o, kWave), so = __shfl_xor(s, o, kWave);
        float mn = fmaxf(m, mo);
        s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f(m - mn)) +
            (mo == -INFINITY ? 0.0f : so * __builtin_amdgcn_exp2f(mo - mn));
        m = mn;
    }
    if (lane == 0) { red_m[w] = m; red_s[w] = s; }
    __syncthreads();
    if (tid == 0) {
        float M = red_m[0];
        for (int i = 1; i < 4; ++i) M = fmaxf(M, red_m[i]);
        float S = 0.0f;
        for (int i = 0; i < 4; ++i) S += red_s[i] * __builtin_amdgcn_exp2f(red_m[i] - M);
        const float l = (M + __builtin_amdgcn_logf(S)) * kLn2;
        lse[n] = l;
        const int t = targets[n];
        float lr = 0.0f;
        if (t >= V) raise_error(err, kErrBadTarget);
        else if (t >= 0) lr = l - to_f32(zr[t]);
        loss_rows[n] = lr;
    }
}

hipError_t launch_ce_fwd_rows(Dt dt, const void* logits, const int32_t* targets, float* lse, float* loss_rows, int N,
                              int V, uint32_t* err, hipStream_t s) {
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(ce_fwd_rows_kernel<bf16>, dim3(N), dim3(256), 0, s, (const bf16*)logits, targets, lse,
                           loss_rows, V, err);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(ce_fwd_rows_kernel<f16>, dim3(N), dim3(256), 0, s, (const f16*)logits, targets, lse,
                           loss_rows, V, err);
    else
        hipLaunchKernelGGL(ce_fwd_rows_kernel<float>, dim3(N), dim3(256), 0, s, (const float*)logits, targets, lse,
                           loss_rows, V, err);
    return hipGetLastError();
}

// The same lse and per-row loss from the LM-head GEMM's per-block statistics (its CeStats epilogue):
// part[b][n] = (max of z log2 e over block b of row n, sum of 2^(z log2 e - max)), zt[n] = z[target].
// One lane per row merges the row's blocks in order with the running (max, sum) rule above; a wave's
// reads of one block are 512 contiguous bytes.
__global__ void __launch_bounds__(64)
ce_merge_kernel(const float2* __restrict__ part, int nblk, const float* __restrict__ zt,
                const int32_t* __restrict__ targets, float* __restrict__ lse, float* __restrict__ loss_rows, int N,
                int V, uint32_t* err)
{
    constexpr float kLn2 = 0.6931471805599453f;
    const int n = blockIdx.x * 64 + threadIdx.x;
    if (n >= N) return;
    float m = -INFINITY, s = 0.0f;
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) {
        const float2 p = part[(size_t)b * N + n];
        const float mn = fmaxf(m, p.x);
        s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f(m - mn)) + p.y * __builtin_amdgcn_exp2f(p.x - mn);
        m = mn;
    }
    const float l = (m + __builtin_amdgcn_logf(s)) * kLn2;
    lse[n] = l;
    const int t = targets[n];
    float lr = 0.0f;
    if (t >= V) raise_error(err, kErrBadTarget);
    else if (t >= 0) lr = l - zt[n];
    loss_rows[n] = lr;
}

hipError_t launch_ce_merge(const void* part, int nblk, const float* zt, const int32_t* targets, float* lse,
                           float* loss_rows, int N, int V, uint32_t* err, hipStream_t s) {
    if (nblk < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ce_merge_kernel, dim3((N + 63) / 64), dim3(64), 0, s, (const float2*)part, nblk, zt,
                       targets, lse, loss_rows, N, V, err);
    return hipGetLastError();
}

// loss = sum(loss_rows over valid targets) / #valid, in a fixed order (one
// workgroup); inv_valid = 1/#valid is kept for the backward.  No valid
// target raises kErrNoTargets and yields loss = NaN, inv_valid = 0.
__global__ void __launch_bounds__(1024)
loss_reduce_kernel(const float* __restrict__ loss_rows, const int32_t* __restrict__ targets, int N, int V,
                   float* __restrict__ loss, float* __restrict__ inv_valid, uint32_t* err)
{
    __shared__ double ssum[1024];
    __shared__ int scnt[1024];
    const int tid = threadIdx.x;
    double acc = 0.0;
    int cnt = 0;
    for (int i = tid; i < N; i += 1024) {
        int t = targets[i];
        if (t >= 0 && t < V) { acc += (double)loss_rows[i]; ++cnt; }
    }
    ssum[tid] = acc;
    scnt[tid] = cnt;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (tid < o) { ssum[tid] += ssum[tid + o]; scnt[tid] += scnt[tid + o]; }
        __syncthreads();
    }
    if (tid == 0) {
        if (scnt[0] == 0) {
            raise_error(err, kErrNoTargets);
            *loss = NAN;
            *inv_valid = 0.0f;
        } else {
            *loss = (float)(ssum[0] / (double)scnt[0]);
            *inv_valid = (float)(1.0 / (double)scnt[0]);
        }
    }
}

hipError_t launch_loss_reduce(const float* loss_rows, const int32_t* targets, int N, int V, float* loss,
                              float* inv_valid, uint32_t* err, hipStream_t s) {
    hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, s, loss_rows, targets, N, V, loss, inv_valid, err);
    return hipGetLastError();
}

// dz = grad_scale * inv_valid * (exp(z - lse) - onehot(target)) on valid rows,
// 0 on ignored rows; written over the logits.  With a soft-cap the logits are
// the capped ones and dz is taken back through the cap: times 1 - (z / c)^2.
// One workgroup per row, 8 consecutive logits per thread and chunk; a thread loads four chunks before it
// stores any, so each wave keeps 4 KB of reads in flight (one chunk at a time left HBM latency exposed).
template <typename T>
__device__ __forceinline__ void ce_bwd_chunk(float (&v)[8], int c, int t, float k, float l2, const SoftCap& cap) {
    constexpr float kL2e = 1.4426950408889634f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float zc = v[e];
        v[e] = k * (__builtin_amdgcn_exp2f(zc * kL2e - l2) - (c + e == t ? 1.0f : 0.0f));
        if (cap.c > 0.0f) v[e] = v[e] * softcap_grad(zc, cap);
    }
}

template <typename T>
__global__ void __launch_bounds__(256)
ce_bwd_kernel(T* __restrict__ z, const float* __restrict__ lse, const int32_t* __restrict__ targets,
              const float* __restrict__ inv_valid, float grad_scale, SoftCap cap, int V)
{
    constexpr float kL2e = 1.4426950408889634f;
    constexpr int U = 4, STEP = 2048;          // 256 threads x 8 logits
    const int n = blockIdx.x;
    const int t = targets[n];
    T* zr = z + (size_t)n * V;
    if (!(t >= 0 && t < V)) {                  // ignored row: zero gradient
        const float zero[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = threadIdx.x * 8; c < V; c += STEP) store8(zr + c, zero);
        return;
    }
    const float k = grad_scale * (*inv_valid), l2 = lse[n] * kL2e;
    const int full = V / (U * STEP) * (U * STEP);   // columns in whole groups of U chunks
    for (int c0 = threadIdx.x * 8; c0 < full; c0 += U * STEP) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8(zr + c0 + u * STEP, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ce_bwd_chunk<T>(v[u], c0 + u * STEP, t, k, l2, cap);
            store8(zr + c0 + u * STEP, v[u]);
        }
    }
    for (int c = full + threadIdx.x * 8; c < V; c += STEP) {
        float v[8];
        load8(zr + c, v);
        ce_bwd_chunk<T>(v, c, t, k, l2, cap);
        store8(zr + c, v);
    }
}

hipError_t launch_ce_bwd(Dt dt, void* logits, const float* lse, const int32_t* targets, const float* inv_valid,
                         float grad_scale, const SoftCap& cap, int N, int V, hipStream_t s) {
    if (V % 8) return hipErrorInvalidValue;
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(ce_bwd_kernel<bf16>, dim3(N), dim3(256), 0, s, (bf16*)logits, lse, targets, inv_valid,
                           grad_scale, cap, V);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(ce_bwd_kernel<f16>, dim3(N), dim3(256), 0, s, (f16*)logits, lse, targets, inv_valid,
                           grad_scale, cap, V);
    else
        hipLaunchKernelGGL(ce_bwd_kernel<float>, dim3(N), dim3(256), 0, s, (float*)logits, lse, targets, inv_valid,
                           grad_scale, cap, V);
    return hipGetLastError();
}

// z = c tanh(z / c) in place: the fp32 LM head's logits before the cross-entropy of the soft-capped variant.
template <typename T>
__global__ void __launch_bounds__(256)
softcap_kernel(T* __restrict__ z, size_t n4, SoftCap cap)
{
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        float v[4];
        Vec4<T>::load(z + 4 * i, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = softcap_fwd(v[e], cap);
        Vec4<T>::store(z + 4 * i, v);
    }
}

hipError_t launch_softcap(Dt dt, void* z, size_t n, const SoftCap& cap, hipStream_t s) {
    if (n % 4 || !(cap.c > 0.0f)) return hipErrorInvalidValue;
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 256 * 32);
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(softcap_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16*)z, n4, cap);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(softcap_kernel<f16>, dim3(blocks), dim3(256), 0, s, (f16*)z, n4, cap);
    else
        hipLaunchKernelGGL(softcap_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)z, n4, cap);
    return hipGetLastError();
}

// ------------------------------------------------------------------ fp8 row quantisation
// Row r of x -> q (OCP E4M3 bytes, the same layout) and the scale s[r] = amax / 448 with x ~ s q: every
// |x| / s <= 448, the largest finite E4M3 value (v_cvt_pk_fp8_f32 rounds to nearest even and does not
// saturate: 464 and beyond become NaN, so the scale keeps the row inside).  An all-zero row gets s = 1.
// One wave per row; blockIdx.y walks `layers` matrices at the given strides.
template <typename T>
__global__ void __launch_bounds__(256)
quant_rows_fp8_kernel(const T* __restrict__ x, size_t x_layer, uint8_t* __restrict__ q, size_t q_layer,
                      float* __restrict__ s, size_t s_layer, int rows, int cols)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const T* xr = x + blockIdx.y * x_layer + (size_t)row * cols;
    uint8_t* qr = q + blockIdx.y * q_layer + (size_t)row * cols;
    float amax = 0.0f;
    for (int c = lane * 8; c < cols; c += 512) {
        float v[8];
        load8(xr + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    for (int c = lane * 8; c < cols; c += 512) {
        float v[8];
        load8(xr + c, v);
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int t = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h] * inv, v[4 * h + 1] * inv, 0, false);
            t = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * h + 2] * inv, v[4 * h + 3] * inv, t, true);
            w[h] = (uint32_t)t;
        }
        *reinterpret_cast<uint2*>(qr + c) = make_uint2(w[0], w[1]);
    }
    if (lane == 0) s[blockIdx.y * s_layer + row] = amax > 0.0f ? amax / 448.0f : 1.0f;
}

// The same quantisation with the row held in registers (cols = 8 G NCH): G lanes per row, 256 / G rows per
// workgroup, lane j holding the 8-element chunks j, j + G, ...; x is read once.
template <typename T, int G, int NCH>
__global__ void __launch_bounds__(256)
quant_rows_fp8_regs(const T* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ s, int rows)
{
    constexpr int cols = 8 * G * NCH;
    const int row = blockIdx.x * (256 / G) + threadIdx.x / G, j = threadIdx.x % G;
    const bool live = row < rows;                // no early return before the lane-group maximum
    const size_t base = (size_t)(live ? row : 0) * cols + 8 * j;
    float v[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) load8(x + base + 8 * G * i, v[i]);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    amax = group_max<G>(amax);
    if (!live) return;
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) *reinterpret_cast<uint2*>(q + base + 8 * G * i) = fp8x8(v[i], inv);
    if (j == 0) s[row] = amax > 0.0f ? amax / 448.0f : 1.0f;
}

template <typename T>
static bool quant_rows_regs_launch(const T* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st) {
#define NCGPT_QR(g, n)                                                                                            \
    if (cols == 8 * g * n) {                                                                                       \
        hipLaunchKernelGGL((quant_rows_fp8_regs<T, g, n>), dim3((rows + 256 / g - 1) / (256 / g)), dim3(256), 0, \
                           st, x, q, s, rows);                                                                     \
        return true;                                                                                               \
    }
    NCGPT_QR(32, 1) NCGPT_QR(32, 2) NCGPT_QR(32, 3) NCGPT_QR(32, 5) NCGPT_QR(32, 6)
    NCGPT_QR(64, 2) NCGPT_QR(64, 4) NCGPT_QR(64, 6) NCGPT_QR(64, 8) NCGPT_QR(64, 10) NCGPT_QR(64, 12)
#undef NCGPT_QR
    return false;
}

hipError_t launch_quant_rows_fp8(Dt src, const void* x, size_t x_layer, void* q, size_t q_layer, float* s,
                                 size_t s_layer, int rows, int cols, int layers, hipStream_t st) {
    if (cols % 8 || rows < 0 || layers < 1) return hipErrorInvalidValue;
    if (rows == 0) return hipSuccess;
    // one bf16 matrix (the activations): rows in registers where the width has a kernel
    if (src == Dt::BF16 && layers == 1 && quant_rows_regs_launch((const bf16*)x, (uint8_t*)q, s, rows, cols, st))
        return hipGetLastError();
    const dim3 grid((unsigned)((rows + 3) / 4), (unsigned)layers);
    if (src == Dt::BF16)
        hipLaunchKernelGGL(quant_rows_fp8_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)x, x_layer, (uint8_t*)q,
                           q_layer, s, s_layer, rows, cols);
    else if (src == Dt::F16)
        hipLaunchKernelGGL(quant_rows_fp8_kernel<f16>, grid, dim3(256), 0, st, (const f16*)x, x_layer, (uint8_t*)q,
                           q_layer, s, s_layer, rows, cols);
    else
        hipLaunchKernelGGL(quant_rows_fp8_kernel<float>, grid, dim3(256), 0, st, (const float*)x, x_layer,
                           (uint8_t*)q, q_layer, s, s_layer, rows, cols);
    return hipGetLastError();
}

// ------------------------------------------------------------------ loss-scaling check
// ok = 1, then any thread that meets a non-finite value stores 0 (every writer stores the same value).
__global__ void __launch_bounds__(64) set_one_kernel(int32_t* ok) { if (threadIdx.x == 0) *ok = 1; }
__global__ void __launch_bounds__(256) finite_kernel(const float* __restrict__ x, size_t n, int32_t* ok)
{
    const size_t stride = (size_t)gridDim.x * 256;
    bool bad = false;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) bad |= !__builtin_isfinite(x[i]);
    if (__any(bad) && bad) *ok = 0;
}

hipError_t launch_finite(const float* x, size_t n, int32_t* ok, hipStream_t s) {
    hipLaunchKernelGGL(set_one_kernel, dim3(1), dim3(64), 0, s, ok);
    if (n == 0) return hipGetLastError();
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(finite_kernel, dim3(blocks), dim3(256), 0, s, x, n, ok);
    return hipGetLastError();
}

// ------------------------------------------------------------------ embedding backward
// dwte[v] = sum of dx rows of the tokens with id v, summed in a fixed order so
// the result is bitwise reproducible (no float atomics):
//   1. a stable counting sort of (id, position) pairs by id: per block of 1024
//      tokens an id histogram, an exclusive prefix over blocks per id and over
//      ids, and a scatter at base[id] + (earlier blocks' count of id) + (earlier
//      tokens of id in the block);
//   2. the sorted array is cut into fixed chunks of 64; each chunk sums the
//      rows of every run of equal ids inside it and writes the partial sum at
//      the run's first sorted index;
//   3. each vocab row sums its runs' partials (its sorted range [a, b) has
//      partials at a and at every chunk start inside it), in order.
constexpr int kSortBlock = 1024;   // tokens per counting block
constexpr int kMaxSortVocab = 65536;
constexpr int kChunk = 64;

__device__ __forceinline__ int clamp_id(int id, int V) { return (id >= 0 && id < V) ? id : 0; }  // bad ids: reported by the forward

// cnt[b][v] = number of tokens of block b with id v (two 16-bit counters per LDS word)
__global__ void __launch_bounds__(1024)
embed_hist_kernel(const int32_t* __restrict__ ids, int N, int V, uint32_t* __restrict__ cnt)
{
    __shared__ uint32_t h[kMaxSortVocab / 2];
    const int b = blockIdx.x, t = threadIdx.x;
    for (int i = t; i < (V + 1) / 2; i += 1024) h[i] = 0;
    __syncthreads();
    const int n = b * kSortBlock + t;
    if (n < N) {
        const int id = clamp_id(ids[n], V);
        atomicAdd(&h[id >> 1], 1u << (16 * (id & 1)));
    }
    __syncthreads();
    uint32_t* row = cnt + (size_t)b * V;
    for (int v = t; v < V; v += 1024) row[v] = (h[v >> 1] >> (16 * (v & 1))) & 0xffffu;
}

// per id: cnt[b][v] <- tokens of id v in blocks before b; total[v] <- all tokens of id v
__global__ void __launch_bounds__(256)
embed_colscan_kernel(uint32_t* __restrict__ cnt, int G, int V, uint32_t* __restrict__ total)
{
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= V) return;
    uint32_t run = 0;
    for (int b = 0; b < G; ++b) {
        const uint32_t c = cnt[(size_t)b * V + v];
        cnt[(size_t)b * V + v] = run;
        run += c;
    }
    total[v] = run;
}

// total[v] <- exclusive prefix sum over ids (one workgroup)
__global__ void __launch_bounds__(1024)
embed_idscan_kernel(uint32_t* __restrict__ total, int V)
{
    __shared__ uint32_t part[1024];
    const int t = threadIdx.x;
    const int per = (V + 1023) / 1024, beg = min(V, t * per), end = min(V, beg + per);
    uint32_t sum = 0;
    for (int v = beg; v < end; ++v) sum += total[v];
    part[t] = sum;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the per-thread sums
        const uint32_t x = t >= o ? part[t - o] : 0u;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    uint32_t run = t > 0 ? part[t - 1] : 0u;
    for (int v = beg; v < end; ++v) {
        const uint32_t c = total[v];
        total[v] = run;
        run += c;
    }
}

__global__ void __launch_bounds__(1024)
embed_scatter_kernel(const int32_t* __restrict__ ids, int N, int V, const uint32_t* __restrict__ cnt,
                     const uint32_t* __restrict__ base, int32_t* __restrict__ skeys, int32_t* __restrict__ spos)
{
    __shared__ int32_t bid[kSortBlock];
    const int b = blockIdx.x, t = threadIdx.x, n = b * kSortBlock + t;
    const int id = n < N ? clamp_id(ids[n], V) : -1;
    bid[t] = id;
    __syncthreads();
    if (n >= N) return;
    int rank = 0;  // earlier tokens of the block with the same id (all lanes read the same word: a broadcast)
    for (int j = 0; j < t; ++j) rank += bid[j] == id;
    const uint32_t pos = base[id] + cnt[(size_t)b * V + id] + (uint32_t)rank;
    skeys[pos] = id;
    spos[pos] = n;
}

__global__ void __launch_bounds__(256)
embed_bwd_chunks_kernel(const int32_t* __restrict__ skeys, const int32_t* __restrict__ spos, const float* __restrict__ dx,
                        float* __restrict__ partial, int N, int C)
{
    const int c0 = blockIdx.x * kChunk, c1 = min(N, c0 + kChunk);
    for (int c = threadIdx.x * 4; c < C; c += 1024) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        int start = c0;
        for (int i = c0; i < c1; ++i) {
            float v[4];
            Vec4<float>::load(dx + (size_t)spos[i] * C + c, v);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += v[e];
            if (i + 1 == c1 || skeys[i + 1] != skeys[i]) {
                Vec4<float>::store(partial + (size_t)start * C + c, acc);
                acc[0] = acc[1] = acc[2] = acc[3] = 0.0f;
                start = i + 1;
            }
        }
    }
}

__global__ void __launch_bounds__(256)
embed_bwd_combine_kernel(const int32_t* __restrict__ skeys, const float* __restrict__ partial, float* __restrict__ dwte,
                         int N, int C, int accumulate)
{
    const int v = blockIdx.x;
    // [a, b) = sorted range of id v
    int lo = 0, hi = N;
    while (lo < hi) { int mid = (lo + hi) >> 1; if (skeys[mid] < v) lo = mid + 1; else hi = mid; }
    const int a = lo;
    hi = N;
    while (lo < hi) { int mid = (lo + hi) >> 1; if (skeys[mid] <= v) lo = mid + 1; else hi = mid; }
    const int b = lo;
    for (int c = threadIdx.x * 4; c < C; c += 1024) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (accumulate) Vec4<float>::load(dwte + (size_t)v * C + c, acc);
        if (a < b) {
            float s[4];
            Vec4<float>::load(partial + (size_t)a * C + c, s);
            for (int p = (a / kChunk + 1) * kChunk; p < b; p += kChunk) {
                float q[4];
                Vec4<float>::load(partial + (size_t)p * C + c, q);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[e] += q[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += s[e];
        }
        Vec4<float>::store(dwte + (size_t)v * C + c, acc);
    }
}

size_t embed_bwd_scratch_ints(int N, int V) {
    const size_t G = ((size_t)N + kSortBlock - 1) / kSortBlock;
    return 2 * (size_t)N + G * (size_t)V + (size_t)V;
}

hipError_t launch_embed_bwd(const int32_t* ids, const float* dx, float* dwte, int N, int C, int V, int accumulate,
                            int32_t* iscratch, float* partial, hipStream_t s) {
    if (V > kMaxSortVocab || N <= 0) return hipErrorInvalidValue;
    const int G = (N + kSortBlock - 1) / kSortBlock;
    int32_t* skeys = iscratch;
    int32_t* spos = iscratch + N;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(iscratch + 2 * (size_t)N);
    uint32_t* base = cnt + (size_t)G * V;
    hipLaunchKernelGGL(embed_hist_kernel, dim3(G), dim3(1024), 0, s, ids, N, V, cnt);
    hipLaunchKernelGGL(embed_colscan_kernel, dim3((V + 255) / 256), dim3(256), 0, s, cnt, G, V, base);
    hipLaunchKernelGGL(embed_idscan_kernel, dim3(1), dim3(1024), 0, s, base, V);
    hipLaunchKernelGGL(embed_scatter_kernel, dim3(G), dim3(1024), 0, s, ids, N, V, cnt, base, skeys, spos);
    hipLaunchKernelGGL(embed_bwd_chunks_kernel, dim3((N + kChunk - 1) / kChunk), dim3(256), 0, s, skeys, spos, dx,
                       partial, N, C);
    hipLaunchKernelGGL(embed_bwd_combine_kernel, dim3(V), dim3(256), 0, s, skeys, partial, dwte, N, C, accumulate);
    return hipGetLastError();
}

// ------------------------------------------------------------------ zero fill
// Clears n 32-bit words with ordinary stores (a kernel rather than a memset node, so
// that a caller may capture the call in a HIP graph).
__global__ void __launch_bounds__(256) zero_u32_kernel(uint32_t* __restrict__ p, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ------------------------------------------------------------------ probe helper
template <typename T>
__global__ void __launch_bounds__(256) to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst, size_t n)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = to_f32(src[i]);
}

hipError_t launch_to_f32(Dt dt, const void* src, float* dst, size_t n, hipStream_t s) {
    unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
    if (blocks == 0) return hipSuccess;
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(to_f32_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)src, dst, n);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(to_f32_kernel<f16>, dim3(blocks), dim3(256), 0, s, (const f16*)src, dst, n);
    else
        hipLaunchKernelGGL(to_f32_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)src, dst, n);
    return hipGetLastError();
}

}  // namespace ncgpt
