// KV-cache decode: one new token per sequence against a preallocated cache laid out (layers, 2, B, Hkv, T, D)
// with a position pointer ("nanochat 项目深度分析", engine section on the KV cache).  The block math is the
// training forward's; these kernels are the parts that differ: storing k and v into the cache, attention of
// one query row per head over the cached positions, and finishing the split-K products of B-row GEMMs.
#include "common.h"
#include "kernels.h"

namespace ncgpt {

// ---------------------------------------------------------------- cache stores
// For b < B and t in [t0, t0 + nt): cache[0][b][g][t][:] = k head g and cache[1][b][g][t][:] = v head g of
// qkv row b * rb + (t - t0).  rb = 1: the B rows of a decode step (nt = 1); rb = T: a forward's saved qkv.
template <typename T>
__global__ void __launch_bounds__(256)
kv_store_kernel(const T* __restrict__ qkv, T* __restrict__ cache, int B, int H, int Hkv, int D, int Tc, int t0, int nt,
                int rb)
{
    const int KD = Hkv * D, QKV = (H + 2 * Hkv) * D;
    const size_t per_b = (size_t)nt * KD / 4;          // 4-element groups of one sequence and one of k / v
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= 2 * (size_t)B * per_b) return;
    const int kv = (int)(i / ((size_t)B * per_b));
    const size_t r = i % ((size_t)B * per_b);
    const int b = (int)(r / per_b);
    const size_t e = (r % per_b) * 4;                  // element inside [nt][KD]
    const int tt = (int)(e / KD), col = (int)(e % KD), g = col / D, d = col % D;
    const T* src = qkv + ((size_t)b * rb + tt) * QKV + (size_t)H * D + (size_t)kv * KD + col;
    T* dst = cache + ((((size_t)kv * B + b) * Hkv + g) * Tc + (t0 + tt)) * D + d;
    float v[4];
    Vec4<T>::load(src, v);
    Vec4<T>::store(dst, v);
}

hipError_t launch_kv_store(Dt dt, const void* qkv, void* cache, int B, int H, int Hkv, int D, int Tc, int t0, int nt,
                           int rb, hipStream_t s) {
    const size_t n = 2 * (size_t)B * nt * Hkv * D / 4;
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(kv_store_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)cache, B, H, Hkv, D, Tc,
                           t0, nt, rb);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(kv_store_kernel<f16>, grid, dim3(256), 0, s, (const f16*)qkv, (f16*)cache, B, H, Hkv, D, Tc,
                           t0, nt, rb);
    else
        hipLaunchKernelGGL(kv_store_kernel<float>, grid, dim3(256), 0, s, (const float*)qkv, (float*)cache, B, H, Hkv,
                           D, Tc, t0, nt, rb);
    return hipGetLastError();
}

// ---------------------------------------------------------------- attention of one query row per head
// Workgroup (chunk, kv head g, sequence b): the r = H / Hkv query heads of g against cache positions
// [256 chunk, 256 chunk + 256) that are <= pos.  QK-norm bounds every scaled score by sqrt(D), so the
// softmax uses the static shift sqrt(D) (as the training kernels do) and chunks combine by plain sums:
// part[b][h][chunk] = (sum_j p_j v_j [D values], sum_j p_j).  LP = D / 8 lanes share one position, each
// holding 8 consecutive dims; a wave covers 64 / LP positions per step.
template <typename T, int D, int R>
__global__ void __launch_bounds__(256)
decode_attn_kernel(const T* __restrict__ qkv, const T* __restrict__ cache, float* __restrict__ part, int B, int H,
                   int Hkv, int Tc, int pos, int nchunk)
{
    constexpr int LP = D / 8, PW = 64 / LP;            // lanes per position, positions per wave step
    __shared__ float red[4][R][D + 1];
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int pg = lane / LP, dl = lane % LP;
    const int QKV = (H + 2 * Hkv) * D;
    const float c1 = 1.4426950408889634f * rsqrtf((float)D), c2 = sqrtf((float)D) * 1.4426950408889634f;
    float q[R][8], o[R][8], l[R];
#pragma unroll
    for (int hh = 0; hh < R; ++hh) {
        const T* qp = qkv + (size_t)b * QKV + (size_t)(g * R + hh) * D + 8 * dl;
        float a[4], c[4];
        Vec4<T>::load(qp, a);
        Vec4<T>::load(qp + 4, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) { q[hh][e] = a[e]; q[hh][4 + e] = c[e]; }
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.0f;
        l[hh] = 0.0f;
    }
    const T* kb = cache + (((size_t)0 * B + b) * Hkv + g) * (size_t)Tc * D;
    const T* vb = cache + (((size_t)1 * B + b) * Hkv + g) * (size_t)Tc * D;
    const int j0 = chunk * 256 + w * 64;
    for (int s = 0; s < 64; s += PW) {
        const int j = j0 + s + pg;
        if (j > pos) break;                              // positions only grow along the loop
        float k8[8], v8[8], a[4], c[4];
        Vec4<T>::load(kb + (size_t)j * D + 8 * dl, a);
        Vec4<T>::load(kb + (size_t)j * D + 8 * dl + 4, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) { k8[e] = a[e]; k8[4 + e] = c[e]; }
        Vec4<T>::load(vb + (size_t)j * D + 8 * dl, a);
        Vec4<T>::load(vb + (size_t)j * D + 8 * dl + 4, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v8[e] = a[e]; v8[4 + e] = c[e]; }
#pragma unroll
        for (int hh = 0; hh < R; ++hh) {
            float sdot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sdot += q[hh][e] * k8[e];
#pragma unroll
            for (int off = LP / 2; off > 0; off >>= 1) sdot += __shfl_xor(sdot, off, kWave);
            const float p = __builtin_amdgcn_exp2f(sdot * c1 - c2);
            l[hh] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[hh][e] += p * v8[e];
        }
    }
    // the position groups of a wave hold disjoint positions: add them (lanes with equal dl), then the waves
#pragma unroll
    for (int hh = 0; hh < R; ++hh) {
#pragma unroll
        for (int off = LP; off < 64; off <<= 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[hh][e] += __shfl_xor(o[hh][e], off, kWave);
            l[hh] += __shfl_xor(l[hh], off, kWave);
        }
        if (pg == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w][hh][8 * dl + e] = o[hh][e];
            if (dl == 0) red[w][hh][D] = l[hh];
        }
    }
    __syncthreads();
    for (int i = tid; i < R * (D + 1); i += 256) {
        const int hh = i / (D + 1), d = i % (D + 1);
        const float v = (red[0][hh][d] + red[1][hh][d]) + (red[2][hh][d] + red[3][hh][d]);
        part[(((size_t)b * H + g * R + hh) * nchunk + chunk) * (D + 1) + d] = v;
    }
}

// y[b][h D + d] = sum_chunks o / sum_chunks l, in chunk order.
template <typename T, int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(const float* __restrict__ part, T* __restrict__ y, int H, int nchunk)
{
    const int bh = blockIdx.x, d = threadIdx.x;
    const float* pp = part + (size_t)bh * nchunk * (D + 1);
    float o = 0.0f, l = 0.0f;
    int c = 0;
    for (; c + 4 <= nchunk; c += 4) {   // chunk order, four chunks' loads in flight
        float po[4], pl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            po[u] = pp[(c + u) * (D + 1) + d];
            pl[u] = pp[(c + u) * (D + 1) + D];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            o += po[u];
            l += pl[u];
        }
    }
    for (; c < nchunk; ++c) {
        o += pp[c * (D + 1) + d];
        l += pp[c * (D + 1) + D];
    }
    y[(size_t)(bh / H) * H * D + (size_t)(bh % H) * D + d] = from_f32<T>(o / l);
}

template <typename T, int D>
static hipError_t decode_attn_t(const void* qkv, const void* cache, float* part, void* y, int B, int H, int Hkv,
                                int Tc, int pos, hipStream_t s) {
    const int nchunk = pos / 256 + 1, r = H / Hkv;
    const dim3 grid(nchunk, Hkv, B);
#define NCGPT_DEC(RR)                                                                                           \
    case RR:                                                                                                    \
        hipLaunchKernelGGL((decode_attn_kernel<T, D, RR>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)cache, part, \
                           B, H, Hkv, Tc, pos, nchunk);                                                         \
        break;
    switch (r) {
        NCGPT_DEC(1) NCGPT_DEC(2) NCGPT_DEC(3) NCGPT_DEC(4)
    default: return hipErrorInvalidValue;
    }
#undef NCGPT_DEC
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(B * H), dim3(D), 0, s, part, (T*)y, H, nchunk);
    return hipGetLastError();
}

size_t decode_attn_part_floats(int B, int H, int D, int Tc) { return (size_t)B * H * ((Tc + 255) / 256) * (D + 1); }

hipError_t launch_decode_attn(Dt dt, const void* qkv, const void* cache, float* part, void* y, int B, int H, int Hkv,
                              int D, int Tc, int pos, hipStream_t s) {
    if (pos < 0 || pos >= Tc || H % Hkv) return hipErrorInvalidValue;
    if (dt == Dt::BF16) {
        if (D == 128) return decode_attn_t<bf16, 128>(qkv, cache, part, y, B, H, Hkv, Tc, pos, s);
        if (D == 64) return decode_attn_t<bf16, 64>(qkv, cache, part, y, B, H, Hkv, Tc, pos, s);
    } else if (dt == Dt::F16) {
        if (D == 128) return decode_attn_t<f16, 128>(qkv, cache, part, y, B, H, Hkv, Tc, pos, s);
    } else {
        if (D == 128) return decode_attn_t<float, 128>(qkv, cache, part, y, B, H, Hkv, Tc, pos, s);
        if (D == 64) return decode_attn_t<float, 64>(qkv, cache, part, y, B, H, Hkv, Tc, pos, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- split-K finish of B-row GEMMs
// v = sum over splits of part[s][m][n] (in split order); rows m < rows only.
//   mode 0: out = cd(v);  1: out = cd(in + v) (residual; in may equal out);
//   mode 2: out = cd(a * a), a = cd(max(v, 0)) (the MLP activation);  3: out(f32) = v, or c tanh(v / c)
//   with a soft-cap (the logits).
template <typename T>
__global__ void __launch_bounds__(256)
decode_finish_kernel(const float* __restrict__ part, int splits, size_t stride, int rows, int N, int mode,
                     void* __restrict__ out, const T* in, SoftCap cap)
{
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)rows * N) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    // partials added in split order, four loads in flight at a time (one at a time left the chain of load
    // latencies exposed: these kernels move little data)
    int sp = 0;
    for (; sp + 4 <= splits; sp += 4) {
        float p[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) Vec4<float>::load(part + (sp + u) * stride + i, p[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += p[u][e];
    }
    for (; sp < splits; ++sp) {
        float p[4];
        Vec4<float>::load(part + sp * stride + i, p);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += p[e];
    }
    if (mode == 3) {
        if (cap.c > 0.0f) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = softcap_fwd(v[e], cap);
        }
        Vec4<float>::store((float*)out + i, v);
        return;
    }
    if (mode == 1) {
        float x[4];
        Vec4<T>::load(in + i, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += x[e];
    } else if (mode == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = to_f32(from_f32<T>(fmaxf(v[e], 0.0f)));
            v[e] = a * a;
        }
    }
    Vec4<T>::store((T*)out + i, v);
}

hipError_t launch_decode_finish(Dt dt, const float* part, int splits, size_t stride, int rows, int N, int mode,
                                void* out, const void* in, hipStream_t s, const SoftCap& cap) {
    if (N % 4) return hipErrorInvalidValue;
    const size_t n4 = (size_t)rows * N / 4;
    if (n4 == 0) return hipSuccess;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(decode_finish_kernel<bf16>, grid, dim3(256), 0, s, part, splits, stride, rows, N, mode, out,
                           (const bf16*)in, cap);
    else if (dt == Dt::F16)
        hipLaunchKernelGGL(decode_finish_kernel<f16>, grid, dim3(256), 0, s, part, splits, stride, rows, N, mode, out,
                           (const f16*)in, cap);
    else
        hipLaunchKernelGGL(decode_finish_kernel<float>, grid, dim3(256), 0, s, part, splits, stride, rows, N, mode, out,
                           (const float*)in, cap);
    return hipGetLastError();
}

}  // namespace ncgpt
