// Device-side helpers shared by the ncgpt HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace ncgpt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- scalar conversions (fp32 -> bf16 is round-to-nearest-even in hardware) ----
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// 16-byte vector of eight 16-bit values of type T (bf16 or f16)
template <typename T> struct V8 { typedef bf16x8 type; };
template <> struct V8<f16> { typedef f16x8 type; };

// Round a and b to the 16-bit type H and back (the values a store of H keeps), with one packed conversion.
template <typename H>
__device__ __forceinline__ void round2(float a, float b, float& ra, float& rb) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {a, b};
    if constexpr (std::is_same<H, f16>::value) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 h = __builtin_convertvector(f, f16x2);
        ra = (float)h[0];
        rb = (float)h[1];
    } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
        ra = __uint_as_float(u << 16);
        rb = __uint_as_float(u & 0xffff0000u);
    }
}

// One 32x32x16 product of 16-bit operands held as 16-byte fragments (bit patterns): bf16, or fp16 when H is f16.
template <typename H>
__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    if constexpr (std::is_same<H, f16>::value)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- 4-element vector load/store of T (8 B for bf16, 16 B for fp32) ----
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    __device__ static __forceinline__ void load(const float* p, float (&v)[4]) {
        float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec4<bf16> {
    __device__ static __forceinline__ void load(const bf16* p, float (&v)[4]) {
        bf16x4 t = *reinterpret_cast<const bf16x4*>(p);
        v[0] = (float)t[0]; v[1] = (float)t[1]; v[2] = (float)t[2]; v[3] = (float)t[3];
    }
    __device__ static __forceinline__ void store(bf16* p, const float (&v)[4]) {
        bf16x4 t;
        t[0] = (bf16)v[0]; t[1] = (bf16)v[1]; t[2] = (bf16)v[2]; t[3] = (bf16)v[3];
        *reinterpret_cast<bf16x4*>(p) = t;
    }
};
template <> struct Vec4<f16> {
    __device__ static __forceinline__ void load(const f16* p, float (&v)[4]) {
        f16x4 t = *reinterpret_cast<const f16x4*>(p);
        v[0] = (float)t[0]; v[1] = (float)t[1]; v[2] = (float)t[2]; v[3] = (float)t[3];
    }
    __device__ static __forceinline__ void store(f16* p, const float (&v)[4]) {
        f16x4 t;
        t[0] = (f16)v[0]; t[1] = (f16)v[1]; t[2] = (f16)v[2]; t[3] = (f16)v[3];
        *reinterpret_cast<f16x4*>(p) = t;
    }
};

// ---- wave reductions (64 lanes) ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// ---- workgroup order: workgroups are dealt round-robin to the 8 XCDs (each with its own L2), and an XCD
// starts its share in dispatch order; renumber them so XCD x runs one contiguous range of the logical order
// (a bijection on [0, nwg)) ----
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    constexpr int NX = 8;
    int per = (nwg + NX - 1) / NX;
    int xcd = wg % NX, local = wg / NX;
    int tall = nwg % NX;
    if (tall == 0) tall = NX;
    if (xcd < tall) return xcd * per + local;
    return tall * per + (xcd - tall) * (per - 1) + local;
}

// ---- logit soft-cap: c tanh(z / c) = c - 2c / (e^{2z/c} + 1), one exp and one reciprocal; saturates at +-c
// (e^{2z/c} -> inf gives c, -> 0 gives -c) without a NaN ----
__device__ __forceinline__ float softcap_fwd(float z, const SoftCap& s) {
    return fmaf(-s.c2, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(z * s.k) + 1.0f), s.c);
}
// d(capped) / dz from the capped value zc: 1 - tanh^2 = 1 - (zc / c)^2
__device__ __forceinline__ float softcap_grad(float zc, const SoftCap& s) {
    const float q = zc * s.ic;
    return fmaf(-q, q, 1.0f);
}

__device__ __forceinline__ void raise_error(uint32_t* flag, uint32_t bit) { atomicOr(flag, bit); }

}  // namespace ncgpt
