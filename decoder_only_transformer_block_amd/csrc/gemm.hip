// GEMMs of the block stack: the bias-free linears y = x W^T (forward), their
// input gradients dx = dy W and weight gradients dW = dy^T x (backward).
//
// bf16 path: MFMA kernels (v_mfma_f32_32x32x16_bf16, fp32 accumulation) for
// all three operand layouts.  Operand tiles travel from memory straight into
// LDS (buffer_load ... lds) in 32-deep stages held in a four-stage ring, three
// stages ahead of the MFMAs; 4 or 8 waves per workgroup (2 x 2 or 2 x 4),
// either one output tile per workgroup or persistent over (split, tile)
// items.  Operands whose K index is not contiguous in memory (the token-major
// activations of a weight gradient, the [out,in] weight of an input gradient)
// stay in LDS in their natural layout and their MFMA fragments are read with
// gfx950's transposing LDS load (ds_read_b64_tr_b16).
//
// The MFMA is issued with the two operands swapped (it computes C^T), which
// leaves each lane holding 4 consecutive columns of one output row: the
// epilogues get (row, col..col+3) and row-wise work stays inside a lane.
//
// fp32 path: a plain LDS-tiled SIMT kernel with the same epilogues (the fp32
// compute mode of the precision scheme is a correctness path).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ncgpt {

// ------------------------------------------------------------------ epilogues
// Each epilogue takes (row m, first column n, k split, 4 consecutive values).
// The bf16 ones also take 8 consecutive values (put8): the MFMA kernels
// exchange half-tiles between lanes l and l+32 so that a lane owns 8
// consecutive columns and stores 16 bytes at once.
template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&v)[8]) {
    const typename V8<T>::type t = *reinterpret_cast<const typename V8<T>::type*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
}
template <typename T>
__device__ __forceinline__ void st8(T* p, const float (&v)[8]) {
    typename V8<T>::type t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (T)v[e];
    *reinterpret_cast<typename V8<T>::type*>(p) = t;
}

template <typename T> struct EStoreCd {
    static constexpr bool kWide = sizeof(T) == 2, kLoads = false;
    T* out; int ldo;
    int64_t sOut = 0;  // batch stride (elements) of a batched GEMM
    __device__ EStoreCd at(int z) const { EStoreCd e = *this; e.out += z * sOut; return e; }
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        Vec4<T>::store(out + (size_t)m * ldo + n, v);
    }
    __device__ void put8(int m, int n, int, const float (&v)[8]) const { st8(out + (size_t)m * ldo + n, v); }
};
template <typename T> struct EResidual {
    static constexpr bool kWide = sizeof(T) == 2, kLoads = true;
    typedef typename V8<T>::type vec8;
    T* out; const T* in; int ldo;
    __device__ vec8 fetch8(int m, int n) const { return *reinterpret_cast<const vec8*>(in + (size_t)m * ldo + n); }
    __device__ void put8(int m, int n, int, const float (&v)[8], const vec8& x) const {
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (float)x[i] + v[i];
        st8(out + (size_t)m * ldo + n, r);
    }
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        size_t o = (size_t)m * ldo + n;
        float x[4];
        Vec4<T>::load(in + o, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] += v[i];
        Vec4<T>::store(out + o, x);
    }
    __device__ void put8(int m, int n, int, const float (&v)[8]) const {
        const size_t o = (size_t)m * ldo + n;
        float x[8];
        ld8(in + o, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] += v[i];
        st8(out + o, x);
    }
};
// out = cd(alpha in + beta v): the Newton-Schulz steps B = b A + c A A and X = a X + B X (bf16)
struct EAxpby {
    static constexpr bool kWide = true, kLoads = true;
    typedef bf16x8 vec8;
    bf16* out; const bf16* in; int ldo;
    float alpha, beta;
    int64_t sOut, sIn;  // batch strides (elements)
    __device__ EAxpby at(int z) const {
        EAxpby e = *this;
        e.out += z * sOut;
        e.in += z * sIn;
        return e;
    }
    __device__ bf16x8 fetch8(int m, int n) const { return *reinterpret_cast<const bf16x8*>(in + (size_t)m * ldo + n); }
    __device__ void put8(int m, int n, int, const float (&v)[8], const bf16x8& x) const {
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = alpha * (float)x[i] + beta * v[i];
        st8(out + (size_t)m * ldo + n, r);
    }
    __device__ void put8(int, int, int, const float (&)[8]) const {}
    __device__ void operator()(int, int, int, const float (&)[4]) const {}
};

// Epilogues of batched GEMMs shift their pointers to batch item z (at()); the others take z = 0 only.
template <class E, class = void> struct BatchEpi : std::false_type {};
template <class E> struct BatchEpi<E, std::void_t<decltype(std::declval<const E&>().at(0))>> : std::true_type {};
template <class E> __device__ __forceinline__ E epi_at(const E& e, int z) {
    if constexpr (BatchEpi<E>::value) return e.at(z);
    else return e;
}

// act = a^2 with a = relu(v) rounded to the compute dtype: the only stored output of
// the MLP's first linear; the backward recovers a as sqrt(act)
template <typename T> struct EReluSq {
    static constexpr bool kWide = sizeof(T) == 2, kLoads = false;
    T* act; int ldo;
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float r = to_f32(from_f32<T>(fmaxf(v[i], 0.0f)));
            s[i] = r * r;
        }
        Vec4<T>::store(act + (size_t)m * ldo + n, s);
    }
    __device__ void put8(int m, int n, int, const float (&v)[8]) const {
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float r = to_f32(from_f32<T>(fmaxf(v[i], 0.0f)));
            s[i] = r * r;
        }
        st8(act + (size_t)m * ldo + n, s);
    }
};
// dh = dact * d(relu(h)^2)/dh = dact * 2 relu(h), with relu(h) = sqrt(act)
template <typename T> struct EReluSqBwd {
    static constexpr bool kWide = sizeof(T) == 2, kLoads = true;
    typedef typename V8<T>::type vec8;
    T* out; const T* act; int ldo;
    __device__ vec8 fetch8(int m, int n) const { return *reinterpret_cast<const vec8*>(act + (size_t)m * ldo + n); }
    __device__ void put8(int m, int n, int, const float (&v)[8], const vec8& x) const {
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = v[i] * 2.0f * __builtin_amdgcn_sqrtf((float)x[i]);
        st8(out + (size_t)m * ldo + n, r);
    }
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        size_t o = (size_t)m * ldo + n;
        float x[4];
        Vec4<T>::load(act + o, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = v[i] * 2.0f * __builtin_amdgcn_sqrtf(x[i]);
        Vec4<T>::store(out + o, x);
    }
    __device__ void put8(int m, int n, int, const float (&v)[8]) const {
        const size_t o = (size_t)m * ldo + n;
        float x[8];
        ld8(act + o, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = v[i] * 2.0f * __builtin_amdgcn_sqrtf(x[i]);
        st8(out + o, x);
    }
};
struct EGrad {
    static constexpr bool kWide = false, kLoads = false;
    float* out; int ldo; int acc;
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        float* p = out + (size_t)m * ldo + n;
        float x[4] = {v[0], v[1], v[2], v[3]};
        if (acc) {
            float o[4];
            Vec4<float>::load(p, o);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += o[i];
        }
        Vec4<float>::store(p, x);
    }
    __device__ void put8(int, int, int, const float (&)[8]) const {}
};
struct ESplitK {
    static constexpr bool kWide = false, kLoads = false;
    float* out; int ldo; size_t stride;
    __device__ void operator()(int m, int n, int split, const float (&v)[4]) const {
        Vec4<float>::store(out + (size_t)split * stride + (size_t)m * ldo + n, v);
    }
    __device__ void put8(int, int, int, const float (&)[8]) const {}
};

// The 8 consecutive columns n0w + 32 j + 16 p + 8 (lane >> 5) + 0..7 of row block i for this lane: the
// registers of column groups 2p and 2p+1 trade halves between lanes l and l + 32.
template <int FM, int FN>
__device__ __forceinline__ void wide8(const f32x16 (&acc)[FM][FN], int i, int j, int p, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][8 * p + e]),
                                                        __float_as_uint(acc[i][j][8 * p + 4 + e]), false, false);
        v[e] = __uint_as_float(r[0]);
        v[4 + e] = __uint_as_float(r[1]);
    }
}

// Epilogues that read a tensor 8 values at a time (fetch8 / put8)
template <class E, class = void> struct WideLoads : std::false_type {};
template <class E> struct WideLoads<E, std::void_t<decltype(E::kLoads)>> : std::bool_constant<E::kWide && E::kLoads> {};
// The type of one fetch8 of a loads-epilogue (int where there is none)
template <class E, bool P> struct EpiIn { typedef int type; };
template <class E> struct EpiIn<E, true> { typedef typename E::vec8 type; };

// The inputs of a loads-epilogue for RG row blocks from row block i0: in[ii][j][p] holds the 8 values at the
// columns the lane stores for row block i0 + ii (see wide8).
template <int RG, int FN, class E>
__device__ __forceinline__ void fetch_rows(typename E::vec8 (&in)[RG][FN][2], int i0,
                                           int m0, int n0, int M, int N, int lane, const E& epi) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int m = m0 + 32 * (i0 + ii) + l32, n = n0 + 32 * j + 16 * p + 8 * h;
                if (m < M && n < N) in[ii][j][p] = epi.fetch8(m, n);
            }
}
// The loads-epilogue of RG row blocks from i0, given their fetched inputs.
template <int FM, int FN, int RG, class E>
__device__ __forceinline__ void apply_rows(const f32x16 (&acc)[FM][FN], const typename E::vec8 (&in)[RG][FN][2],
                                           int i0, int m0, int n0, int split, int M, int N, int lane, const E& epi) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int i = i0 + ii;
                float v[8];
                wide8<FM, FN>(acc, i, j, p, v);
                const int m = m0 + 32 * i + l32, n = n0 + 32 * j + 16 * p + 8 * h;
                if (m < M && n < N) epi.put8(m, n, split, v, in[ii][j][p]);
            }
}

// Epilogue of an MFMA wave tile: FM x FN accumulators of 32 x 32 (operand-swapped
// layout: lane l holds row l % 32 and, in registers 4g..4g+3, columns
// 8g + 4(l / 32) + 0..3).  m0, n0: the wave tile's first row and column.
// RG: row blocks whose epilogue inputs are fetched together (FM by default; the
// persistent kernels, which keep more registers live, fetch half as many at once).
template <int FM, int FN, class E, int RG = FM>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], int m0, int n0, int split, int M, int N,
                                           int lane, const E& epi) {
    const int h = lane >> 5, l32 = lane & 31;
    if constexpr (E::kWide && E::kLoads) {
        // epilogues that read a tensor: issue every load of RG row blocks first, so the
        // tile waits for memory once per group instead of once per column group
        static_assert(FM % RG == 0, "row groups must divide the row blocks");
#pragma unroll
        for (int i0 = 0; i0 < FM; i0 += RG) {
            typename E::vec8 in[RG][FN][2];
            fetch_rows<RG, FN, E>(in, i0, m0, n0, M, N, lane, epi);
            apply_rows<FM, FN, RG, E>(acc, in, i0, m0, n0, split, M, N, lane, epi);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + 32 * i + l32;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (E::kWide) {
                // registers of column groups 2p and 2p+1 trade halves: lanes 0..31 end up with
                // columns 16p + 0..7, lanes 32..63 with columns 16p + 8..15
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][8 * p + e]),
                                                                        __float_as_uint(acc[i][j][8 * p + 4 + e]),
                                                                        false, false);
                        v[e] = __uint_as_float(r[0]);
                        v[4 + e] = __uint_as_float(r[1]);
                    }
                    const int n = n0 + 32 * j + 16 * p + 8 * h;
                    if (m < M && n < N) epi.put8(m, n, split, v);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + 32 * j + 8 * g + 4 * h;
                    if (m < M && n < N) {
                        float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                      acc[i][j][4 * g + 3]};
                        epi(m, n, split, v);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ LM-head epilogues (16-bit compute dtypes)
// The cross-entropy needs, per row of logits z, lse = log sum exp z and z[target].  The LM-head GEMM
// forms them from its accumulators, so no pass over the [N, V] logits is needed for the loss: per row and
// per wave column block (32 FN columns), the max of z log2(e) and the sum of 2^(z log2(e) - max), and the
// logit at the row's target when the block holds it.  Statistics use the bf16-rounded logits, the values
// the backward turns into dz, so loss and gradient see the same logits (the shift is the max of the
// unrounded values: any shift near the max keeps the sum in range, and the merge is exact for any shift).
constexpr float kLog2eF = 1.4426950408889634f;

// Max and sum over lanes l and l ^ 32 (the two halves of one accumulator row).  The swap leaves lanes
// 0..31 with (own, partner) and lanes 32..63 with (partner, own); both orders give the same result.
__device__ __forceinline__ float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Detects epilogues that take the whole wave tile (kTile) instead of per-element stores.
template <class E, class = void> struct TileEpi : std::false_type {};
template <class E> struct TileEpi<E, std::void_t<decltype(E::kTile)>> : std::bool_constant<E::kTile> {};

// Round the 16 accumulators of one 32x32 block to T and back (one packed conversion per pair).
template <typename T>
__device__ __forceinline__ void round16(const f32x16& a, float (&z)[16]) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) round2<T>(a[r], a[r + 1], z[r], z[r + 1]);
}

template <typename T>
struct ECeStats {
    static constexpr bool kTile = true;
    T* out;                  // [M][ldo] rounded logits, or null (not stored)
    int ldo;
    float2* part;            // [nblk][M]: a wave's 32 rows of one block are 256 contiguous bytes
    int nblk;
    float* zt;               // [M]
    const int32_t* targets;  // [M]
    SoftCap cap;

    // acc is the kernel's accumulator of this tile, dead after the epilogue: a soft-cap rewrites it in place
    template <int FM, int FN>
    __device__ void tile(f32x16 (&acc)[FM][FN], int m0, int n0, int M, int N, int lane) const {
        const int h = lane >> 5, l32 = lane & 31;
        if (cap.c > 0.0f) {                       // uniform: the soft-capped variant
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = softcap_fwd(acc[i][j][r], cap);
        }
        // the rounded logits leave first, so their stores drain while the statistics are formed
        if (out) store_tile<FM, FN>(acc, m0, n0, 0, M, N, lane, EStoreCd<T>{out, ldo});
        if (n0 >= N) return;                      // wave-uniform: the block lies past a ragged vocab edge
        const bool full = n0 + 32 * FN <= N;      // wave-uniform: no column of the block is past the edge
        const int blk = n0 / (32 * FN);
        int tv[FM];  // every row's target, fetched before any is needed (one memory wait per tile)
#pragma unroll
        for (int i = 0; i < FM; ++i) tv[i] = m0 + 32 * i + l32 < M ? targets[m0 + 32 * i + l32] : -1;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + 32 * i + l32;
            float z[FN][16];
#pragma unroll
            for (int j = 0; j < FN; ++j) round16<T>(acc[i][j], z[j]);
            if (!full) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (n0 + 32 * j + 8 * (r >> 2) + 4 * h + (r & 3) >= N) z[j][r] = -INFINITY;
            }
            float mx = z[0][0];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, z[j][r]);
            mx = pair_max(mx) * kLog2eF;
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(z[j][r] * kLog2eF - mx);
            sum = pair_sum(sum);
            if (m < M && h == 0) part[(size_t)blk * M + m] = make_float2(mx, sum);
            // the target logit: only a lane whose half-row holds the target column takes this branch
            // (rare: the block is 32 FN of the vocab's columns)
            const int c = tv[i] - n0;
            if (c >= 0 && c < 32 * FN && ((c >> 2) & 1) == h && m < M) {
                float v = 0.0f;
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (c == 32 * j + 8 * (r >> 2) + 4 * h + (r & 3)) v = z[j][r];
                zt[m] = v;
            }
        }
    }
};

// dz = grad_scale * inv_valid * (softmax(z) - onehot(target)) from recomputed logits, rounded to T
// first exactly as the stored logits are, so the result equals the stored-logit backward's.
template <typename T>
struct EDz {
    static constexpr bool kTile = true;
    T* out;
    int ldo;
    const float* lse;
    const int32_t* targets;
    const float* inv_valid;
    float grad_scale;
    SoftCap cap;

    template <int FM, int FN>
    __device__ void tile(f32x16 (&acc)[FM][FN], int m0, int n0, int M, int N, int lane) const {
        const int h = lane >> 5, l32 = lane & 31;
        const bool capped = cap.c > 0.0f;         // uniform
        if (capped) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = softcap_fwd(acc[i][j][r], cap);
        }
        // every row's target and log2-domain lse first (one memory wait per tile)
        int tv[FM];
        float l2v[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + 32 * i + l32;
            tv[i] = m < M ? targets[m] : -1;
            l2v[i] = m < M ? lse[m] : 0.0f;
        }
        const float kv = grad_scale * (*inv_valid);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + 32 * i + l32, t = tv[i];
            const bool valid = t >= 0 && t < N;
            const float k = valid ? kv : 0.0f, l2 = valid ? l2v[i] * kLog2eF : 0.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    float v[8];
                    wide8<FM, FN>(acc, i, j, p, v);
                    const int n = n0 + 32 * j + 16 * p + 8 * h;
                    float z[8];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) round2<T>(v[e], v[e + 1], z[e], z[e + 1]);
                    float r[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = valid ? k * __builtin_amdgcn_exp2f(z[e] * kLog2eF - l2) : 0.0f;
                    // the target column (rare): k (p - 1) instead of k p, the same expression as ce_bwd's
                    if (t >= n && t < n + 8) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (n + e == t) r[e] = k * (__builtin_amdgcn_exp2f(z[e] * kLog2eF - l2) - 1.0f);
                    }
                    if (capped) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) r[e] = r[e] * softcap_grad(z[e], cap);
                    }
                    if (m < M && n < N) st8(out + (size_t)m * ldo + n, r);
                }
        }
    }
};

// ------------------------------------------------------------------ qkv epilogue: RoPE + QK-norm (16-bit)
// The qkv projection's output leaves already rotated and normalised ("nanochat 项目深度分析" §2.1 items 1-2):
// for token m (position t = m mod T) and each q or k head, pair (i, i + 64) is rotated by the angle of
// (t, i) as y_i = x_i cos + x_{i+64} sin, y_{i+64} = -x_i sin + x_{i+64} cos, and the head is divided by
// its RMS, sqrt(mean(y^2) + eps).  The rotation preserves each pair's norm, so the RMS is taken from the
// unrotated accumulators (equal up to rounding).  The head is rounded to bf16 once, at the store; 1/rms
// is saved for the backward.  With the 4 x 2 wave grid a wave owns 128 columns = one head, and in the
// accumulator layout the pair (i, i + 64) sits in one lane (column blocks j and j + 2), so everything is
// lane-local except the head sum, which adds the two lane halves of a row.
template <typename O>  // the stored type (bf16 or f16)
struct ERopeNorm {
    static constexpr bool kTile = true;
    O* out;
    int ldo;
    const float* cosv;   // [T][64]
    const float* sinv;
    float* rstdq;        // [M][H]
    float* rstdk;        // [M][Hkv]
    int T, H, Hkv;
    float eps;

    // 8 consecutive columns (16 p + 8 h .. + 7 of a 32-column block) of a per-lane array in the accumulator
    // layout: registers of column groups 2p and 2p+1 trade halves between lanes l and l + 32
    __device__ static void swap8(const float (&y)[16], int p, float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[8 * p + e]),
                                                            __float_as_uint(y[8 * p + 4 + e]), false, false);
            v[e] = __uint_as_float(r[0]);
            v[4 + e] = __uint_as_float(r[1]);
        }
    }

    template <int FM, int FN>
    __device__ void tile(const f32x16 (&acc)[FM][FN], int m0, int n0, int M, int N, int lane) const {
        static_assert(FN == 4, "a wave must own one 128-column head");
        if (n0 >= N) return;                 // wave-uniform: past the last head
        const int head = n0 >> 7;
        if (head >= H + Hkv) {               // v head: stored as computed
            store_tile<FM, FN>(acc, m0, n0, 0, M, N, lane, EStoreCd<O>{out, ldo});
            return;
        }
        const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + 32 * i + l32;
            const bool live = m < M;
            const int t = (live ? m : 0) % T;
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) ss += acc[i][j][r] * acc[i][j][r];
            const float rs = 1.0f / sqrtf(pair_sum(ss) * (1.0f / 128.0f) + eps);
            if (live && h == 0) {
                if (head < H) rstdq[(size_t)m * H + head] = rs;
                else rstdk[(size_t)m * Hkv + head - H] = rs;
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // this lane's cos / sin: pair index 32 j + 8 g + 4 h + e sits in register 4 g + e of block j
                float cs[16], sn[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 c4 = *reinterpret_cast<const float4*>(cosv + t * 64 + 32 * j + 8 * g + 4 * h);
                    const float4 s4 = *reinterpret_cast<const float4*>(sinv + t * 64 + 32 * j + 8 * g + 4 * h);
                    cs[4 * g] = c4.x; cs[4 * g + 1] = c4.y; cs[4 * g + 2] = c4.z; cs[4 * g + 3] = c4.w;
                    sn[4 * g] = s4.x; sn[4 * g + 1] = s4.y; sn[4 * g + 2] = s4.z; sn[4 * g + 3] = s4.w;
                }
                float y1[16], y2[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x1 = acc[i][j][r], x2 = acc[i][j + 2][r];
                    y1[r] = (x1 * cs[r] + x2 * sn[r]) * rs;
                    y2[r] = (-x1 * sn[r] + x2 * cs[r]) * rs;
                }
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    float v1[8], v2[8];
                    swap8(y1, p, v1);
                    swap8(y2, p, v2);
                    if (live) {
                        O* row = out + (size_t)m * ldo + n0 + 16 * p + 8 * h;
                        st8(row + 32 * j, v1);
                        st8(row + 32 * (j + 2), v2);
                    }
                }
            }
        }
    }
};

template <int FM, int FN, class E, int RG = FM>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[FM][FN], int m0, int n0, int split, int M, int N,
                                         int lane, const E& epi) {
    if constexpr (TileEpi<E>::value) epi.template tile<FM, FN>(acc, m0, n0, M, N, lane);
    else store_tile<FM, FN, E, RG>(acc, m0, n0, split, M, N, lane, epi);
}

// ------------------------------------------------------------------ tile order
// Each XCD takes a contiguous range of tiles (xcd_remap, so shared A / B tiles stay in
// one L2), walked in bands of group_m tile-rows (a per-call choice: GemmDesc::group_m).

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    int in_group = group_m * tiles_n;
    int gid = t / in_group;
    int first_m = gid * group_m;
    int gsz = min(tiles_m - first_m, group_m);
    int r = t % in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// ------------------------------------------------------------------ LDS layouts (bf16)
// A K-strided operand (element (r, k) at P[k*ld + r]) is kept in LDS in its
// natural layout, [k][R r] in 16-byte chunks along r, and the MFMA fragment (8
// consecutive k of one r) is read with two ds_read_b64_tr_b16.  A transposing
// read of one 16-lane group covers 4 consecutive k rows x 32 bytes; the chunk
// index is XOR-ed with ((k & 3) << 2) so those 4 rows land in 4 different
// 64-byte bank groups.
__device__ __forceinline__ int mn_chunk(int k, int c, int R) { return k * (R / 8) + (c ^ ((k & 3) << 2)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// MFMA fragment of lane `lane` from a [k][R] tile: operand row r0 + (lane & 31),
// k = kk*16 + 8h .. +7 (h = lane >> 5).  ds_read_b64_tr_b16: lane i of a 16-lane
// group receives element e of the 4-value row addressed by lane 4e + i/4, at
// position i % 4.
template <int R>
__device__ __forceinline__ bf16x8 frag_mn(const bf16* S, int r0, int kk, int lane) {
    const int h = lane >> 5;
    const int sl = lane & 15;
    const int r = r0 + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
    const int c = r >> 3, o = r & 7;
    const int k = kk * 16 + 8 * h + (sl >> 2);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + mn_chunk(k, c, R) * 8 + o));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + mn_chunk(k + 4, c, R) * 8 + o));
    s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------------ bf16 MFMA kernel, four-stage ring
// Stages of 32 k in a ring of four LDS buffers, filled straight from memory
// three stages ahead.  The barrier that publishes stage s+1 sits between the
// two k-steps of stage s: after it, the first fragments of stage s+1 are read
// while the last MFMAs of stage s run, so no MFMA waits on a cold LDS read.
// The barrier is a bare s_barrier after explicit waits: each wave's own loads
// of stage s+1 (the two later stages stay in flight) and its own LDS reads
// (stage s-1's buffer is refilled right after the barrier).
//
// 32-deep tiles: K-contiguous [R][32] (4 chunks of 16 bytes per row, chunk
// XOR-ed with (row >> 2) & 3, so 16 consecutive rows hit 16 distinct bank
// groups); K-strided [32 k][R] in the mn_chunk layout.
__device__ __forceinline__ int lds_chunk32(int row, int ch) { return row * 4 + (ch ^ ((row >> 2) & 3)); }

template <int R, bool KC, int NW>
struct DmaTile32 {
    static constexpr int CPR = R / 8;                    // 16-byte chunks per k-row (MN layout)
    static constexpr int NI = R * 4 / (64 * NW);         // wave-instructions per wave and stage
    static_assert(NI >= 1 && (64 * NW / CPR) % 4 == 0, "tile too small for the wave count");
    unsigned vo;
    int step;
    int w;

    __device__ __forceinline__ void init(int ld, int tid) {
        const int lane = tid & 63;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        if constexpr (KC) {
            // chunk q = 64 (w + NW i) + lane: row q / 4 (advances 16 NW per i), slot q % 4;
            // (row >> 2) & 3 = (lane >> 4) & 3 for every i
            const int row = 16 * w + (lane >> 2);
            const int ch = (lane & 3) ^ ((lane >> 4) & 3);
            vo = (unsigned)(row * ld * 2 + ch * 16);
            step = 16 * NW * ld * 2;
        } else {
            const int k = (64 * w + lane) / CPR;
            const int c = (lane % CPR) ^ ((k & 3) << 2);
            vo = (unsigned)(k * ld * 2 + c * 16);
            step = (64 * NW / CPR) * ld * 2;
        }
    }
    __device__ __forceinline__ void load(const bf16* __restrict__ P, int ld, int r0, int rmax, int k0, bool valid,
                                         bf16* S) const {
        const bf16* base;
        unsigned bytes;
        if constexpr (KC) {
            base = P + (size_t)r0 * ld + k0;
            bytes = (unsigned)(((min(rmax - r0, R) - 1) * ld + 32) * 2);
        } else {
            base = P + (size_t)k0 * ld + r0;
            bytes = (unsigned)((31 * ld + min(rmax - r0, R)) * 2);
        }
        if (!valid) bytes = 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(S + 64 * (w + NW * i) * 8), 16, vo, i * step, 0,
                                                     0);
    }
};

template <int R, bool KC>
__device__ __forceinline__ bf16x8 frag32(const bf16* S, int r0, int kk, int lane) {
    if constexpr (KC) {
        const int row = r0 + (lane & 31);
        return *reinterpret_cast<const bf16x8*>(S + lds_chunk32(row, kk * 2 + (lane >> 5)) * 8);
    } else {
        return frag_mn<R>(S, r0, kk, lane);
    }
}

// ------------------------------------------------------------------ fp8 operands (F8 kernels)
// An fp8 (OCP E4M3) operand row is moved and laid out in LDS exactly as a bf16 row of half the length: a
// 64-byte stage row holds 64 k.  v_mfma_scale_f32_32x32x64_f8f6f4 takes per lane the 16-byte chunks hh and
// 2 + hh of its row (hh the lane half) -- the two fragments the bf16 k-steps 0 and 1 read -- so one MFMA
// covers the stage.  Its block scales are left at 1 (E8M0 127); the per-row scales of both operands multiply
// the accumulators before the epilogue (dequant_rows).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 cat_frag(bf16x8 lo, bf16x8 hi) {
    const u32x4 a = __builtin_bit_cast(u32x4, lo), b = __builtin_bit_cast(u32x4, hi);
    const i32x8 r = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    return r;
}
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& x, const i32x8& y, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
}
// acc[i][j][e] (row m0 + 32 i + l32, column n0 + 32 j + 8 (e >> 2) + 4 h + (e & 3)) *= sa[row] sb[column]
template <int FM, int FN>
__device__ __forceinline__ void dequant_rows(f32x16 (&acc)[FM][FN], int m0, int n0, int M, int N, int lane,
                                             const float* __restrict__ sa, const float* __restrict__ sb) {
    const int h = lane >> 5, l32 = lane & 31;
    float ra[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) ra[i] = m0 + 32 * i + l32 < M ? sa[m0 + 32 * i + l32] : 0.0f;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + 32 * j + 8 * g + 4 * h;   // N is a multiple of 4: a group is all in or all out
            float cb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (n < N) Vec4<float>::load(sb + n, cb);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] *= ra[i] * cb[e];
        }
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BK, class E, bool F8 = false, typename H = bf16>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
gemm_bf16_mfma_ring(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                    int k_split, int group_m, E epi_, int64_t sA, int64_t sB, const float* __restrict__ rsa,
                    const float* __restrict__ rsb)
{
    // batched GEMMs: item blockIdx.z reads A + z sA and B + z sB and writes through its shifted epilogue
    A += blockIdx.z * sA;
    B += blockIdx.z * sB;
    const E epi = epi_at(epi_, blockIdx.z);
    __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB0[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB1[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA2[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB2[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA3[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB3[BN * 32];
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    constexpr int NL = DmaTile32<BM, AK, NW>::NI + DmaTile32<BN, BK, NW>::NI;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WGN, wn = w % WGN, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 32;

    DmaTile32<BM, AK, NW> da;
    DmaTile32<BN, BK, NW> db;
    da.init(lda, tid);
    db.init(ldb, tid);
    auto dma = [&](int kt, bf16* sA, bf16* sB) {
        da.load(A, lda, m0, M, kbeg + kt * 32, kt < nk, sA);
        db.load(B, ldb, n0, N, kbeg + kt * 32, kt < nk, sB);
    };
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, const bf16* sA, const bf16* sB, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag32<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag32<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    auto mma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mfma16<H>(fb[buf][j], fa[buf][i], acc[i][j]);
    };
    // Instruction order inside one k-step's region: each MFMA is followed by at most one
    // load and one fragment read, so neither memory queue receives a burst.  None of the
    // region's MFMAs depends on its reads (they fill the other fragment buffer).
    auto interleave = [&](auto with_loads) {
        constexpr int NDS = (AK ? FM : 2 * FM) + (BK ? FN : 2 * FN);  // LDS read instructions of one k-step
        constexpr int NMF = FM * FN;
        constexpr int NV = decltype(with_loads)::value ? NL : 0;
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
            if constexpr (NV > 0) if (q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one load
            if (q < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one fragment read
        }
        if constexpr (NDS > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NMF, 0);
        if constexpr (NV > NMF) __builtin_amdgcn_sched_group_barrier(0x020, NV - NMF, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // own loads of the next stage done (the two later stages may still fly, and X later loads of the epilogue's
    // input: vector-memory loads complete in issue order), own LDS reads done, then the barrier
    auto sync_next = [&](auto X) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL + decltype(X)::value) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // one stage: its loads three stages ahead, k-step 0, publish the next stage, k-step 1
    auto stage = [&](int kt, const bf16* cA, const bf16* cB, const bf16* nA, const bf16* nB, bf16* xA, bf16* xB,
                     auto X) {
        dma(kt + 3, xA, xB);
        lfrag(1, cA, cB, 1);
        mma(0);
        interleave(std::true_type{});
        sync_next(X);
        lfrag(0, nA, nB, 0);
        mma(1);
        interleave(std::false_type{});
    };
    using X0 = std::integral_constant<int, 0>;
    // An epilogue that reads a tensor has it fetched into registers under the MFMAs of the last three stages:
    // FM x FN x 2 loads per lane, every one issued (addresses clamped into the tensor) so the wait counts hold.
    constexpr bool kPf = WideLoads<E>::value && !F8;
    using XE = std::integral_constant<int, kPf ? FM * FN * 2 : 0>;
    typename EpiIn<E, kPf>::type pin[FM][FN][2];

    if constexpr (F8) {
        // fp8: one MFMA per (i, j) and stage.  The stage's A fragments are reloaded with the next stage's
        // right after their last MFMA; the B fragments alternate between two buffers.
        i32x8 a8[FM], b8[2][FN];
        auto lfa8 = [&](int i, const bf16* S) {
            a8[i] = cat_frag(frag32<BM, AK>(S, wm * WM + 32 * i, 0, lane), frag32<BM, AK>(S, wm * WM + 32 * i, 1, lane));
        };
        auto lfb8 = [&](int buf, const bf16* S) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b8[buf][j] = cat_frag(frag32<BN, BK>(S, wn * WN + 32 * j, 0, lane),
                                      frag32<BN, BK>(S, wn * WN + 32 * j, 1, lane));
        };
        auto stage8 = [&](int kt, int cb, const bf16* nA, const bf16* nB, bf16* xA, bf16* xB) {
            dma(kt + 3, xA, xB);
            sync_next(X0{});
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f8(b8[cb][j], a8[i], acc[i][j]);
                lfa8(i, nA);
            }
            lfb8(cb ^ 1, nB);
        };
        dma(0, sA0, sB0);
        dma(1, sA1, sB1);
        dma(2, sA2, sB2);
        sync_next(X0{});
#pragma unroll
        for (int i = 0; i < FM; ++i) lfa8(i, sA0);
        lfb8(0, sB0);
        for (int kt = 0; kt < nk; kt += 4) {
            stage8(kt, 0, sA1, sB1, sA3, sB3);
            stage8(kt + 1, 1, sA2, sB2, sA0, sB0);
            stage8(kt + 2, 0, sA3, sB3, sA1, sB1);
            stage8(kt + 3, 1, sA0, sB0, sA2, sB2);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        dequant_rows<FM, FN>(acc, m0 + wm * WM, n0 + wn * WN, M, N, lane, rsa, rsb);
    } else {
        dma(0, sA0, sB0);
        dma(1, sA1, sB1);
        dma(2, sA2, sB2);
        sync_next(X0{});
        lfrag(0, sA0, sB0, 0);
        const int kl = kPf ? (nk + 3) / 4 * 4 - 4 : nk;   // stages before the last block of four
        for (int kt = 0; kt < kl; kt += 4) {
            stage(kt, sA0, sB0, sA1, sB1, sA3, sB3, X0{});
            stage(kt + 1, sA1, sB1, sA2, sB2, sA0, sB0, X0{});
            stage(kt + 2, sA2, sB2, sA3, sB3, sA1, sB1, X0{});
            stage(kt + 3, sA3, sB3, sA0, sB0, sA2, sB2, X0{});
        }
        if constexpr (kPf) {
            stage(kl, sA0, sB0, sA1, sB1, sA3, sB3, X0{});
            const int mw = m0 + wm * WM, nw = n0 + wn * WN;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        pin[i][j][p] = epi.fetch8(min(mw + 32 * i + l32, M - 1),
                                                  min(nw + 32 * j + 16 * p + 8 * h, N - 8));
            stage(kl + 1, sA1, sB1, sA2, sB2, sA0, sB0, XE{});
            stage(kl + 2, sA2, sB2, sA3, sB3, sA1, sB1, XE{});
            stage(kl + 3, sA3, sB3, sA0, sB0, sA2, sB2, XE{});
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the loads past the end before the stores
    }

    if constexpr (kPf)
        apply_rows<FM, FN, FM, E>(acc, pin, 0, m0 + wm * WM, n0 + wn * WN, split, M, N, lane, epi);
    else
        epilogue<FM, FN>(acc, m0 + wm * WM, n0 + wn * WN, split, M, N, lane, epi);
}

// ------------------------------------------------------------------ persistent four-stage ring
// The ring kernel made persistent: a workgroup walks work items (k split,
// tile) number r G + slot for rounds r = 0, 1, ..., where G is the grid size
// and slot the workgroup's XCD-contiguous position, and its loads stream three
// stages ahead across item boundaries, so the first stages of the next item
// are in flight while the current item's epilogue stores run.  Each item runs
// a multiple of four stages (stages past its k range read zeros).  Loads and
// stores share the vector-memory counter and may complete out of order, so the
// first wait after an epilogue waits for everything.
template <int BM, int BN, int WGM, int WGN, bool AK, bool BK, class E, typename H = bf16>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
gemm_bf16_mfma_pring(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                     int k_split, int splits, int group_m, E epi)
{
    __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB0[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB1[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA2[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB2[BN * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sA3[BM * 32];
    __shared__ __attribute__((aligned(1024))) bf16 sB3[BN * 32];
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    constexpr int NL = DmaTile32<BM, AK, NW>::NI + DmaTile32<BN, BK, NW>::NI;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WGN, wn = w % WGN, h = lane >> 5, l32 = lane & 31;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN, tiles = tiles_m * tiles_n;
    const int items = tiles * splits;
    const int G = gridDim.x, slot = xcd_remap(blockIdx.x, G);

    struct Item {
        int m0, n0, split, kbeg, nk4;
        int nk;
        bool valid;
    };
    auto item = [&](int r) {
        Item it;
        const int L = r * G + slot;
        it.valid = L < items;
        const int Lc = it.valid ? L : 0;
        it.split = Lc / tiles;
        int tm, tn;
        tile_coords(Lc % tiles, tiles_m, tiles_n, group_m, tm, tn);
        it.m0 = tm * BM;
        it.n0 = tn * BN;
        it.kbeg = it.split * k_split;
        it.nk = min(k_split, K - it.kbeg) / 32;
        it.nk4 = (it.nk + 3) & ~3;
        return it;
    };

    DmaTile32<BM, AK, NW> da;
    DmaTile32<BN, BK, NW> db;
    da.init(lda, tid);
    db.init(ldb, tid);
    auto dma_at = [&](const Item& it, int kt, bf16* sA, bf16* sB) {
        const bool v = it.valid && kt < it.nk;
        da.load(A, lda, it.m0, M, it.kbeg + kt * 32, v, sA);
        db.load(B, ldb, it.n0, N, it.kbeg + kt * 32, v, sB);
    };
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, const bf16* sA, const bf16* sB, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag32<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag32<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };
    f32x16 acc[FM][FN];
    auto mma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mfma16<H>(fb[buf][j], fa[buf][i], acc[i][j]);
    };
    // Instruction order inside one k-step's region: each MFMA is followed by at most one
    // load and one fragment read, so neither memory queue receives a burst.  None of the
    // region's MFMAs depends on its reads (they fill the other fragment buffer).
    auto interleave = [&](auto with_loads) {
        constexpr int NDS = (AK ? FM : 2 * FM) + (BK ? FN : 2 * FN);  // LDS read instructions of one k-step
        constexpr int NMF = FM * FN;
        constexpr int NV = decltype(with_loads)::value ? NL : 0;
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
            if constexpr (NV > 0) if (q < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one load
            if (q < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one fragment read
        }
        if constexpr (NDS > NMF) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NMF, 0);
        if constexpr (NV > NMF) __builtin_amdgcn_sched_group_barrier(0x020, NV - NMF, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto sync_next = [&](bool drain) {
        if (drain) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    Item cur = item(0), nxt = item(1);
    auto stage = [&](int kt, const bf16* cA, const bf16* cB, const bf16* nA, const bf16* nB, bf16* xA, bf16* xB) {
        if (kt + 3 < cur.nk4) dma_at(cur, kt + 3, xA, xB);
        else dma_at(nxt, kt + 3 - cur.nk4, xA, xB);
        lfrag(1, cA, cB, 1);
        mma(0);
        interleave(std::true_type{});
        sync_next(kt == 0);
        lfrag(0, nA, nB, 0);
        mma(1);
        interleave(std::false_type{});
    };

    dma_at(cur, 0, sA0, sB0);
    dma_at(cur, 1, sA1, sB1);
    dma_at(cur, 2, sA2, sB2);
    sync_next(true);
    lfrag(0, sA0, sB0, 0);
    for (int r = 0; cur.valid; ++r) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
        for (int kt = 0; kt < cur.nk4; kt += 4) {
            stage(kt, sA0, sB0, sA1, sB1, sA3, sB3);
            stage(kt + 1, sA1, sB1, sA2, sB2, sA0, sB0);
            stage(kt + 2, sA2, sB2, sA3, sB3, sA1, sB1);
            stage(kt + 3, sA3, sB3, sA0, sB0, sA2, sB2);
        }
        epilogue<FM, FN, E, (FM >= 2 ? FM / 2 : FM)>(acc, cur.m0 + wm * WM, cur.n0 + wn * WN, cur.split, M, N,
                                                    lane, epi);
        cur = nxt;
        nxt = item(r + 2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ fp32 SIMT kernel
template <bool AK, bool BK, class E>
__global__ void __launch_bounds__(256)
gemm_f32_simt(const float* __restrict__ A, const float* __restrict__ B, int M, int N, int K, int lda, int ldb,
              int k_split, E epi)
{
    __shared__ float sA[16][68];
    __shared__ float sB[16][68];
    const int tid = threadIdx.x;
    const int tiles_m = (M + 63) / 64;
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * 64, n0 = tn * 64;
    const int split = blockIdx.y;
    const int kbeg = split * k_split, kend = min(K, kbeg + k_split);
    const int tr = tid >> 4, tc = tid & 15;
    float acc[4][4] = {};

    for (int k0 = kbeg; k0 < kend; k0 += 16) {
        if (AK) {
            int row = tid >> 2, kq = (tid & 3) * 4;
            int gm = min(m0 + row, M - 1);
            float4 t = *reinterpret_cast<const float4*>(A + (size_t)gm * lda + k0 + kq);
            sA[kq][row] = t.x; sA[kq + 1][row] = t.y; sA[kq + 2][row] = t.z; sA[kq + 3][row] = t.w;
        } else {
            int kr = tid >> 4, mq = (tid & 15) * 4;
            int gm = min(m0 + mq, M - 4);
            float4 t = *reinterpret_cast<const float4*>(A + (size_t)(k0 + kr) * lda + gm);
            sA[kr][mq] = t.x; sA[kr][mq + 1] = t.y; sA[kr][mq + 2] = t.z; sA[kr][mq + 3] = t.w;
        }
        if (BK) {
            int row = tid >> 2, kq = (tid & 3) * 4;
            int gn = min(n0 + row, N - 1);
            float4 t = *reinterpret_cast<const float4*>(B + (size_t)gn * ldb + k0 + kq);
            sB[kq][row] = t.x; sB[kq + 1][row] = t.y; sB[kq + 2][row] = t.z; sB[kq + 3][row] = t.w;
        } else {
            int kr = tid >> 4, nq = (tid & 15) * 4;
            int gn = min(n0 + nq, N - 4);
            float4 t = *reinterpret_cast<const float4*>(B + (size_t)(k0 + kr) * ldb + gn);
            sB[kr][nq] = t.x; sB[kr][nq + 1] = t.y; sB[kr][nq + 2] = t.z; sB[kr][nq + 3] = t.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = sA[kk][tr * 4 + i]; b[i] = sB[kk][tc * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = m0 + tr * 4 + i, n = n0 + tc * 4;
        if (m < M && n < N) epi(m, n, split, acc[i]);
    }
}

// ------------------------------------------------------------------ host side
// compute units of the current device (queried once per process)
static int num_cus() {
    static int n = 0;
    if (n == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
    }
    return n;
}

template <class E> struct IsRope : std::false_type {};
template <typename T> struct IsRope<ERopeNorm<T>> : std::true_type {};

// H: the 16-bit operand type (bf16, or f16 in the fp16 compute mode)
template <int BM, int BN, bool AK, bool BK, typename H, class E>
static hipError_t run_mfma(const GemmDesc& d, E e, hipStream_t s) {
    const int splits = (d.K + d.k_split - 1) / d.k_split;
    const int tiles = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
    if constexpr (IsRope<E>::value) {
        if constexpr (BM == 256 && BN == 256) {
            if (d.loop != GemmLoop::Persist8Heads) return hipErrorInvalidValue;
            auto pk = gemm_bf16_mfma_pring<256, 256, 4, 2, AK, BK, E, H>;
            static int occ = 0;
            if (occ == 0) {
                hipError_t st = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(pk), 512, 0);
                if (st != hipSuccess) return st;
                if (occ < 1) occ = 1;
            }
            const int grid = std::min(tiles * splits, occ * num_cus());
            hipLaunchKernelGGL(pk, dim3(grid), dim3(512), 0, s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, d.K,
                               d.lda, d.ldb, d.k_split, splits, d.group_m, e);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    } else {
    if (d.loop == GemmLoop::Persist8Heads) return hipErrorInvalidValue;
    if (d.batch > 1 && d.loop != GemmLoop::Ring8) return hipErrorInvalidValue;  // batches run on the ring only
    if (d.loop == GemmLoop::Ring8) {
        if (d.batch > 1 && !BatchEpi<E>::value) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_bf16_mfma_ring<BM, BN, 2, 4, AK, BK, E, false, H>), dim3(tiles, splits, d.batch),
                           dim3(512), 0,
                           s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, d.K, d.lda, d.ldb, d.k_split, d.group_m, e,
                           (int64_t)d.sA, (int64_t)d.sB, nullptr, nullptr);
        return hipGetLastError();
    }
    const bool eight = d.loop == GemmLoop::Persist8;
    auto pk = eight ? gemm_bf16_mfma_pring<BM, BN, 2, 4, AK, BK, E, H> : gemm_bf16_mfma_pring<BM, BN, 2, 2, AK, BK, E, H>;
    const int nt = eight ? 512 : 256;
    static int resident[2] = {0, 0};  // workgroups per CU, from the occupancy query
    int& occ = resident[eight ? 1 : 0];
    if (occ == 0) {
        hipError_t st = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(pk), nt, 0);
        if (st != hipSuccess) return st;
        if (occ < 1) occ = 1;
    }
    const int grid = std::min(tiles * splits, occ * num_cus());
    hipLaunchKernelGGL(pk, dim3(grid), dim3(nt), 0, s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, d.K, d.lda,
                       d.ldb, d.k_split, splits, d.group_m, e);
    return hipGetLastError();
    }
}

// fp8 operands (NT, 256 x 256 tiles, no split): d.K, d.lda and d.ldb count fp8 elements; the kernels move the
// rows as bf16 rows of half the length.  Always the non-persistent eight-wave ring (the persistent kernels
// spill with the fp8 fragments), in the 4 x 2 wave grid for the RoPE epilogue (a wave owns a head).
template <class E>
static hipError_t run_f8(const GemmDesc& d, E e, hipStream_t s) {
    if (!d.rsa || !d.rsb || d.K % 128 || d.lda % 2 || d.ldb % 2 || d.tile != 0 || d.splits != 1 || d.batch != 1)
        return hipErrorInvalidValue;
    const int K = d.K / 2, lda = d.lda / 2, ldb = d.ldb / 2;
    const int tiles = ((d.M + 255) / 256) * ((d.N + 255) / 256);
    constexpr bool heads = IsRope<E>::value;
    hipLaunchKernelGGL((gemm_bf16_mfma_ring<256, 256, heads ? 4 : 2, heads ? 2 : 4, true, true, E, true>),
                       dim3(tiles, 1, 1), dim3(512), 0, s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, K, lda, ldb,
                       K, d.group_m, e, (int64_t)0, (int64_t)0, d.rsa, d.rsb);
    return hipGetLastError();
}

template <bool AK, bool BK, typename H, class E>
static hipError_t run_bf16(const GemmDesc& d, E e, hipStream_t s) {
    switch (d.tile) {
    case 0: return run_mfma<256, 256, AK, BK, H>(d, e, s);
    case 1: return run_mfma<256, 128, AK, BK, H>(d, e, s);
    default: return run_mfma<128, 128, AK, BK, H>(d, e, s);
    }
}

template <bool AK, bool BK, class E>
static hipError_t run_f32(const GemmDesc& d, E e, hipStream_t s) {
    int tiles = ((d.M + 63) / 64) * ((d.N + 63) / 64);
    dim3 grid(tiles, (d.K + d.k_split - 1) / d.k_split);
    hipLaunchKernelGGL((gemm_f32_simt<AK, BK, E>), grid, dim3(256), 0, s, (const float*)d.A, (const float*)d.B,
                       d.M, d.N, d.K, d.lda, d.ldb, d.k_split, e);
    return hipGetLastError();
}

// Only the (layout, epilogue) pairs of the block stack are instantiated:
//   NT  (x W^T, forward):           store, residual add, ReLU^2, CE statistics, dz, RoPE + QK-norm, split-K
//                                   partials (decode)
//   NN  (dY W, input gradients):    store, ReLU^2 backward, alpha in + beta v (Newton-Schulz)
//   TN  (dY^T X, weight gradients): fp32 gradient, split-K partial, store (Newton-Schulz X^T X)
template <typename T, bool AK, bool BK>
static hipError_t dispatch_epi(const GemmDesc& d, hipStream_t s) {
    auto run = [&](auto e) -> hipError_t {
        if constexpr (sizeof(T) == 2) {
            if constexpr (AK && BK && std::is_same<T, bf16>::value && !std::is_same<decltype(e), ESplitK>::value) {
                if (d.fp8) return run_f8(d, e, s);
            }
            if (d.fp8) return hipErrorInvalidValue;
            return run_bf16<AK, BK, T>(d, e, s);
        } else {
            if (d.fp8) return hipErrorInvalidValue;
            return run_f32<AK, BK>(d, e, s);
        }
    };
    if constexpr (AK && BK) {
        switch (d.epi) {
        case Epi::StoreCd: return run(EStoreCd<T>{(T*)d.out, d.ldo, d.sOut});
        case Epi::ResidualCd: return run(EResidual<T>{(T*)d.out, (const T*)d.in, d.ldo});
        case Epi::ReluSq: return run(EReluSq<T>{(T*)d.out, d.ldo});
        case Epi::SplitK: return run(ESplitK{(float*)d.out, d.ldo, d.split_stride});  // B-row decode products
        case Epi::CeStats:
            if constexpr (sizeof(T) == 2)
                return run(ECeStats<T>{(T*)d.out, d.ldo, (float2*)d.part, d.nblk, d.zt, d.targets, d.cap});
            break;
        case Epi::Dz:
            if constexpr (sizeof(T) == 2)
                return run(EDz<T>{(T*)d.out, d.ldo, d.lse, d.targets, d.inv_valid, d.grad_scale, d.cap});
            break;
        case Epi::RopeNorm:
            if constexpr (sizeof(T) == 2) {
                if (d.T <= 0 || d.H <= 0 || d.Hkv <= 0 || !d.cosv || !d.sinv || !d.rstdq || !d.rstdk ||
                    d.N != (d.H + 2 * d.Hkv) * 128 || d.tile != 0)
                    return hipErrorInvalidValue;
                return run(ERopeNorm<T>{(T*)d.out, d.ldo, d.cosv, d.sinv, d.rstdq, d.rstdk, d.T, d.H, d.Hkv, d.eps});
            }
            break;
        default: break;
        }
    } else if constexpr (AK && !BK) {
        switch (d.epi) {
        case Epi::StoreCd: return run(EStoreCd<T>{(T*)d.out, d.ldo, d.sOut});
        case Epi::ReluSqBwd: return run(EReluSqBwd<T>{(T*)d.out, (const T*)d.in, d.ldo});
        case Epi::Axpby:
            if constexpr (std::is_same<T, bf16>::value)
                return run(EAxpby{(bf16*)d.out, (const bf16*)d.in, d.ldo, d.alpha, d.beta, d.sOut, d.sIn});
            break;
        default: break;
        }
    } else if constexpr (!AK && !BK) {
        switch (d.epi) {
        case Epi::StoreCd:  // the Newton-Schulz X^T X (bf16)
            if constexpr (std::is_same<T, bf16>::value) return run(EStoreCd<T>{(T*)d.out, d.ldo, d.sOut});
            break;
        case Epi::Grad: return run(EGrad{(float*)d.out, d.ldo, d.accumulate});
        case Epi::SplitK: return run(ESplitK{(float*)d.out, d.ldo, d.split_stride});
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_layout(const GemmDesc& d, hipStream_t s) {
    if (d.a_kcontig && d.b_kcontig) return dispatch_epi<T, true, true>(d, s);
    if (d.a_kcontig && !d.b_kcontig) return dispatch_epi<T, true, false>(d, s);
    if (!d.a_kcontig && !d.b_kcontig) return dispatch_epi<T, false, false>(d, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmDesc& in, hipStream_t s) {
    GemmDesc d = in;
    if (d.K <= 0 || d.K % 64 || d.M % 8 || d.N % 8 || d.M <= 0 || d.N <= 0 || d.splits < 1) return hipErrorInvalidValue;
    if (d.k_split <= 0) {
        if (d.K % d.splits || (d.K / d.splits) % 64) return hipErrorInvalidValue;
        d.k_split = d.K / d.splits;
    }
    if (d.k_split % 64) return hipErrorInvalidValue;
    if (d.epi != Epi::SplitK && d.k_split < d.K) return hipErrorInvalidValue;  // only SplitK writes partials
    if (d.dt == Dt::BF16) return dispatch_layout<bf16>(d, s);
    if (d.dt == Dt::F16) return dispatch_layout<f16>(d, s);
    return dispatch_layout<float>(d, s);
}

int gemm_wave_cols(const GemmDesc& d) {
    static const int bn[3] = {256, 128, 128};
    const int t = d.tile < 0 ? 0 : (d.tile > 2 ? 2 : d.tile);
    return bn[t] / (d.loop == GemmLoop::Persist4 || d.loop == GemmLoop::Persist8Heads ? 2 : 4);
}

const char* gemm_kernel_name(const GemmDesc& d) {
    int li = (d.a_kcontig ? 2 : 0) + (d.b_kcontig ? 1 : 0);
    if (d.dt == Dt::F32) return li == 3 ? "gemm_f32_nt" : (li == 2 ? "gemm_f32_nn" : "gemm_f32_tn");
    if (d.fp8) return "gemm_fp8_nt_256x256";
    static const char* names[2][3][3] = {
        {{"gemm_bf16_nt_256x256", "gemm_bf16_nt_256x128", "gemm_bf16_nt_128x128"},
         {"gemm_bf16_nn_256x256", "gemm_bf16_nn_256x128", "gemm_bf16_nn_128x128"},
         {"gemm_bf16_tn_256x256", "gemm_bf16_tn_256x128", "gemm_bf16_tn_128x128"}},
        {{"gemm_f16_nt_256x256", "gemm_f16_nt_256x128", "gemm_f16_nt_128x128"},
         {"gemm_f16_nn_256x256", "gemm_f16_nn_256x128", "gemm_f16_nn_128x128"},
         {"gemm_f16_tn_256x256", "gemm_f16_tn_256x128", "gemm_f16_tn_128x128"}}};
    int r = li == 3 ? 0 : (li == 2 ? 1 : 2);
    int t = d.tile < 0 ? 0 : (d.tile > 2 ? 2 : d.tile);
    return names[d.dt == Dt::F16 ? 1 : 0][r][t];
}

// ------------------------------------------------------------------ split-K reduction
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, size_t stride, float* __restrict__ g, size_t n4,
                     int accumulate)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 acc = accumulate ? reinterpret_cast<const float4*>(g)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    // partials added in split order; four loads in flight at a time
    int sidx = 0;
    for (; sidx + 4 <= splits; sidx += 4) {
        float4 p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = reinterpret_cast<const float4*>(part + (size_t)(sidx + u) * stride)[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) { acc.x += p[u].x; acc.y += p[u].y; acc.z += p[u].z; acc.w += p[u].w; }
    }
    for (; sidx < splits; ++sidx) {
        float4 p = reinterpret_cast<const float4*>(part + (size_t)sidx * stride)[i];
        acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    reinterpret_cast<float4*>(g)[i] = acc;
}

hipError_t launch_splitk_reduce(const float* part, int splits, size_t stride, float* grads, size_t n,
                                int accumulate, hipStream_t s) {
    size_t n4 = n / 4;
    dim3 grid((unsigned)((n4 + 255) / 256));
    hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, s, part, splits, stride, grads, n4, accumulate);
    return hipGetLastError();
}

}  // namespace ncgpt
