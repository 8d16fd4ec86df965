// GEMMs of the block stack: the bias-free linears y = x W^T (forward), their
// input gradients dx = dy W and weight gradients dW = dy^T x (backward).
//
// bf16 path: one MFMA kernel (v_mfma_f32_32x32x16_bf16, fp32 accumulation)
// for all three operand layouts.  Tiles of BM x BN x 64 are staged through
// LDS (two stages, XOR-swizzled 16-byte chunks), 4 waves per workgroup in a
// 2 x 2 grid.  Operands whose K index is not contiguous in memory (the
// token-major activations of a weight gradient, the [out,in] weight of an
// input gradient) are copied to LDS in their natural layout and their MFMA
// fragments are read with gfx950's transposing LDS load (ds_read_b64_tr_b16).
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
__device__ __forceinline__ void ld8(const bf16* p, float (&v)[8]) {
    const bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
}
__device__ __forceinline__ void st8(bf16* p, const float (&v)[8]) {
    bf16x8 t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(p) = t;
}

template <typename T> struct EStoreCd {
    static constexpr bool kWide = std::is_same<T, bf16>::value, kLoads = false;
    T* out; int ldo;
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        Vec4<T>::store(out + (size_t)m * ldo + n, v);
    }
    __device__ void put8(int m, int n, int, const float (&v)[8]) const { st8(out + (size_t)m * ldo + n, v); }
};
struct EStoreF32 {
    static constexpr bool kWide = false, kLoads = false;
    float* out; int ldo;
    __device__ void operator()(int m, int n, int, const float (&v)[4]) const {
        Vec4<float>::store(out + (size_t)m * ldo + n, v);
    }
    __device__ void put8(int, int, int, const float (&)[8]) const {}
};
template <typename T> struct EResidual {
    static constexpr bool kWide = std::is_same<T, bf16>::value, kLoads = true;
    T* out; const T* in; int ldo;
    __device__ bf16x8 fetch8(int m, int n) const { return *reinterpret_cast<const bf16x8*>(in + (size_t)m * ldo + n); }
    __device__ void put8(int m, int n, int, const float (&v)[8], const bf16x8& x) const {
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
// act = a^2 with a = relu(v) rounded to the compute dtype: the only stored output of
// the MLP's first linear; the backward recovers a as sqrt(act)
template <typename T> struct EReluSq {
    static constexpr bool kWide = std::is_same<T, bf16>::value, kLoads = false;
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
            const float r = (float)(bf16)fmaxf(v[i], 0.0f);
            s[i] = r * r;
        }
        st8(act + (size_t)m * ldo + n, s);
    }
};
// dh = dact * d(relu(h)^2)/dh = dact * 2 relu(h), with relu(h) = sqrt(act)
template <typename T> struct EReluSqBwd {
    static constexpr bool kWide = std::is_same<T, bf16>::value, kLoads = true;
    T* out; const T* act; int ldo;
    __device__ bf16x8 fetch8(int m, int n) const { return *reinterpret_cast<const bf16x8*>(act + (size_t)m * ldo + n); }
    __device__ void put8(int m, int n, int, const float (&v)[8], const bf16x8& x) const {
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

// Epilogue of an MFMA wave tile: FM x FN accumulators of 32 x 32 (operand-swapped
// layout: lane l holds row l % 32 and, in registers 4g..4g+3, columns
// 8g + 4(l / 32) + 0..3).  m0, n0: the wave tile's first row and column.
template <int FM, int FN, class E>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], int m0, int n0, int split, int M, int N,
                                           int lane, const E& epi) {
    const int h = lane >> 5, l32 = lane & 31;
    if constexpr (E::kWide && E::kLoads) {
        // epilogues that read a tensor: issue every load of the wave tile first, so the
        // tile waits for memory once instead of once per column group
        bf16x8 in[FM][FN][2];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int m = m0 + 32 * i + l32, n = n0 + 32 * j + 16 * p + 8 * h;
                    if (m < M && n < N) in[i][j][p] = epi.fetch8(m, n);
                }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
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
                    const int m = m0 + 32 * i + l32, n = n0 + 32 * j + 16 * p + 8 * h;
                    if (m < M && n < N) epi.put8(m, n, split, v, in[i][j][p]);
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

// ------------------------------------------------------------------ tile order
// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// gets a contiguous range of tiles (shared A / B tiles stay in one L2), then
// walk tiles in bands of group_m tile-rows (a per-call choice: GemmDesc::group_m).
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    constexpr int NX = 8;
    int per = (nwg + NX - 1) / NX;
    int xcd = wg % NX, local = wg / NX;
    int tall = nwg % NX;
    if (tall == 0) tall = NX;
    if (xcd < tall) return xcd * per + local;
    return tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    int in_group = group_m * tiles_n;
    int gid = t / in_group;
    int first_m = gid * group_m;
    int gsz = min(tiles_m - first_m, group_m);
    int r = t % in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// ------------------------------------------------------------------ LDS staging (bf16)
// An LDS tile holds R rows x 64 k (bf16): 8 chunks of 16 bytes per row.  The
// gfx950 LDS serves 16 lanes of a 16-byte access per cycle from 64 banks, so
// the 16 consecutive rows read together must cover all (row parity, chunk)
// pairs: the chunk index is XOR-ed with (row & 7) ^ ((row >> 3) & 1), which
// gives the even rows of a 16-row group 8 distinct chunks and the odd rows 8
// distinct chunks (bank-conflict counter reads 0 on the MFMA reads).
__device__ __forceinline__ int lds_chunk(int row, int ch) { return row * 8 + (ch ^ ((row & 7) ^ ((row >> 3) & 1))); }

// K-contiguous operand: element (r, k) at P[r*ld + k].
template <int R, int NT = 256> struct StageK {
    static constexpr int NC = R * 8 / NT;  // 16-byte chunks per thread
    u32x4 v[NC];
    __device__ __forceinline__ void load(const bf16* __restrict__ P, int ld, int r0, int rmax, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            int u = tid + NT * i;
            int row = u >> 3, ch = u & 7;
            int gr = min(r0 + row, rmax - 1);
            v[i] = *reinterpret_cast<const u32x4*>(P + (size_t)gr * ld + k0 + ch * 8);
        }
    }
    __device__ __forceinline__ void store(bf16* S, int tid) const {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            int u = tid + NT * i;
            int row = u >> 3, ch = u & 7;
            *reinterpret_cast<u32x4*>(S + lds_chunk(row, ch) * 8) = v[i];
        }
    }
};

// MN-contiguous operand: element (r, k) at P[k*ld + r].  The tile is kept in
// LDS in this natural layout, [64 k][R r] (16-byte chunks along r), and the
// MFMA fragment (8 consecutive k of one r) is read with two
// ds_read_b64_tr_b16.  A transposing read of one 16-lane group covers 4
// consecutive k rows x 32 bytes; the chunk index is XOR-ed with
// ((k & 3) << 2) so those 4 rows land in 4 different 64-byte bank groups.
__device__ __forceinline__ int mn_chunk(int k, int c, int R) { return k * (R / 8) + (c ^ ((k & 3) << 2)); }

template <int R, int NT = 256> struct StageMN {
    static constexpr int CPR = R / 8;            // 16-byte chunks per k row
    static constexpr int NC = 64 * CPR / NT;     // chunks per thread
    u32x4 v[NC];
    __device__ __forceinline__ void load(const bf16* __restrict__ P, int ld, int r0, int rmax, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            int u = tid + NT * i;
            int k = u / CPR, c = u % CPR;
            int gr = min(r0 + c * 8, rmax - 8);
            v[i] = *reinterpret_cast<const u32x4*>(P + (size_t)(k0 + k) * ld + gr);
        }
    }
    __device__ __forceinline__ void store(bf16* S, int tid) const {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            int u = tid + NT * i;
            int k = u / CPR, c = u % CPR;
            *reinterpret_cast<u32x4*>(S + mn_chunk(k, c, R) * 8) = v[i];
        }
    }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA fragment of lane `lane`: operand row r0 + (lane & 31), k = kk*16 + 8h .. +7.
template <int R, bool KC>
__device__ __forceinline__ bf16x8 frag(const bf16* S, int r0, int kk, int lane) {
    const int h = lane >> 5;
    if constexpr (KC) {
        const int row = r0 + (lane & 31);
        return *reinterpret_cast<const bf16x8*>(S + lds_chunk(row, kk * 2 + h) * 8);
    } else {
        // ds_read_b64_tr_b16: lane i of a 16-lane group receives element e of the
        // 4-value row addressed by lane 4e + i/4, at position i % 4
        const int sl = lane & 15;
        const int r = r0 + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
        const int c = r >> 3, o = r & 7;
        const int k = kk * 16 + 8 * h + (sl >> 2);
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + mn_chunk(k, c, R) * 8 + o));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + mn_chunk(k + 4, c, R) * 8 + o));
        s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
}

template <int R, bool KC, int NT = 256> struct Stage;
template <int R, int NT> struct Stage<R, true, NT> : StageK<R, NT> {};
template <int R, int NT> struct Stage<R, false, NT> : StageMN<R, NT> {};

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int BM, int BN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(256, 1)
gemm_bf16_mfma(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
               int k_split, int group_m, E epi)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int TA = BM * 64, TB = BN * 64;
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    bf16* base = reinterpret_cast<bf16*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 64;

    Stage<BM, AK> sa;
    Stage<BN, BK> sb;
    auto gload = [&](int k0) {
        sa.load(A, lda, m0, M, k0, tid);
        sb.load(B, ldb, n0, N, k0, tid);
    };
    auto lstore = [&](int st) {
        sa.store(base + st * (TA + TB), tid);
        sb.store(base + st * (TA + TB) + TA, tid);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(kbeg);
        lstore(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kbeg + (kt + 1) * 64);
        const bf16* sA = base + cur * (TA + TB);
        const bf16* sB = sA + TA;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = frag<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[j] = frag<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // lane holds C[m0 + wm*WM + 32i + l32][n0 + wn*WN + 32j + 8g + 4h + (0..3)] = acc[i][j][4g + (0..3)]
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + 32 * i + l32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + 32 * j + 8 * g + 4 * h;
                if (n < N) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    epi(m, n, split, v);
                }
            }
    }
}

// ------------------------------------------------------------------ bf16 MFMA kernel, software-pipelined
// Same tiling as above, with the LDS fragment reads of k-step kk+1 issued
// while the MFMAs of k-step kk run (two fragment register sets), one
// branch-free basic block per 64-deep stage (the prefetch of the stage after
// the last one is clamped to a valid address and never stored), and
// scheduling-group hints that interleave MFMAs with LDS reads and global loads.
template <int BM, int BN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(256, 1)
gemm_bf16_mfma_pipe(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                    int k_split, int group_m, E epi)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int TA = BM * 64, TB = BN * 64;
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    bf16* base = reinterpret_cast<bf16*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 64;

    Stage<BM, AK> sa;
    Stage<BN, BK> sb;
    auto gload = [&](int k0) {
        sa.load(A, lda, m0, M, k0, tid);
        sb.load(B, ldb, n0, N, k0, tid);
    };
    auto lstore = [&](int st) {
        sa.store(base + st * (TA + TB), tid);
        sb.store(base + st * (TA + TB) + TA, tid);
    };
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, int st, int kk) {
        const bf16* sA = base + st * (TA + TB);
        const bf16* sB = sA + TA;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(kbeg);
        lstore(0);
    }
    __syncthreads();
    if (nk > 0) lfrag(0, 0, 0);
    const int klast = kbeg + (nk - 1) * 64;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        gload(min(kbeg + (kt + 1) * 64, klast));  // past the end: a harmless reload of the last stage
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int fc = kk & 1;
            if (kk < 3) lfrag(fc ^ 1, cur, kk + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fc][j], fa[fc][i], acc[i][j], 0, 0, 0);
            if (kk == 0) {
                // spread this stage's global loads over the first k-step's MFMAs
#pragma unroll
                for (int q = 0; q < FM + FN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                }
#pragma unroll
                for (int q = 0; q < FM * FN - (FM + FN); ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global load
                }
            } else if (kk < 3) {
#pragma unroll
                for (int q = 0; q < FM + FN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        }
        lstore(cur ^ 1);
        __syncthreads();
        lfrag(0, cur ^ 1, 0);
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + 32 * i + l32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + 32 * j + 8 * g + 4 * h;
                if (n < N) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    epi(m, n, split, v);
                }
            }
    }
}

// ------------------------------------------------------------------ bf16 MFMA kernel, 8 waves
// The pipelined loop above with 512 threads: 8 waves in a 2 x 4 grid, each
// owning a (BM/2) x (BN/4) sub-tile, so a wave holds half the accumulators and
// fits in 256 registers.  Two waves then share each SIMD, and one wave's LDS
// reads, barrier and memory waits overlap the other's MFMAs; the LDS read
// traffic per MFMA grows by half, which the 64-bank LDS absorbs.
template <int BM, int BN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(512, 1)
gemm_bf16_mfma_w8(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                  int k_split, int group_m, E epi)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int TA = BM * 64, TB = BN * 64;
    constexpr int WM = BM / 2, WN = BN / 4, FM = WM / 32, FN = WN / 32;
    bf16* base = reinterpret_cast<bf16*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 64;

    Stage<BM, AK, 512> sa;
    Stage<BN, BK, 512> sb;
    auto gload = [&](int k0) {
        sa.load(A, lda, m0, M, k0, tid);
        sb.load(B, ldb, n0, N, k0, tid);
    };
    auto lstore = [&](int st) {
        sa.store(base + st * (TA + TB), tid);
        sb.store(base + st * (TA + TB) + TA, tid);
    };
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, int st, int kk) {
        const bf16* sA = base + st * (TA + TB);
        const bf16* sB = sA + TA;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(kbeg);
        lstore(0);
    }
    __syncthreads();
    if (nk > 0) lfrag(0, 0, 0);
    const int klast = kbeg + (nk - 1) * 64;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        gload(min(kbeg + (kt + 1) * 64, klast));  // past the end: a harmless reload of the last stage
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int fc = kk & 1;
            if (kk < 3) lfrag(fc ^ 1, cur, kk + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fc][j], fa[fc][i], acc[i][j], 0, 0, 0);
        }
        lstore(cur ^ 1);
        __syncthreads();
        lfrag(0, cur ^ 1, 0);
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + 32 * i + l32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + 32 * j + 8 * g + 4 * h;
                if (n < N) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    epi(m, n, split, v);
                }
            }
    }
}

// ------------------------------------------------------------------ bf16 MFMA kernel, direct-to-LDS loads
// Tiles travel from memory straight into LDS (buffer_load_dwordx4 ... lds):
// no registers stage them and no LDS store instructions are issued.  One
// wave-instruction fills 1 KB of consecutive LDS chunk slots; each lane
// fetches the global 16-byte chunk whose swizzled slot it fills, so the LDS
// layouts are exactly those of the register-staged kernels.  A lane's byte
// offset differs between its instructions only by a wave-uniform stride,
// which goes into the scalar offset, and the buffer base moves with k, so a
// lane keeps one offset register per operand.  Rows past the matrix end lie
// past the buffer's record count and read as zeros; columns past a ragged
// edge read neighbouring elements of the same matrix and only reach outputs
// that are never stored.  The loads of stage k+1 run under the MFMAs of stage
// k; each wave waits for its own loads and a barrier publishes the stage.
// The two stages are distinct LDS arrays, which lets the compiler see that
// fragment reads of one never wait for the loads into the other.
typedef __attribute__((address_space(3))) void lds_void;

template <int R, bool KC, int NW>
struct DmaTile {
    static constexpr int NI = R / (8 * NW);              // wave-instructions per wave and stage
    static constexpr int CPR = R / 8;                    // 16-byte chunks per k-row (MN layout)
    static_assert(NI >= 1 && (64 * NW / CPR) % 4 == 0, "tile too small for the wave count");
    unsigned vo;                                         // lane's byte offset in its first instruction
    int step;                                            // bytes between a lane's instructions
    int w;                                               // wave index (uniform)

    __device__ __forceinline__ void init(int ld, int tid) {
        const int lane = tid & 63;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        if constexpr (KC) {
            // chunk q = 64 (w + NW i) + lane: row q / 8 (advances 8 NW per i), slot q % 8
            const int row = 8 * w + (lane >> 3);
            const int ch = (lane & 7) ^ ((lane >> 3) ^ (w & 1));
            vo = (unsigned)(row * ld * 2 + ch * 16);
            step = 8 * NW * ld * 2;
        } else {
            // chunk q: k-row q / CPR (advances 64 NW / CPR per i), slot q % CPR
            const int k = (64 * w + lane) / CPR;
            const int c = (lane % CPR) ^ ((k & 3) << 2);
            vo = (unsigned)(k * ld * 2 + c * 16);
            step = (64 * NW / CPR) * ld * 2;
        }
    }
    // one 64-deep stage starting at k0 into S
    __device__ __forceinline__ void load(const bf16* __restrict__ P, int ld, int r0, int rmax, int k0, bool valid,
                                         bf16* S) const {
        const bf16* base;
        unsigned bytes;
        if constexpr (KC) {
            base = P + (size_t)r0 * ld + k0;
            bytes = (unsigned)(((min(rmax - r0, R) - 1) * ld + 64) * 2);
        } else {
            base = P + (size_t)k0 * ld + r0;
            bytes = (unsigned)((63 * ld + min(rmax - r0, R)) * 2);
        }
        if (!valid) bytes = 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(S + 64 * (w + NW * i) * 8), 16, vo, i * step, 0,
                                                     0);
    }
};

// WGM x WGN waves (4 or 8); with 8, two waves share each SIMD and one wave's
// memory-instruction stalls are covered by the other's MFMAs.
template <int BM, int BN, int WGM, int WGN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
gemm_bf16_mfma_dma(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                   int k_split, int group_m, E epi)
{
    __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * 64];
    __shared__ __attribute__((aligned(1024))) bf16 sB0[BN * 64];
    __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * 64];
    __shared__ __attribute__((aligned(1024))) bf16 sB1[BN * 64];
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    constexpr int NL = DmaTile<BM, AK, NW>::NI + DmaTile<BN, BK, NW>::NI;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WGN, wn = w % WGN, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 64;

    DmaTile<BM, AK, NW> da;
    DmaTile<BN, BK, NW> db;
    da.init(lda, tid);
    db.init(ldb, tid);
    auto dma = [&](int kt, bf16* sA, bf16* sB) {
        da.load(A, lda, m0, M, kbeg + kt * 64, kt < nk, sA);
        db.load(B, ldb, n0, N, kbeg + kt * 64, kt < nk, sB);
    };
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, const bf16* sA, const bf16* sB, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // the MFMAs of one stage (its first fragments already in registers), with the
    // next stage's loads spread over the first k-step
    auto compute = [&](const bf16* sA, const bf16* sB) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int fc = kk & 1;
            if (kk < 3) lfrag(fc ^ 1, sA, sB, kk + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fc][j], fa[fc][i], acc[i][j], 0, 0, 0);
            if (kk < 3) {
#pragma unroll
                for (int q = 0; q < FM + FN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                }
            }
            if (kk == 0) {
#pragma unroll
                for (int q = 0; q < NL && q < FM * FN - (FM + FN); ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 memory load
                }
            }
        }
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // two stages per iteration; a stage past the end reads as zeros (its buffer
    // holds no records), so an odd count costs one idle stage and no branch
    dma(0, sA0, sB0);
    publish();
    lfrag(0, sA0, sB0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
        dma(kt + 1, sA1, sB1);
        compute(sA0, sB0);
        publish();
        lfrag(0, sA1, sB1, 0);
        dma(kt + 2, sA0, sB0);
        compute(sA1, sB1);
        publish();
        lfrag(0, sA0, sB0, 0);
    }

    store_tile<FM, FN>(acc, m0 + wm * WM, n0 + wn * WN, split, M, N, lane, epi);
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
        return frag<R, false>(S, r0, kk, lane);
    }
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
gemm_bf16_mfma_ring(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                    int k_split, int group_m, E epi)
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
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
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
    // own loads of the next stage done (the two later stages may still fly), own LDS reads done, then the barrier
    auto sync_next = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // one stage: its loads three stages ahead, k-step 0, publish the next stage, k-step 1
    auto stage = [&](int kt, const bf16* cA, const bf16* cB, const bf16* nA, const bf16* nB, bf16* xA, bf16* xB) {
        dma(kt + 3, xA, xB);
        lfrag(1, cA, cB, 1);
        mma(0);
        interleave(std::true_type{});
        sync_next();
        lfrag(0, nA, nB, 0);
        mma(1);
        interleave(std::false_type{});
    };

    dma(0, sA0, sB0);
    dma(1, sA1, sB1);
    dma(2, sA2, sB2);
    sync_next();
    lfrag(0, sA0, sB0, 0);
    for (int kt = 0; kt < nk; kt += 4) {
        stage(kt, sA0, sB0, sA1, sB1, sA3, sB3);
        stage(kt + 1, sA1, sB1, sA2, sB2, sA0, sB0);
        stage(kt + 2, sA2, sB2, sA3, sB3, sA1, sB1);
        stage(kt + 3, sA3, sB3, sA0, sB0, sA2, sB2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the loads past the end before the stores

    store_tile<FM, FN>(acc, m0 + wm * WM, n0 + wn * WN, split, M, N, lane, epi);
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
template <int BM, int BN, int WGM, int WGN, bool AK, bool BK, class E>
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
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
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
        store_tile<FM, FN>(acc, cur.m0 + wm * WM, cur.n0 + wn * WN, cur.split, M, N, lane, epi);
        cur = nxt;
        nxt = item(r + 2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ bf16 MFMA kernel, two register stages
// The global loads of stage k+2 are issued while stage k is computed and
// written to LDS only at the end of stage k+1, so every load has two stages of
// MFMA work (~4k cycles) to arrive: the single-stage prefetch above leaves the
// one wave per SIMD waiting on memory.  Two register sets alternate, so the
// stage loop is unrolled by two.
template <int BM, int BN, bool AK, bool BK, class E>
__global__ void __launch_bounds__(256, 1)
gemm_bf16_mfma_db(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K, int lda, int ldb,
                  int k_split, int group_m, E epi)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int TA = BM * 64, TB = BN * 64;
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
    bf16* base = reinterpret_cast<bf16*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1, h = lane >> 5, l32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = blockIdx.y;
    const int kbeg = split * k_split;
    const int nk = min(k_split, K - kbeg) / 64;
    const int klast = kbeg + (nk - 1) * 64;

    Stage<BM, AK> sa0, sa1;
    Stage<BN, BK> sb0, sb1;
    bf16x8 fa[2][FM], fb[2][FN];
    auto lfrag = [&](int buf, int st, int kk) {
        const bf16* sA = base + st * (TA + TB);
        const bf16* sB = sA + TA;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = frag<BM, AK>(sA, wm * WM + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = frag<BN, BK>(sB, wn * WN + 32 * j, kk, lane);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // one 64-deep stage out of LDS buffer st, with the fragment reads of the
    // next k-step overlapping the MFMAs of the current one
    auto compute = [&](int st) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int fc = kk & 1;
            if (kk < 3) lfrag(fc ^ 1, st, kk + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fc][j], fa[fc][i], acc[i][j], 0, 0, 0);
            if (kk < 3) {
#pragma unroll
                for (int q = 0; q < FM + FN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                }
            }
        }
    };

    if (nk > 0) {
        sa0.load(A, lda, m0, M, kbeg, tid);
        sb0.load(B, ldb, n0, N, kbeg, tid);
        sa0.store(base, tid);
        sb0.store(base + TA, tid);
        sa1.load(A, lda, m0, M, min(kbeg + 64, klast), tid);
        sb1.load(B, ldb, n0, N, min(kbeg + 64, klast), tid);
    }
    __syncthreads();
    if (nk > 0) lfrag(0, 0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
        // even stage: buffer 0; prefetch stage kt+2 into set 0; publish stage kt+1 (set 1) to buffer 1
        {
            const int kn = min(kbeg + (kt + 2) * 64, klast);
            sa0.load(A, lda, m0, M, kn, tid);
            sb0.load(B, ldb, n0, N, kn, tid);
            compute(0);
            sa1.store(base + (TA + TB), tid);
            sb1.store(base + (TA + TB) + TA, tid);
            __syncthreads();
            lfrag(0, 1, 0);
        }
        if (kt + 1 < nk) {
            const int kn = min(kbeg + (kt + 3) * 64, klast);
            sa1.load(A, lda, m0, M, kn, tid);
            sb1.load(B, ldb, n0, N, kn, tid);
            compute(1);
            sa0.store(base, tid);
            sb0.store(base + TA, tid);
            __syncthreads();
            lfrag(0, 0, 0);
        }
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + 32 * i + l32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + 32 * j + 8 * g + 4 * h;
                if (n < N) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    epi(m, n, split, v);
                }
            }
    }
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
static int g_variant = 9;
void gemm_set_variant(int v) { g_variant = v; }

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

template <int BM, int BN, bool AK, bool BK, class E>
static hipError_t run_mfma(const GemmDesc& d, E e, hipStream_t s) {
    constexpr size_t lds = 2 * (size_t)(BM + BN) * 64 * sizeof(bf16);
    const int v = d.variant >= 0 && d.variant <= 9 ? d.variant : g_variant;
    if (v >= 8) {
        auto pk = v == 9 ? gemm_bf16_mfma_pring<BM, BN, 2, 4, AK, BK, E> : gemm_bf16_mfma_pring<BM, BN, 2, 2, AK, BK, E>;
        const int nt = v == 9 ? 512 : 256;
        static int resident[2] = {0, 0};  // workgroups per CU, from the occupancy query
        int& occ = resident[v - 8];
        if (occ == 0) {
            hipError_t st = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(pk), nt, 0);
            if (st != hipSuccess) return st;
            if (occ < 1) occ = 1;
        }
        const int splits = (d.K + d.k_split - 1) / d.k_split;
        const int items = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN) * splits;
        const int grid = std::min(items, occ * num_cus());
        hipLaunchKernelGGL(pk, dim3(grid), dim3(nt), 0, s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, d.K, d.lda,
                           d.ldb, d.k_split, splits, d.group_m, e);
        return hipGetLastError();
    }
    auto kern = v == 7   ? gemm_bf16_mfma_ring<BM, BN, 2, 4, AK, BK, E>
                : v == 6 ? gemm_bf16_mfma_ring<BM, BN, 2, 2, AK, BK, E>
                : v == 5 ? gemm_bf16_mfma_dma<BM, BN, 2, 4, AK, BK, E>
                : v == 4 ? gemm_bf16_mfma_dma<BM, BN, 2, 2, AK, BK, E>
                : v == 3 ? gemm_bf16_mfma_w8<BM, BN, AK, BK, E>
                : v == 2 ? gemm_bf16_mfma_db<BM, BN, AK, BK, E>
                : v == 1 ? gemm_bf16_mfma_pipe<BM, BN, AK, BK, E>
                         : gemm_bf16_mfma<BM, BN, AK, BK, E>;
    const int nthreads = v == 3 || v == 5 || v == 7 ? 512 : 256;
    const size_t dyn = v >= 4 ? 0 : lds;  // the direct-to-LDS kernels use static LDS
    static bool attr_done[4] = {false, false, false, false};
    if (v < 4 && !attr_done[v]) {
        hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (st != hipSuccess) return st;
        attr_done[v] = true;
    }
    int tiles = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
    dim3 grid(tiles, (d.K + d.k_split - 1) / d.k_split);
    hipLaunchKernelGGL(kern, grid, dim3(nthreads), dyn, s, (const bf16*)d.A, (const bf16*)d.B, d.M, d.N, d.K, d.lda,
                       d.ldb, d.k_split, d.group_m, e);
    return hipGetLastError();
}

template <bool AK, bool BK, class E>
static hipError_t run_bf16(const GemmDesc& d, E e, hipStream_t s) {
    switch (d.tile) {
    case 0: return run_mfma<256, 256, AK, BK>(d, e, s);
    case 1: return run_mfma<256, 128, AK, BK>(d, e, s);
    default: return run_mfma<128, 128, AK, BK>(d, e, s);
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

template <typename T, bool AK, bool BK>
static hipError_t dispatch_epi(const GemmDesc& d, hipStream_t s) {
    auto run = [&](auto e) -> hipError_t {
        if constexpr (sizeof(T) == 2) return run_bf16<AK, BK>(d, e, s);
        else return run_f32<AK, BK>(d, e, s);
    };
    switch (d.epi) {
    case Epi::StoreCd: return run(EStoreCd<T>{(T*)d.out, d.ldo});
    case Epi::StoreF32: return run(EStoreF32{(float*)d.out, d.ldo});
    case Epi::ResidualCd: return run(EResidual<T>{(T*)d.out, (const T*)d.in, d.ldo});
    case Epi::ReluSq: return run(EReluSq<T>{(T*)d.out, d.ldo});
    case Epi::ReluSqBwd: return run(EReluSqBwd<T>{(T*)d.out, (const T*)d.in, d.ldo});
    case Epi::Grad: return run(EGrad{(float*)d.out, d.ldo, d.accumulate});
    case Epi::SplitK: return run(ESplitK{(float*)d.out, d.ldo, d.split_stride});
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_layout(const GemmDesc& d, hipStream_t s) {
    if (d.a_kcontig && d.b_kcontig) return dispatch_epi<T, true, true>(d, s);
    if (d.a_kcontig && !d.b_kcontig) return dispatch_epi<T, true, false>(d, s);
    if (!d.a_kcontig && !d.b_kcontig) return dispatch_epi<T, false, false>(d, s);
    return dispatch_epi<T, false, true>(d, s);
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
    return dispatch_layout<float>(d, s);
}

const char* gemm_kernel_name(const GemmDesc& d) {
    static const char* lay[4] = {"tn", "tk", "nt_mn", "nt"};
    int li = (d.a_kcontig ? 2 : 0) + (d.b_kcontig ? 1 : 0);
    (void)lay;
    if (d.dt == Dt::F32) return li == 3 ? "gemm_f32_nt" : (li == 2 ? "gemm_f32_nn" : "gemm_f32_tn");
    static const char* names[3][3] = {
        {"gemm_bf16_nt_256x256", "gemm_bf16_nt_256x128", "gemm_bf16_nt_128x128"},
        {"gemm_bf16_nn_256x256", "gemm_bf16_nn_256x128", "gemm_bf16_nn_128x128"},
        {"gemm_bf16_tn_256x256", "gemm_bf16_tn_256x128", "gemm_bf16_tn_128x128"}};
    int r = li == 3 ? 0 : (li == 2 ? 1 : 2);
    int t = d.tile < 0 ? 0 : (d.tile > 2 ? 2 : d.tile);
    (void)lay;
    return names[r][t];
}

hipError_t gemm_init_attributes() { return hipSuccess; }

// ------------------------------------------------------------------ split-K reduction
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, size_t stride, float* __restrict__ g, size_t n4,
                     int accumulate)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 acc = accumulate ? reinterpret_cast<const float4*>(g)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sidx = 0; sidx < splits; ++sidx) {
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
