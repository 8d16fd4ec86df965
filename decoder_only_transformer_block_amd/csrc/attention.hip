// Causal self-attention with grouped-query heads (query head h reads kv head
// h / (H/Hkv)), forward and backward, on the packed qkv activation.
//
// q and k arrive RoPE-rotated and RMS-normalised over the head dim (QK-norm,
// "nanochat 项目深度分析" §2.1 items 1-2), so |q.k| <= |q||k| <= D and every
// scaled score s/sqrt(D) lies in [-sqrt(D), sqrt(D)].  The softmax therefore
// uses the static shift sqrt(D) instead of a running row max: exp(s/sqrt(D) -
// sqrt(D)) is in [e^-2sqrt(D), ~1] (>= 1.5e-10 for D = 128), so no rescaling of the
// partial output is ever needed and the row sum cannot underflow.
//
// bf16 path (D = 128): MFMA flash kernels.  Each lane of a wave owns one query
// row (operand-swapped v_mfma_f32_32x32x16_bf16, as in the GEMMs), so the
// row-wise softmax work stays in registers; the probabilities are fed back to
// the next MFMA straight from the accumulator registers by contracting over
// keys in the order the accumulator holds them.  Tiles travel from memory
// straight into LDS, double-buffered, and are stored once in their natural
// layout; products contracting over a tile's rows read it with the gfx950
// transposing LDS read.  The backward is two kernels: dQ with the query block
// outer (it also forms delta), then dK/dV with the key block outer (sums over
// the r query heads of a kv group in a fixed order), so no floating-point
// atomics are used and results are bitwise reproducible.
//
// fp32 path: plain SIMT kernels, one wave per row, for the fp32 compute mode.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ncgpt {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- workgroup order
// Forward: a stream is the set of workgroups that read the same K / V rows, one (sequence, kv head) with its
// r query heads; a stream has npos workgroups, position 0 the heaviest.  Each XCD runs a contiguous range of
// the order below (xcd_remap), which walks groups of G streams -- G chosen so one group fills the XCD's
// resident slots -- and inside a group takes the positions heaviest first, streams fastest.  The group's
// workgroups start together and stream the same rows at about the same time, so those rows come from the
// XCD's L2 rather than from HBM, while the heaviest-first order inside each group keeps the tail short.
__device__ __forceinline__ void attn_order(int bid, int nwg, int npos, int nstream, int G, int& stream, int& pos) {
    const int L = xcd_remap(bid, nwg);
    const int grp = L / (G * npos), in = L % (G * npos);
    const int g0 = grp * G, gn = min(G, nstream - g0);
    pos = in / gn;
    stream = g0 + in % gn;
}
// G for kernels with per_cu resident workgroups per CU (32 CUs per XCD)
inline int attn_group(int npos, int per_cu) { return std::max(1, 32 * per_cu / npos); }

// ---------------------------------------------------------------- LDS tiles
// Every tile is [64 rows][128] bf16 in its natural memory layout (256-byte
// rows of 16 chunks of 16 bytes).  Two kinds of reads hit it:
//  - row fragments: 16 consecutive rows at one chunk per 16-lane group
//    (ds_read_b128), the MFMA operand whose K index runs along the row;
//  - transposed fragments: ds_read_b64_tr_b16, 4 consecutive rows x 4
//    consecutive chunks per 32 lanes, the operand whose K index runs down
//    the rows (V for P.V, dO and Q for dV and dK, K for dQ).
// The chunk index is XOR-ed with swz(row) = ((row & 3) << 2) | ((row >> 2) & 3):
// a bijection over 16 consecutive rows (row reads hit 16 distinct chunks) whose
// high bits differ across 4 consecutive rows (transposed reads hit 4 distinct
// 64-byte bank groups), so neither read conflicts on the 64-bank LDS.
// rfrag / trfrag below are the definitional forms; the kernels read through the
// closed-form offsets further down (rz, tz, frag_at, trfrag_at; frag_in, trfrag_in).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int toff(int r, int c) { return r * 128 + ((c ^ swz(r)) << 3); }

__device__ __forceinline__ bf16x8 rfrag(const bf16* S, int r, int c) {
    return *reinterpret_cast<const bf16x8*>(S + toff(r, c));
}

// Transposed fragment for MFMA lane l: X[row = d0 + (l & 31)][k] with the 8 k
// slots of lane half hh = l >> 5 being tile rows kbase + 4hh + (0..3) and
// kbase + 8 + 4hh + (0..3) -- the order in which an operand-swapped MFMA
// accumulator holds its 32 columns, so P and dS feed back from registers.
// ds_read_b64_tr_b16 gives lane i of a 16-lane group element e of the 4-value
// row addressed by lane 4e + i/4, at position i % 4.
__device__ __forceinline__ bf16x8 trfrag(const bf16* S, int d0, int kbase, int lane) {
    const int s = lane & 15, hh = lane >> 5;
    const int d = d0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const int c = d >> 3, o = d & 7;
    const int r = kbase + 4 * hh + (s >> 2);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + toff(r, c) + o));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(S + toff(r + 8, c) + o));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// The same fragments with their byte offsets in closed form.  Rows 16 apart share
// swz, and the chunk bits (4..7 of the byte offset) sit apart from the row bits, so
//   rfrag(S, r, 2 kk + hv) lies at rz(r, hv) ^ (kk << 5), and
//   trfrag(S, 32 db, kbase, lane), kbase a multiple of 16, reads its low rows at
//   256 kbase + (tz(lane) ^ (db << 6)) and its high rows (8 further) at
//   256 kbase + 2048 + (tz(lane) ^ (db << 6) ^ 32).
// A lane forms rz / tz once; a fragment then costs at most one XOR, and the row
// block and the LDS array fold into the instruction's offset field.
__device__ __forceinline__ int rz(int r, int hv) { return r * 256 | (((hv ^ swz(r)) & 15) << 4); }
__device__ __forceinline__ int tz(int lane) {
    const int s = lane & 15, rl = 4 * (lane >> 5) + (s >> 2), cl = 2 * ((lane >> 4) & 1) + ((s & 3) >> 1);
    return rl * 256 + (((cl ^ swz(rl)) & 15) << 4) + 8 * (s & 1);
}
__device__ __forceinline__ bf16x8 frag_at(const bf16* S, int off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(S) + off);
}
// trfrag(S, 32 db, 0, lane) from t = tz(lane) (pass S + 128 kbase for a later row block)
__device__ __forceinline__ bf16x8 trfrag_at(const bf16* S, int t, int db) {
    const char* p = reinterpret_cast<const char*>(S);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (t ^ (db << 6))));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2048 + (t ^ (db << 6) ^ 32)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Row and transposed fragments from byte offsets into tile S (tiles are 16 KB-aligned, so an offset XOR-ed
// with a fragment's chunk bits stays inside the tile).  The reads keep S as their object, so where S is an LDS
// array of its own the compiler knows they do not touch direct-to-LDS loads in flight into other arrays, and
// issues them without waiting for those loads (a read it cannot place is made to wait for all).
__device__ __forceinline__ bf16x8 frag_in(const bf16* S, uint32_t off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(S) + off);
}
__device__ __forceinline__ bf16x8 trfrag_in(const bf16* S, uint32_t lo, uint32_t hi) {
    const char* p = reinterpret_cast<const char*>(S);
    s16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + lo));
    s16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 8 accumulator values rounded to the 16-bit operand type H, as an MFMA fragment (bit pattern)
template <typename HT>
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
    typename V8<HT>::type r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (HT)s[base + e];
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ void zero16(f32x16& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}


// ======================================================================== delta = rowsum(dO * O) (fp32 path)
template <typename T>
__global__ void __launch_bounds__(256)
attn_delta(const T* __restrict__ dy, const T* __restrict__ y, float* __restrict__ delta, int N, int T_, int H, int D)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;  // (n, h)
    if (gid >= N * H) return;
    const int n = gid / H, h = gid % H;
    const T* a = dy + (size_t)n * H * D + h * D;
    const T* c = y + (size_t)n * H * D + h * D;
    float acc = 0.0f;
    for (int d = 0; d < D; d += 4) {
        float u[4], v[4];
        Vec4<T>::load(a + d, u);
        Vec4<T>::load(c + d, v);
        acc += u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
    }
    const int b = n / T_, t = n % T_;
    delta[((size_t)b * H + h) * T_ + t] = acc;
}

// ======================================================================== LDS-direct tile loads
// LDS-direct loads: one wave-instruction fills 1 KB (64 consecutive 16-byte
// chunk slots) of a [rows][128] tile; each lane fetches the global chunk whose
// swizzled slot it fills.  With NW waves, slot q = 64 (w + NW i) + lane lies in
// row 4 w + 4 NW i + lane / 16 at physical chunk lane % 16; that row's swizzle
// is ((lane / 16) << 2) | (w & 3) for every i (NW is a multiple of 4), so a lane
// keeps one byte offset per tensor and instruction i adds 4 NW rows x i.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// lane's byte offset of its chunk in a wave's first instruction (row stride ld elements)
__device__ __forceinline__ unsigned dma_voff(int ld, int lane, int w) {
    const int c = (lane & 15) ^ (((lane >> 4) << 2) | (w & 3));
    return (unsigned)(((4 * w + (lane >> 4)) * ld + c * 8) * 2);
}
// wave w's share of a [ROWS][128] tile among NW waves: ROWS / (4 NW) instructions of 4 rows each
template <int ROWS, int NW = 4>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, unsigned vo, int ld, bf16* S, int w) {
    static_assert(NW % 4 == 0 && ROWS % (4 * NW) == 0, "row count must split evenly over the waves");
#pragma unroll
    for (int i = 0; i < ROWS / (4 * NW); ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(S + 64 * (w + NW * i) * 8), 16, vo,
                                                 i * 4 * NW * ld * 2, 0, 0);
}

// ======================================================================== fused RoPE + QK-norm backward
// A head row's gradient g (w.r.t. the normalised, rotated q or k) held by a lane
// pair in the MFMA accumulator layout: lane half hh holds dims
// d = 32 db + 8 gg + 4 hh + e in v[db][4 gg + e].  The QK-norm derivative needs
// the saved normalised row y and 1/rms rs: r = rs (g - y mean(g y)); the
// rotation's transpose then maps the pair (i, i + D/2):
// out_i = r_i cos - r_{i+D/2} sin, out_{i+D/2} = r_i sin + r_{i+D/2} cos.
// Dims d and d + 64 sit in the same lane (db and db + 2).
template <typename HT>
__device__ __forceinline__ void rope_qknorm_bwd_row(float (&v)[4][16], const bf16* __restrict__ yrow, float rs,
                                                    const float* __restrict__ cs, const float* __restrict__ sn,
                                                    int hh) {
    float yv[4][16];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            float t[4];
            Vec4<HT>::load(reinterpret_cast<const HT*>(yrow + 32 * db + 8 * gg + 4 * hh), t);
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[db][4 * gg + e] = t[e];
        }
    float dot = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dot += v[db][i] * yv[db][i];
    dot = (dot + __shfl_xor(dot, 32, kWave)) * (1.0f / 128.0f);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            float c[4], s[4];
            const int i0 = 32 * db + 8 * gg + 4 * hh;
            Vec4<float>::load(cs + i0, c);
            Vec4<float>::load(sn + i0, s);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 4 * gg + e;
                const float r1 = rs * (v[db][k] - yv[db][k] * dot), r2 = rs * (v[db + 2][k] - yv[db + 2][k] * dot);
                v[db][k] = r1 * c[e] - r2 * s[e];
                v[db + 2][k] = r1 * s[e] + r2 * c[e];
            }
        }
}

// ======================================================================== bf16 forward
// Workgroup: 4 waves x 32 QB queries of one head; K/V tiles travel
// straight from memory into LDS, double-buffered, KT keys per tile.  QB = 2
// reuses every K and V fragment read from LDS for two 32-query blocks at one
// wave per SIMD; QB = 1 runs several workgroups per CU, so one wave's softmax
// runs under the others' MFMAs: two with 64-key tiles (64 KB of LDS each),
// three with 32-key tiles (32 KB each; 158 VGPRs fit three waves per SIMD).
template <int QB, typename HT, int KT = 64>
__global__ void __launch_bounds__(256, QB == 1 ? (KT == 32 ? 3 : 2) : 1)
attn_fwd_bf16(const bf16* __restrict__ qkv, bf16* __restrict__ y, float* __restrict__ lse, int T, int H, int Hkv,
              int B, int G)
{
    constexpr int D = 128, QW = 32 * QB, QBLK = 4 * QW;
    __shared__ __attribute__((aligned(1024))) bf16 sK0[KT * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sV0[KT * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sK1[KT * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sV1[KT * 128];
    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // stream (sequence, kv head); positions: late (heavy) query blocks first, the group's query heads fastest
    const int nqb = (T + QBLK - 1) / QBLK, r = H / Hkv;
    int st, pos;
    attn_order(blockIdx.x, gridDim.x, nqb * r, B * Hkv, G, st, pos);
    const int b = st / Hkv, g = st % Hkv;
    const int hq = g * r + pos % r, qblk = nqb - 1 - pos / r;
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const int q0 = qblk * QBLK;
    const int qw = q0 + QW * w;                 // first query of this wave
    const bool active = qw < T;                 // T is a multiple of 64
    const size_t rowbase = (size_t)b * T;

    bf16x8 qf[QB][8];
    if (active) {
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
            const int q = min(qw + 32 * qq + l32, T - 1);
            const bf16* qp = qkv + (rowbase + q) * QKV + hq * D + 8 * hh;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) qf[qq][kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
        }
    }
    f32x16 o[QB][4];
    float lsum[QB];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
        lsum[qq] = 0.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db) zero16(o[qq][db]);
    }
    // fp16 keeps P = exp(s - sqrt(D)) away from its subnormals by carrying it as 2^15 P (the row sum and the
    // LSE take the factor out again); the largest value, 2^15, stays inside fp16's range
    constexpr float kPow = std::is_same<HT, f16>::value ? 15.0f : 0.0f;
    const float c1 = kLog2e * rsqrtf((float)D), c2 = sqrtf((float)D) * kLog2e - kPow;

    const int nkt = min(q0 + QBLK, T) / KT;     // key tiles at or before the block's last query
    const int zk = rz(l32, hh), tl = tz(lane);  // fragment offsets (rows l32 + 32 kb share them)
    const unsigned vo = dma_voff(QKV, lane, w);
    const bf16* kbase = qkv + rowbase * QKV + HD + g * D;
    auto issue = [&](int kt, bf16* Ks, bf16* Vs) {
        const bf16* kp = kbase + (size_t)kt * KT * QKV;
        const unsigned bytes = (unsigned)(((KT - 1) * QKV + 128) * 2);
        dma_rows<KT>(buf_rsrc(kp, bytes), vo, QKV, Ks, w);
        dma_rows<KT>(buf_rsrc(kp + KD, bytes), vo, QKV, Vs, w);
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    auto compute = [&](int kt, const bf16* Ks, const bf16* Vs) {
        const int kv0 = kt * KT;
        if (!active || kv0 > qw + QW - 1) return;  // wave-uniform: the whole tile lies after the wave's queries
        const bool diag = kv0 + KT - 1 > qw;
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb) {
            f32x16 sc[QB];
#pragma unroll
            for (int qq = 0; qq < QB; ++qq) zero16(sc[qq]);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 kf = frag_at(Ks + 32 * 128 * kb, zk ^ (kk << 5));
#pragma unroll
                for (int qq = 0; qq < QB; ++qq)
                    sc[qq] = mfma16<HT>(kf, qf[qq][kk], sc[qq]);
            }
            // lane holds S[q = qw + 32qq + l32][key = kv0 + 32kb + 8(e>>2) + 4hh + (e&3)] in sc[qq][e]
            auto softmax = [&](auto masked) {
#pragma unroll
                for (int qq = 0; qq < QB; ++qq)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float p = __builtin_amdgcn_exp2f(sc[qq][e] * c1 - c2);
                        if constexpr (decltype(masked)::value)
                            p = kv0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3) > qw + 32 * qq + l32 ? 0.0f : p;
                        sc[qq][e] = p;
                        lsum[qq] += p;
                    }
            };
            if (diag)
                softmax(std::true_type{});
            else
                softmax(std::false_type{});
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bf16x8 pf[QB];
#pragma unroll
                for (int qq = 0; qq < QB; ++qq) pf[qq] = pack8<HT>(sc[qq], 8 * j);
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const bf16x8 vf = trfrag_at(Vs + 128 * (32 * kb + 16 * j), tl, db);
#pragma unroll
                    for (int qq = 0; qq < QB; ++qq)
                        o[qq][db] = mfma16<HT>(vf, pf[qq], o[qq][db]);
                }
            }
        }
    };

    issue(0, sK0, sV0);
    publish();
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) issue(kt + 1, sK1, sV1);
        compute(kt, sK0, sV0);
        publish();
        if (kt + 2 < nkt) issue(kt + 2, sK0, sV0);
        if (kt + 1 < nkt) compute(kt + 1, sK1, sV1);
        publish();
    }
    if (!active) return;
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
        const int q = qw + 32 * qq + l32;
        const float ltot = lsum[qq] + __shfl_xor(lsum[qq], 32, kWave);
        const float inv = 1.0f / ltot;
        if (q >= T) continue;
        bf16* yp = y + (rowbase + q) * HD + hq * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = o[qq][db][4 * gg + e] * inv;
                Vec4<HT>::store(reinterpret_cast<HT*>(yp + 32 * db + 8 * gg + 4 * hh), v);
            }
        if (hh == 0) lse[((size_t)b * H + hq) * T + q] = sqrtf((float)D) + logf(ltot) - kPow * 0.6931471805599453f;
    }
}

// ======================================================================== bf16 backward: dQ (and delta)
// Workgroup: 128 queries of one head, 4 waves x 32 queries.  Each lane first
// forms delta = rowsum(dO * O) of its query row and stores it with the LSE in
// log2 units (both read by the key-outer kernel), keeps its Q and dO fragments
// in registers, then for every 64-key tile recomputes S and dP, forms dS =
// P (dP - delta) and accumulates dQ = dS K (scaled by 1/sqrt(D) at the end).
// K and V tiles travel straight from memory into LDS, double-buffered.
template <int OCC, typename HT>
__global__ void __launch_bounds__(256, OCC)
attn_bwd_dq_bf16(const bf16* __restrict__ qkv, const bf16* __restrict__ y, const bf16* __restrict__ dy,
                 const float* __restrict__ lse, float* __restrict__ delta, bf16* __restrict__ dqkv,
                 const float* __restrict__ rstdq, const float* __restrict__ cosv, const float* __restrict__ sinv,
                 int T, int H, int Hkv, int B)
{
    constexpr int D = 128, QB = 128;
    __shared__ __attribute__((aligned(1024))) bf16 sK0[64 * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sV0[64 * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sK1[64 * 128];
    __shared__ __attribute__((aligned(1024))) bf16 sV1[64 * 128];
    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // late (heavy) query blocks first; (head, sequence) varies fastest (grouping one stream's blocks on an
    // XCD, as the forward does, measured 2 % slower here)
    const int nqb = (T + QB - 1) / QB;
    const int hb = blockIdx.x % (H * B), qblk = nqb - 1 - blockIdx.x / (H * B);
    const int hq = hb / B, b = hb % B;
    const int g = hq / (H / Hkv);
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const int q0 = qblk * QB;
    const int qw = q0 + 32 * w;                 // first query of this wave
    const bool active = qw < T;                 // T is a multiple of 64
    const int q = qw + l32;
    const size_t rowbase = (size_t)b * T;
    const float scale = rsqrtf((float)D), c1 = kLog2e * scale;

    bf16x8 qf[8], dof[8];
    float l2 = 0.0f, dl = 0.0f;
    if (active) {
        const bf16* qp = qkv + (rowbase + q) * QKV + hq * D + 8 * hh;
        const bf16* gp = dy + (rowbase + q) * HD + hq * D + 8 * hh;
        const bf16* yp = y + (rowbase + q) * HD + hq * D + 8 * hh;
        float part = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
            dof[kk] = *reinterpret_cast<const bf16x8*>(gp + 16 * kk);
            const auto yv = *reinterpret_cast<const typename V8<HT>::type*>(yp + 16 * kk);
            const auto dv8 = __builtin_bit_cast(typename V8<HT>::type, dof[kk]);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += (float)dv8[e] * (float)yv[e];
        }
        dl = part + __shfl_xor(part, 32, kWave);
        const size_t li = ((size_t)b * H + hq) * T + q;
        l2 = lse[li] * kLog2e;
        if (hh == 0) {
            delta[li] = dl;
            delta[(size_t)B * H * T + li] = l2;  // the LSE in log2 units, for the key-outer kernel
        }
    }
    f32x16 dq[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) zero16(dq[db]);

    const int nkt = min(q0 + QB, T) / 64;       // key tiles at or before the block's last query
    const int zk = rz(l32, hh), tl = tz(lane);  // fragment offsets (rows l32 + 32 kb share them)
    const unsigned vo = dma_voff(QKV, lane, w);
    const bf16* kbase = qkv + rowbase * QKV + HD + g * D;
    auto issue = [&](int kt, bf16* Ks, bf16* Vs) {
        const bf16* kp = kbase + (size_t)kt * 64 * QKV;
        const unsigned bytes = (unsigned)((63 * QKV + 128) * 2);
        dma_rows<64>(buf_rsrc(kp, bytes), vo, QKV, Ks, w);
        dma_rows<64>(buf_rsrc(kp + KD, bytes), vo, QKV, Vs, w);
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    auto compute = [&](int kt, const bf16* Ks, const bf16* Vs) {
        const int kv0 = kt * 64;
        if (!active || kv0 > qw + 31) return;  // wave-uniform: the whole tile lies after the wave's queries
        const bool diag = kv0 + 63 > qw;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s, dp;
            zero16(s);
            zero16(dp);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                s = mfma16<HT>(frag_at(Ks + 32 * 128 * kb, zk ^ (kk << 5)), qf[kk], s);
                dp = mfma16<HT>(frag_at(Vs + 32 * 128 * kb, zk ^ (kk << 5)), dof[kk], dp);
            }
            // lane holds S[q][key = kv0 + 32kb + 8(e>>2) + 4hh + (e&3)] in s[e]
            auto softmax = [&](auto masked) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float p = __builtin_amdgcn_exp2f(s[e] * c1 - l2);
                    if constexpr (decltype(masked)::value)
                        p = kv0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3) > qw + l32 ? 0.0f : p;
                    dp[e] = p * (dp[e] - dl);
                }
            };
            if (diag)
                softmax(std::true_type{});
            else
                softmax(std::false_type{});
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 dsf = pack8<HT>(dp, 8 * j);
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dq[db] = mfma16<HT>(
                        trfrag_at(Ks + 128 * (32 * kb + 16 * j), tl, db), dsf, dq[db]);
            }
        }
    };

    issue(0, sK0, sV0);
    publish();
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) issue(kt + 1, sK1, sV1);
        compute(kt, sK0, sV0);
        publish();
        if (kt + 2 < nkt) issue(kt + 2, sK0, sV0);
        if (kt + 1 < nkt) compute(kt + 1, sK1, sV1);
        publish();
    }
    if (!active) return;
    float gq[4][16];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) gq[db][i] = dq[db][i] * scale;
    rope_qknorm_bwd_row<HT>(gq, qkv + (rowbase + q) * QKV + hq * D, rstdq[(rowbase + q) * H + hq], cosv + q * (D / 2),
                        sinv + q * (D / 2), hh);
    bf16* qout = dqkv + (rowbase + q) * QKV + hq * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const float a[4] = {gq[db][4 * gg], gq[db][4 * gg + 1], gq[db][4 * gg + 2], gq[db][4 * gg + 3]};
            Vec4<HT>::store(reinterpret_cast<HT*>(qout + 32 * db + 8 * gg + 4 * hh), a);
        }
}

// ======================================================================== bf16 backward: dK, dV
// Workgroup: 128 keys of one kv head and 8 waves, two per SIMD so that one
// wave's softmax runs under the other's MFMAs.  Waves w and w + 4 own the same
// 32 keys (block w % 4) and take the two 32-query halves of every 64-query
// tile; each accumulates its half's share of dK and dV (32 keys x 128 dims
// each) in registers, and the two shares are added in a fixed order at the end
// (deterministic).  V rows of the block sit in LDS, and each wave keeps its
// 32 keys' K fragments in registers; the workgroup loops over the r query heads
// of the group and over the query tiles at or after its first key.  Q, dO, lse and delta tiles travel straight from memory into LDS
// (buffer_load ... lds), double-buffered: the loads of tile i+1 run under the
// MFMAs of tile i.
template <typename HT>
__global__ void __launch_bounds__(512, 1)
attn_bwd_dkdv_bf16(const bf16* __restrict__ qkv, const bf16* __restrict__ dy, const float* __restrict__ delta,
                   bf16* __restrict__ dqkv, const float* __restrict__ rstdk, const float* __restrict__ cosv,
                   const float* __restrict__ sinv, int T, int H, int Hkv, int B)
{
    constexpr int D = 128, KB = 128, NW = 8;
    // K with V 32 KB past it; per stage Q with dO 16 KB past it, and the LSE / delta rows.  Each stage is an LDS
    // array of its own: the compiler then knows that the transposed reads of one stage do not touch the loads in
    // flight into the other, and issues them without waiting for those loads.
    __shared__ __attribute__((aligned(16384))) bf16 sKV[2 * KB * 128];
    __shared__ __attribute__((aligned(16384))) bf16 sS0[2 * 64 * 128];
    __shared__ __attribute__((aligned(16384))) bf16 sS1[2 * 64 * 128];
    __shared__ __attribute__((aligned(256))) float sLD0[128];
    __shared__ __attribute__((aligned(256))) float sLD1[128];
    bf16* const sK = sKV;
    bf16* const sV = sKV + KB * 128;
    bf16* const sQ0 = sS0;
    bf16* const sO0 = sS0 + 64 * 128;
    bf16* const sQ1 = sS1;
    bf16* const sO1 = sS1 + 64 * 128;
    float* const sL0 = sLD0;
    float* const sD0 = sLD0 + 64;
    float* const sL1 = sLD1;
    float* const sD1 = sLD1 + 64;

    const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kq = w & 3, qh = w >> 2;            // key block of the wave, query half of each tile
    // key blocks early in the sequence see the most queries: they come first, and the (head, sequence)
    // index varies fastest (grouping one stream's blocks on an XCD, as the forward does, measured 3 % slower)
    const int gb = blockIdx.x % (Hkv * B), kblk = blockIdx.x / (Hkv * B);
    const int g = gb / B, b = gb % B;
    const int r = H / Hkv;
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const int k0 = kblk * KB;
    const int kw = k0 + 32 * kq;                  // first key of this wave
    const bool active = kw < T;                   // T is a multiple of 64
    const size_t rowbase = (size_t)b * T;
    const float scale = rsqrtf((float)D), c1 = kLog2e * scale;

    // K and V rows of the block (rows past T read as zeros)
    {
        const int rows = min(KB, T - k0);
        const unsigned bytes = (unsigned)(((rows - 1) * QKV + 128) * 2);
        const bf16* kp = qkv + (rowbase + k0) * QKV + HD + g * D;
        const unsigned vo = dma_voff(QKV, lane, w);
        dma_rows<KB, NW>(buf_rsrc(kp, bytes), vo, QKV, sK, w);
        dma_rows<KB, NW>(buf_rsrc(kp + KD, bytes), vo, QKV, sV, w);
    }
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) { zero16(dk[db]); zero16(dv[db]); }

    const int qt0 = k0 / 64, nqt = T / 64 - qt0;
    // fragment offsets: the wave's query half (32 qh + l32) in the Q / dO tiles, its keys
    // (32 kq + l32) in K / V, and the transposed reads of the query half
    const int zq0 = rz(32 * qh + l32, hh), zk0 = rz(32 * kq + l32, hh), tq0 = tz(lane) + 32 * 256 * qh;
    const int total = r * nqt;
    bf16x8 kf[8];                                 // the wave's K fragments, read once (after the first publish)
    const unsigned voq = dma_voff(QKV, lane, w), vod = dma_voff(HD, lane, w);
    // loads of tile it (query head g r + it / nqt, queries from (qt0 + it % nqt) 64) into one stage
    auto issue = [&](int it, bf16* Qs, bf16* Os, float* Ls, float* Ds) {
        const int hq = g * r + it / nqt, q0 = (qt0 + it % nqt) * 64;
        dma_rows<64, NW>(buf_rsrc(qkv + (rowbase + q0) * QKV + hq * D, (unsigned)((63 * QKV + 128) * 2)), voq, QKV,
                         Qs, w);
        dma_rows<64, NW>(buf_rsrc(dy + (rowbase + q0) * HD + hq * D, (unsigned)((63 * HD + 128) * 2)), vod, HD, Os, w);
        const size_t li = ((size_t)b * H + hq) * T + q0;
        if (w == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(delta + (size_t)B * H * T + li, 256), (lds_void*)Ls, 4,
                                                     lane * 4, 0, 0, 0);
        else if (w == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(delta + li, 256), (lds_void*)Ds, 4, lane * 4, 0, 0, 0);
    };
    auto publish = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    // one tile: S and dP for the wave's 32 keys x 32 queries, then dV += P^T dO, dK += dS^T Q
    auto compute = [&](int it, const bf16* Qs, const bf16* Os, const float* Ls, const float* Ds) {
        const int q0 = (qt0 + it % nqt) * 64 + 32 * qh;  // the wave's 32 queries
        if (!active || q0 + 31 < kw) return;  // wave-uniform: every query precedes every key of the wave
        // fragment offsets re-formed per tile (one XOR per fragment) instead of held in registers
        uint32_t aq = zq0, ak = zk0, at = tq0;
        asm volatile("" : "+v"(aq), "+v"(ak), "+v"(at));   // formed per tile, not hoisted into registers
        const bool diag = q0 < kw + 31;
        f32x16 s, dp;
        zero16(s);
        zero16(dp);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint32_t xq = aq ^ (kk << 5), xk = ak ^ (kk << 5);
            s = mfma16<HT>(frag_in(Qs, xq), kf[kk], s);
            dp = mfma16<HT>(frag_in(Os, xq), frag_in(sV, xk), dp);
        }
        // issue order: the fragments of the first two k-steps, then per k-step its two MFMAs and the reads of
        // the k-step two ahead (Q, dO and V: K is in registers)
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // lane holds S[q = q0 + 8(e>>2) + 4hh + (e&3)][key = kw + l32] in s[e]; P = exp2(S c1 - lse2),
        // dS / scale = P (dP - delta) (dK is scaled at the end); the mask only on diagonal tiles
        auto softmax = [&](auto masked) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int ql = 32 * qh + 8 * gg + 4 * hh;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + ql);
                const float lv[4] = {l4[0], l4[1], l4[2], l4[3]}, dv4[4] = {d4[0], d4[1], d4[2], d4[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int idx = 4 * gg + e;
                    float p = __builtin_amdgcn_exp2f(s[idx] * c1 - lv[e]);
                    if constexpr (decltype(masked)::value) p = q0 + 8 * gg + 4 * hh + e < kw + l32 ? 0.0f : p;
                    s[idx] = p;
                    dp[idx] = p * (dp[idx] - dv4[e]);
                }
            }
        };
        if (diag)
            softmax(std::true_type{});
        else
            softmax(std::false_type{});
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
            const bf16x8 pf = pack8<HT>(s, 8 * j2), dsf = pack8<HT>(dp, 8 * j2);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint32_t lo = (at ^ (db << 6)) + 4096 * j2, hi = (at ^ (db << 6) ^ 32) + 4096 * j2 + 2048;
                dv[db] = mfma16<HT>(trfrag_in(Os, lo, hi), pf, dv[db]);
                dk[db] = mfma16<HT>(trfrag_in(Qs, lo, hi), dsf, dk[db]);
            }
        }
        // issue order: transposed fragments (two reads each) two MFMAs ahead of their use
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int m = 0; m < 12; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };

    // two tiles per iteration on the two static stages (so the compiler sees that
    // reads of one stage never wait on loads into the other)
    issue(0, sQ0, sO0, sL0, sD0);
    publish();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kf[kk] = frag_in(sK, zk0 ^ (kk << 5));
    for (int it = 0; it < total; it += 2) {
        if (it + 1 < total) issue(it + 1, sQ1, sO1, sL1, sD1);
        compute(it, sQ0, sO0, sL0, sD0);
        publish();
        if (it + 2 < total) issue(it + 2, sQ0, sO0, sL0, sD0);
        if (it + 1 < total) compute(it + 1, sQ1, sO1, sL1, sD1);
        publish();
    }

    // the second query half's shares go through LDS (all tiles consumed: the last publish
    // was a barrier), 32 KB per key block: dK then dV, 16 KB each, lane-major float4s
    float* red = kq == 0 ? reinterpret_cast<float*>(sK)
               : kq == 1 ? reinterpret_cast<float*>(sV)
               : kq == 2 ? reinterpret_cast<float*>(sQ0) : reinterpret_cast<float*>(sQ1);
    float* red2 = kq == 0 ? reinterpret_cast<float*>(sK) + 4096
                : kq == 1 ? reinterpret_cast<float*>(sV) + 4096
                : kq == 2 ? reinterpret_cast<float*>(sO0) : reinterpret_cast<float*>(sO1);
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int o = ((db * 4 + q4) * 64 + lane) * 4;
                *reinterpret_cast<float4*>(red + o) =
                    make_float4(dk[db][4 * q4], dk[db][4 * q4 + 1], dk[db][4 * q4 + 2], dk[db][4 * q4 + 3]);
                *reinterpret_cast<float4*>(red2 + o) =
                    make_float4(dv[db][4 * q4], dv[db][4 * q4 + 1], dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]);
            }
    }
    __syncthreads();
    if (qh == 1 || !active) return;
    const int key = kw + l32;
    bf16* kout = dqkv + (rowbase + key) * QKV + HD + g * D;
    float gk[4][16];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const int o = ((db * 4 + gg) * 64 + lane) * 4;
            const float4 pk = *reinterpret_cast<const float4*>(red + o);
            const float4 pv = *reinterpret_cast<const float4*>(red2 + o);
            const float ok[4] = {pk.x, pk.y, pk.z, pk.w}, ov[4] = {pv.x, pv.y, pv.z, pv.w};
            float c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gk[db][4 * gg + e] = (dk[db][4 * gg + e] + ok[e]) * scale;
                c[e] = dv[db][4 * gg + e] + ov[e];
            }
            Vec4<HT>::store(reinterpret_cast<HT*>(kout + KD + 32 * db + 8 * gg + 4 * hh), c);
        }
    rope_qknorm_bwd_row<HT>(gk, qkv + (rowbase + key) * QKV + HD + g * D, rstdk[(rowbase + key) * Hkv + g],
                        cosv + key * (D / 2), sinv + key * (D / 2), hh);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const float a[4] = {gk[db][4 * gg], gk[db][4 * gg + 1], gk[db][4 * gg + 2], gk[db][4 * gg + 3]};
            Vec4<HT>::store(reinterpret_cast<HT*>(kout + 32 * db + 8 * gg + 4 * hh), a);
        }
}

// ======================================================================== fp32 SIMT kernels
// One wave per (token, head); lane holds head dims lane, lane+64, ... (D/64 of them).
template <int D>
__global__ void __launch_bounds__(256)
attn_fwd_f32(const float* __restrict__ qkv, float* __restrict__ y, float* __restrict__ lse, int B, int T, int H, int Hkv)
{
    constexpr int E = D / 64;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= B * T * H) return;
    const int hq = wid % H, n = wid / H, t = n % T, b = n / T;
    const int g = hq / (H / Hkv);
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const float scale = 1.0f / sqrtf((float)D);
    float q[E], o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { q[e] = qkv[(size_t)n * QKV + hq * D + lane + 64 * e]; o[e] = 0.0f; }
    float m = -INFINITY, l = 0.0f;
    for (int j = 0; j <= t; ++j) {
        const float* kr = qkv + ((size_t)b * T + j) * QKV + HD + g * D;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) part += q[e] * kr[lane + 64 * e];
        const float sc = wave_sum(part) * scale;
        const float mn = fmaxf(m, sc);
        const float alpha = expf(m - mn), p = expf(sc - mn);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = o[e] * alpha + p * kr[KD + lane + 64 * e];
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) y[(size_t)n * HD + hq * D + lane + 64 * e] = o[e] / l;
    if (lane == 0) lse[((size_t)b * H + hq) * T + t] = m + logf(l);
}

template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_dq_f32(const float* __restrict__ qkv, const float* __restrict__ dy, const float* __restrict__ lse,
                const float* __restrict__ delta, float* __restrict__ dqkv, int B, int T, int H, int Hkv)
{
    constexpr int E = D / 64;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= B * T * H) return;
    const int hq = wid % H, n = wid / H, t = n % T, b = n / T;
    const int g = hq / (H / Hkv);
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const float scale = 1.0f / sqrtf((float)D);
    const float ls = lse[((size_t)b * H + hq) * T + t], dl = delta[((size_t)b * H + hq) * T + t];
    float q[E], go[E], dq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        q[e] = qkv[(size_t)n * QKV + hq * D + lane + 64 * e];
        go[e] = dy[(size_t)n * HD + hq * D + lane + 64 * e];
        dq[e] = 0.0f;
    }
    for (int j = 0; j <= t; ++j) {
        const float* kr = qkv + ((size_t)b * T + j) * QKV + HD + g * D;
        float ps = 0.0f, pd = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) { ps += q[e] * kr[lane + 64 * e]; pd += go[e] * kr[KD + lane + 64 * e]; }
        const float sc = wave_sum(ps) * scale, dpv = wave_sum(pd);
        const float p = expf(sc - ls);
        const float ds = p * (dpv - dl) * scale;
#pragma unroll
        for (int e = 0; e < E; ++e) dq[e] += ds * kr[lane + 64 * e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) dqkv[(size_t)n * QKV + hq * D + lane + 64 * e] = dq[e];
}

template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_dkdv_f32(const float* __restrict__ qkv, const float* __restrict__ dy, const float* __restrict__ lse,
                  const float* __restrict__ delta, float* __restrict__ dqkv, int B, int T, int H, int Hkv)
{
    constexpr int E = D / 64;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= B * T * Hkv) return;
    const int g = wid % Hkv, n = wid / Hkv, j = n % T, b = n / T;
    const int r = H / Hkv;
    const int QKV = (H + 2 * Hkv) * D, HD = H * D, KD = Hkv * D;
    const float scale = 1.0f / sqrtf((float)D);
    float k[E], v[E], dk[E], dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        k[e] = qkv[(size_t)n * QKV + HD + g * D + lane + 64 * e];
        v[e] = qkv[(size_t)n * QKV + HD + KD + g * D + lane + 64 * e];
        dk[e] = 0.0f;
        dv[e] = 0.0f;
    }
    for (int hq = g * r; hq < (g + 1) * r; ++hq)
        for (int t = j; t < T; ++t) {
            const size_t nt = (size_t)b * T + t;
            const float* qr = qkv + nt * QKV + hq * D;
            const float* gr = dy + nt * HD + hq * D;
            float ps = 0.0f, pd = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) { ps += qr[lane + 64 * e] * k[e]; pd += gr[lane + 64 * e] * v[e]; }
            const float sc = wave_sum(ps) * scale, dpv = wave_sum(pd);
            const size_t li = ((size_t)b * H + hq) * T + t;
            const float p = expf(sc - lse[li]);
            const float ds = p * (dpv - delta[li]) * scale;
#pragma unroll
            for (int e = 0; e < E; ++e) { dk[e] += ds * qr[lane + 64 * e]; dv[e] += p * gr[lane + 64 * e]; }
        }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        dqkv[(size_t)n * QKV + HD + g * D + lane + 64 * e] = dk[e];
        dqkv[(size_t)n * QKV + HD + KD + g * D + lane + 64 * e] = dv[e];
    }
}

// ======================================================================== host
hipError_t launch_attn_fwd(const AttnDesc& a, hipStream_t s) {
    if (mfma_dt(a.dt)) {
        if (a.D != 128 || a.T % 64) return hipErrorInvalidValue;
        // one 32-query block per wave, several workgroups per CU (softmax under the others' MFMAs): measured
        // faster than two blocks per wave at one workgroup per CU, and three workgroups with 32-key tiles
        // faster than two with 64-key tiles
        const int npos = (a.T + 127) / 128 * (a.H / a.Hkv);
        auto k = a.dt == Dt::F16 ? attn_fwd_bf16<1, f16, 32> : attn_fwd_bf16<1, bf16, 32>;
        hipLaunchKernelGGL(k, dim3(npos * a.Hkv * a.B), dim3(256), 0, s, (const bf16*)a.qkv, (bf16*)a.y, a.lse, a.T,
                           a.H, a.Hkv, a.B, attn_group(npos, 3));
        return hipGetLastError();
    }
    dim3 grid((unsigned)(((size_t)a.B * a.T * a.H + 3) / 4));
    if (a.D == 128)
        hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(256), 0, s, (const float*)a.qkv, (float*)a.y, a.lse, a.B,
                           a.T, a.H, a.Hkv);
    else if (a.D == 64)
        hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(256), 0, s, (const float*)a.qkv, (float*)a.y, a.lse, a.B,
                           a.T, a.H, a.Hkv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_bwd(const AttnDesc& a, hipStream_t s, int part) {
    const int N = a.B * a.T;
    const bool bf = mfma_dt(a.dt), h16 = a.dt == Dt::F16;
    if (bf ? (a.D != 128 || a.T % 64 || !a.rstdq || !a.rstdk || !a.cosv || !a.sinv) : (a.D != 128 && a.D != 64))
        return hipErrorInvalidValue;
    if (bf) {
        if (part == 0) {
            auto k = h16 ? attn_bwd_dq_bf16<2, f16> : attn_bwd_dq_bf16<2, bf16>;
            hipLaunchKernelGGL(k, dim3(((a.T + 127) / 128) * a.H * a.B), dim3(256), 0, s, (const bf16*)a.qkv,
                               (const bf16*)a.y, (const bf16*)a.dy, (const float*)a.lse, a.delta, (bf16*)a.dqkv, a.rstdq,
                               a.cosv, a.sinv, a.T, a.H, a.Hkv, a.B);
        } else {
            auto k = h16 ? attn_bwd_dkdv_bf16<f16> : attn_bwd_dkdv_bf16<bf16>;
            hipLaunchKernelGGL(k, dim3(((a.T + 127) / 128) * a.Hkv * a.B), dim3(512), 0, s, (const bf16*)a.qkv,
                               (const bf16*)a.dy, (const float*)a.delta, (bf16*)a.dqkv, a.rstdk, a.cosv, a.sinv, a.T,
                               a.H, a.Hkv, a.B);
        }
        return hipGetLastError();
    }
    dim3 gq((unsigned)(((size_t)N * a.H + 3) / 4)), gk((unsigned)(((size_t)N * a.Hkv + 3) / 4));
    const float* q = (const float*)a.qkv;
    const float* dy = (const float*)a.dy;
    float* dq = (float*)a.dqkv;
    if (part == 0) {
        dim3 dg((unsigned)(((size_t)N * a.H + 255) / 256));
        hipLaunchKernelGGL(attn_delta<float>, dg, dim3(256), 0, s, dy, (const float*)a.y, a.delta, N, a.T, a.H, a.D);
        if (a.D == 128)
            hipLaunchKernelGGL(attn_bwd_dq_f32<128>, gq, dim3(256), 0, s, q, dy, (const float*)a.lse,
                               (const float*)a.delta, dq, a.B, a.T, a.H, a.Hkv);
        else
            hipLaunchKernelGGL(attn_bwd_dq_f32<64>, gq, dim3(256), 0, s, q, dy, (const float*)a.lse,
                               (const float*)a.delta, dq, a.B, a.T, a.H, a.Hkv);
    } else {
        if (a.D == 128)
            hipLaunchKernelGGL(attn_bwd_dkdv_f32<128>, gk, dim3(256), 0, s, q, dy, (const float*)a.lse,
                               (const float*)a.delta, dq, a.B, a.T, a.H, a.Hkv);
        else
            hipLaunchKernelGGL(attn_bwd_dkdv_f32<64>, gk, dim3(256), 0, s, q, dy, (const float*)a.lse,
                               (const float*)a.delta, dq, a.B, a.T, a.H, a.Hkv);
    }
    return hipGetLastError();
}

}  // namespace ncgpt
