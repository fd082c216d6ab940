// Decode path: grouped NVFP4 projection over row-major weights (packed
// [N, K/2], scales [N, K/16]) for the few tokens routed to each expert.
//
// nvfp4_moe_grouped.rs, docs of moe_expert_gate_up_act_nvfp4_grouped and
// moe_expert_down_act_nvfp4_grouped: one block row per active-expert slot
// (grid y = cap = min(E, P)); blocks past the device-side active count exit;
// gate+up fuse the SiLU product into fp32 h[position, n]; down reads h and
// writes fp32 y[position, n].
//
// gfx950 mapping.  A block owns one unit of 32 weight rows (gate+up: 16
// columns of each matrix; down: 32 columns) of one expert and streams those
// rows' packed bytes once.  The unit's E4M3 scales are staged in LDS first,
// so the only vector-memory loads in the inner loops are the 16-byte weight
// chunks (and, on the matrix-core path, the activation chunks that travel
// with them): the loops refill a ring of them without branching, which keeps
// the waits partial and several chunks in flight per lane.  The block picks
// one of two code paths from the expert's row count (uniform over the block):
//
//   one routed row  -> VALU GEMV.  16 groups of 16 lanes; group g owns the
//     row pair (g, g+16) (gate and up of one column, or two down columns),
//     lane j of the group the 16-byte chunks j, j+16, ... of the K axis.
//     The activation row is staged in LDS as bf16.  E2M1 -> f32 pairs with the
//     hardware converter, fp32 FMAs, the E4M3 scale applied once per 16
//     products, the 16 partial sums combined with DPP.
//
//   2 .. n rows     -> matrix cores, 16x16x32 bf16 MFMA in passes of 16 rows.
//     The 4 waves split the K axis (wave w takes K-tiles w, w+4, ... of 128
//     k); lane (r, q) decodes the 16-byte chunk of row pair (r, r+16) at
//     k = tile*128 + 32q straight into its B operands (E2M1 -> f32 pairs,
//     times the E4M3 scale, -> bf16: exact) and loads the same 32 k of
//     activation row r as its A operands (bf16 x as is; fp32 h rounded to
//     bf16).  The four waves' partial tiles are summed through LDS.  Decoding
//     each weight once per pass keeps the VALU work per weight byte
//     independent of the row count, which a GEMV does not (its FMAs grow with
//     the rows).
#include "moe_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / moe::kWave;
constexpr int kUnitRows = 32;  // weight rows per block
constexpr int kKT = 128;       // k per MFMA K-tile: one 16-byte chunk per lane group
constexpr int kDepth = 6;      // VALU path: chunks in flight per lane and row
constexpr int kRing = 3;       // MFMA path: K-tiles in flight per wave
constexpr int kPassRows = 16;  // MFMA path: rows per pass (one 16-row tile)
constexpr int kRedBytes = kWaves * 2 * 4 * 64 * (int)sizeof(float);  // MFMA partial tiles

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

struct DecArgs {
    const void *act;            // gate+up: bf16 x [T, K]; down: fp32 h [P, K]
    const int32_t *sorted_tok;  // gate+up only
    const int32_t *offsets;
    const int32_t *active;
    const uint8_t *const *pa;   // gate (or down)
    const uint8_t *const *sa;
    const float *s2a;
    const uint8_t *const *pb;   // up (gate+up only)
    const uint8_t *const *sb;
    const float *s2b;
    float *out;                 // [P, N]
    int N, K;
};

template <int B>
__device__ __forceinline__ f32x2_t e2m1x2_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

// The unit's 32 scale rows -> LDS, row rho at sl + rho * (K/16).  Rows of one
// matrix are consecutive in memory (16 or 32 rows of K/16 bytes each), so the
// copy is one or two contiguous runs of 16-byte units.
template <bool GATED>
__device__ __forceinline__ void stage_scales(int K, int n0, const uint8_t *sA, const uint8_t *sB, uint8_t *sl) {
    const int rowb = K >> 4;
    if constexpr (GATED) {
        const int units = (16 * rowb) >> 4;  // per matrix
        const uint8_t *ga = sA + (size_t)n0 * rowb, *gb = sB + (size_t)n0 * rowb;
        for (int u = threadIdx.x; u < 2 * units; u += kThreads) {
            const uint8_t *src = u < units ? ga + 16 * u : gb + 16 * (u - units);
            *reinterpret_cast<uint4 *>(sl + 16 * u) = moe::gload<uint4>(src);
        }
    } else {
        const int units = (32 * rowb) >> 4;
        const uint8_t *ga = sA + (size_t)n0 * rowb;
        for (int u = threadIdx.x; u < units; u += kThreads)
            *reinterpret_cast<uint4 *>(sl + 16 * u) = moe::gload<uint4>(ga + 16 * u);
    }
}

// ---------------------------------------------------------------------------
// VALU path (one routed row)
// ---------------------------------------------------------------------------

// acc += s_lo * sum_{e<16} w_e a_e + s_hi * sum_{e>=16} w_e a_e over one chunk.
__device__ __forceinline__ float chunk_fma(const uint4 &w, uint32_t sc, const float (&a)[32], float acc) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float p[2] = {0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t v = ww[2 * h + d];
            const f32x2_t e0 = e2m1x2_f32<0>(v), e1 = e2m1x2_f32<1>(v), e2 = e2m1x2_f32<2>(v),
                          e3 = e2m1x2_f32<3>(v);
            const int o = 16 * h + 8 * d;
            s0 = fmaf(e0.x, a[o + 0], s0);
            s1 = fmaf(e0.y, a[o + 1], s1);
            s0 = fmaf(e1.x, a[o + 2], s0);
            s1 = fmaf(e1.y, a[o + 3], s1);
            s0 = fmaf(e2.x, a[o + 4], s0);
            s1 = fmaf(e2.y, a[o + 5], s1);
            s0 = fmaf(e3.x, a[o + 6], s0);
            s1 = fmaf(e3.y, a[o + 7], s1);
        }
        p[h] = s0 + s1;
    }
    return fmaf(moe::e4m3_f32<1>(sc), p[1], fmaf(moe::e4m3_f32<0>(sc), p[0], acc));
}

// The one activation row -> LDS as bf16 (h is rounded to bf16 here).
template <bool GATED>
__device__ __forceinline__ void stage_row(const DecArgs &a, int pos, uint16_t *xs) {
    const int K = a.K;
    if constexpr (GATED) {
        const uint16_t *src =
            static_cast<const uint16_t *>(a.act) + (size_t)moe::gload<int32_t>(a.sorted_tok + pos) * K;
        for (int u = threadIdx.x; u < (K >> 3); u += kThreads)
            reinterpret_cast<uint4 *>(xs)[u] = moe::gload<uint4>(src + 8 * u);
    } else {
        const float *src = static_cast<const float *>(a.act) + (size_t)pos * K;
        for (int u = threadIdx.x; u < (K >> 2); u += kThreads) {
            const float4 f = moe::gload<float4>(src + 4 * u);
            uint2 v;
            v.x = (uint32_t)moe::f32_to_bf16_rne(f.x) | ((uint32_t)moe::f32_to_bf16_rne(f.y) << 16);
            v.y = (uint32_t)moe::f32_to_bf16_rne(f.z) | ((uint32_t)moe::f32_to_bf16_rne(f.w) << 16);
            reinterpret_cast<uint2 *>(xs)[u] = v;
        }
    }
}

template <bool GATED>
__device__ __forceinline__ void valu_one_row(const DecArgs &a, int pos, int n0, const uint8_t *p0,
                                             const uint8_t *p1, float s2A, float s2B, const uint8_t *sl,
                                             const uint16_t *xs) {
    constexpr int D = kDepth;
    const int K = a.K, N = a.N;
    const int g = threadIdx.x >> 4, j = threadIdx.x & 15;
    const int Kc = K >> 5;
    const int nch = (Kc + 15) >> 4;  // uniform trip count
    const int rowb = K >> 4;
    const uint8_t *sl0 = sl + g * rowb, *sl1 = sl + (g + 16) * rowb;

    uint4 w0[D], w1[D];
    bool ok[D];
    auto load = [&](int d, int i) {
        const int cr = j + 16 * i;
        ok[d] = i < nch && cr < Kc;
        const int c = ok[d] ? cr : 0;  // past the end: load chunk 0, its products are dropped
        w0[d] = moe::gload<uint4>(p0 + (size_t)c * 16);
        w1[d] = moe::gload<uint4>(p1 + (size_t)c * 16);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
    }
    __syncthreads();  // scales and the activation row are in LDS

    float acc0 = 0.f, acc1 = 0.f;
    // The trip count is padded to a multiple of the ring and every step refills
    // its slot, so the loop body has no branch around a load; padded and
    // out-of-range chunks add nothing.
    for (int base = 0; base < nch; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = base + d;
            const int c = ok[d] ? j + 16 * i : 0;
            const uint4 *xc = reinterpret_cast<const uint4 *>(xs) + (size_t)c * 4;
            float av[32];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 u = xc[v];
                const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    av[8 * v + 2 * k] = __uint_as_float(uu[k] << 16);
                    av[8 * v + 2 * k + 1] = __uint_as_float(uu[k] & 0xffff0000u);
                }
            }
            const uint32_t s0 = *reinterpret_cast<const uint16_t *>(sl0 + 2 * c);
            const uint32_t s1 = *reinterpret_cast<const uint16_t *>(sl1 + 2 * c);
            const float n0v = chunk_fma(w0[d], s0, av, acc0);
            const float n1v = chunk_fma(w1[d], s1, av, acc1);
            acc0 = ok[d] ? n0v : acc0;
            acc1 = ok[d] ? n1v : acc1;
            __builtin_amdgcn_sched_barrier(0);
            load(d, i + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    acc0 = moe::group_sum<16>(acc0);
    acc1 = moe::group_sum<16>(acc1);
    if (j == 0) {
        if constexpr (GATED) {
            a.out[(size_t)pos * N + n0 + g] = moe::silu_f32(acc0 * s2A) * (acc1 * s2B);
        } else {
            a.out[(size_t)pos * N + n0 + g] = acc0 * s2A;
            a.out[(size_t)pos * N + n0 + g + 16] = acc1 * s2A;
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA path (two or more routed rows)
// ---------------------------------------------------------------------------

// 8 E2M1 codes (one 32-bit word: k .. k+7) times the block scale, as bf16.
// The f32 products are exact (at most 6 significant bits), so is their bf16 form.
__device__ __forceinline__ bf16x8_t decode_b(uint32_t w, float s) {
    const f32x2_t v0 = e2m1x2_f32<0>(w), v1 = e2m1x2_f32<1>(w), v2 = e2m1x2_f32<2>(w), v3 = e2m1x2_f32<3>(w);
    const bf16x2v_t r0 = __builtin_convertvector((f32x2_t){v0.x * s, v0.y * s}, bf16x2v_t);
    const bf16x2v_t r1 = __builtin_convertvector((f32x2_t){v1.x * s, v1.y * s}, bf16x2v_t);
    const bf16x2v_t r2 = __builtin_convertvector((f32x2_t){v2.x * s, v2.y * s}, bf16x2v_t);
    const bf16x2v_t r3 = __builtin_convertvector((f32x2_t){v3.x * s, v3.y * s}, bf16x2v_t);
    bf16x8_t r;
    r[0] = r0.x;
    r[1] = r0.y;
    r[2] = r1.x;
    r[3] = r1.y;
    r[4] = r2.x;
    r[5] = r2.y;
    r[6] = r3.x;
    r[7] = r3.y;
    return r;
}

__device__ __forceinline__ bf16x8_t f32x8_to_bf16(const uint4 &x0, const uint4 &x1) {
    const bf16x2v_t r0 = __builtin_convertvector((f32x2_t){__uint_as_float(x0.x), __uint_as_float(x0.y)}, bf16x2v_t);
    const bf16x2v_t r1 = __builtin_convertvector((f32x2_t){__uint_as_float(x0.z), __uint_as_float(x0.w)}, bf16x2v_t);
    const bf16x2v_t r2 = __builtin_convertvector((f32x2_t){__uint_as_float(x1.x), __uint_as_float(x1.y)}, bf16x2v_t);
    const bf16x2v_t r3 = __builtin_convertvector((f32x2_t){__uint_as_float(x1.z), __uint_as_float(x1.w)}, bf16x2v_t);
    bf16x8_t r;
    r[0] = r0.x;
    r[1] = r0.y;
    r[2] = r1.x;
    r[3] = r1.y;
    r[4] = r2.x;
    r[5] = r2.y;
    r[6] = r3.x;
    r[7] = r3.y;
    return r;
}

template <bool GATED>
struct KTile {
    uint4 w0, w1;             // 16-byte chunk of each row of the pair
    uint4 av[GATED ? 4 : 8];  // activation row r: 32 bf16 (x) or 32 fp32 (h)
};

template <bool GATED>
__device__ __forceinline__ void mfma_rows(const DecArgs &a, int lo, int rows, int n0, const uint8_t *p0,
                                          const uint8_t *p1, float s2A, float s2B, const uint8_t *sl,
                                          float *red) {
    const int K = a.K, N = a.N;
    const int lane = threadIdx.x & 63, w = moe::wave_id();
    const int r = lane & 15, q = lane >> 4;
    const int rowb = K >> 4;
    const uint8_t *sl0 = sl + r * rowb, *sl1 = sl + (r + 16) * rowb;
    const int c0 = n0 + r;
    const int c1 = GATED ? n0 + r : n0 + r + 16;
    const int nkt = (K + kKT - 1) / kKT;
    const int cnt = w < nkt ? (nkt - 1 - w) / kWaves + 1 : 0;
    __syncthreads();  // scales are in LDS

    for (int m0 = 0; m0 < rows; m0 += kPassRows) {
        const int mr = min(kPassRows, rows - m0);
        // Rows past the pass read the pass's row 0: they only feed dropped outputs.
        const int mrow = lo + m0 + (r < mr ? r : 0);
        const void *arow;
        if constexpr (GATED)
            arow = static_cast<const uint16_t *>(a.act) + (size_t)moe::gload<int32_t>(a.sorted_tok + mrow) * K;
        else
            arow = static_cast<const float *>(a.act) + (size_t)mrow * K;

        KTile<GATED> ring[kRing];
        bool kin[kRing];
        int kq_[kRing];
        auto load = [&](int d, int i) {
            const int kr = (w + kWaves * min(i, cnt - 1)) * kKT + 32 * q;
            kin[d] = i < cnt && kr < K;
            const int kq = kin[d] ? kr : 0;  // padding / past the end: k = 0, scaled by zero below
            kq_[d] = kq;
            ring[d].w0 = moe::gload<uint4>(p0 + (kq >> 1));
            ring[d].w1 = moe::gload<uint4>(p1 + (kq >> 1));
            constexpr int NV = GATED ? 4 : 8;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if constexpr (GATED)
                    ring[d].av[v] = moe::gload<uint4>(static_cast<const uint16_t *>(arow) + kq + 8 * v);
                else
                    ring[d].av[v] = moe::gload<uint4>(static_cast<const float *>(arow) + kq + 4 * v);
            }
        };

        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        if (cnt > 0) {  // uniform: a wave past the last K-tile only adds zeros below
#pragma unroll
            for (int d = 0; d < kRing; ++d) {
                load(d, d);
                __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
            }
            // The trip count is padded to a multiple of the ring and every step
            // refills its slot (padding tiles have zero scales), so the loop body
            // has no branch around a load and the waits on the ring stay partial.
            for (int base = 0; base < cnt; base += kRing) {
#pragma unroll
                for (int d = 0; d < kRing; ++d) {
                    const KTile<GATED> &t = ring[d];
                    const uint32_t r0 = *reinterpret_cast<const uint16_t *>(sl0 + (kq_[d] >> 4));
                    const uint32_t r1 = *reinterpret_cast<const uint16_t *>(sl1 + (kq_[d] >> 4));
                    const uint32_t s0 = kin[d] ? r0 : 0u, s1 = kin[d] ? r1 : 0u;
                    const float sl_0 = moe::e4m3_f32<0>(s0), sh_0 = moe::e4m3_f32<1>(s0);
                    const float sl_1 = moe::e4m3_f32<0>(s1), sh_1 = moe::e4m3_f32<1>(s1);
                    const uint32_t u0[4] = {t.w0.x, t.w0.y, t.w0.z, t.w0.w};
                    const uint32_t u1[4] = {t.w1.x, t.w1.y, t.w1.z, t.w1.w};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        bf16x8_t A;
                        if constexpr (GATED)
                            A = moe::bitcast<bf16x8_t>(t.av[ks]);
                        else
                            A = f32x8_to_bf16(t.av[2 * ks], t.av[2 * ks + 1]);
                        const bf16x8_t b0 = decode_b(u0[ks], ks < 2 ? sl_0 : sh_0);
                        const bf16x8_t b1 = decode_b(u1[ks], ks < 2 ? sl_1 : sh_1);
                        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, b0, acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, b1, acc1, 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    load(d, base + d + kRing);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // Sum the four waves' partial tiles: red[((w*2 + mat)*4 + i)*64 + lane].
        __syncthreads();  // the previous pass's readers are done
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[((w * 2 + 0) * 4 + i) * 64 + lane] = acc0[i];
            red[((w * 2 + 1) * 4 + i) * 64 + lane] = acc1[i];
        }
        __syncthreads();
        // Wave w finishes row i = w of each lane's four: row 4q + w of the tile.
        {
            const int i = w;
            float v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                v0 += red[((ww * 2 + 0) * 4 + i) * 64 + lane];
                v1 += red[((ww * 2 + 1) * 4 + i) * 64 + lane];
            }
            const int m = m0 + 4 * q + i;
            if (m < rows) {
                float *o = a.out + (size_t)(lo + m) * N;
                if constexpr (GATED) {
                    o[c0] = moe::silu_f32(v0 * s2A) * (v1 * s2B);
                } else {
                    o[c0] = v0 * s2A;
                    o[c1] = v1 * s2A;
                }
            }
        }
    }
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_decode_row(DecArgs a) {
    // LDS: [the unit's scales: 32 x K/16 bytes][activation row (VALU) | partial tiles (MFMA)]
    extern __shared__ uint4 lds4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);

    const int e = a.active[blockIdx.y];  // -1 past the active count
    if (e < 0) return;
    const int lo = a.offsets[e], rows = a.offsets[e + 1] - lo;
    const int K = a.K;
    const int n0 = blockIdx.x * (GATED ? kUnitRows / 2 : kUnitRows);
    const uint8_t *pA = a.pa[e];
    const uint8_t *pB = GATED ? a.pb[e] : pA;
    if (pA == nullptr || pB == nullptr) {  // absent expert: its rows are zero
        const int ncols = GATED ? kUnitRows / 2 : kUnitRows;
        for (int i = threadIdx.x; i < rows * ncols; i += kThreads) {
            const int m = i / ncols;
            a.out[(size_t)(lo + m) * a.N + n0 + (i - m * ncols)] = 0.f;
        }
        return;
    }
    const uint8_t *sA = a.sa[e];
    const uint8_t *sB = GATED ? a.sb[e] : sA;
    const float s2A = a.s2a[e];
    const float s2B = GATED ? a.s2b[e] : s2A;
    const size_t rb = (size_t)(K >> 1);
    uint8_t *sl = lds;
    uint8_t *rest = lds + 2 * (size_t)K;  // after 32 rows x K/16 bytes of scales
    stage_scales<GATED>(K, n0, sA, sB, sl);

    if (rows == 1) {
        const int g = threadIdx.x >> 4;
        const uint8_t *p0 = pA + (size_t)(n0 + g) * rb;
        const uint8_t *p1 = GATED ? pB + (size_t)(n0 + g) * rb : pA + (size_t)(n0 + g + 16) * rb;
        stage_row<GATED>(a, lo, reinterpret_cast<uint16_t *>(rest));
        valu_one_row<GATED>(a, lo, n0, p0, p1, s2A, s2B, sl, reinterpret_cast<const uint16_t *>(rest));
    } else {
        const int r = threadIdx.x & 15;
        const uint8_t *p0 = pA + (size_t)(n0 + r) * rb;
        const uint8_t *p1 = GATED ? pB + (size_t)(n0 + r) * rb : pA + (size_t)(n0 + r + 16) * rb;
        mfma_rows<GATED>(a, lo, rows, n0, p0, p1, s2A, s2B, sl, reinterpret_cast<float *>(rest));
    }
}

}  // namespace

// Launch the row-major grouped projection (used by the two C-ABI entry points).
int moe_launch_decode_row(bool gated, const void *act, const int32_t *sorted_tok, const int32_t *offsets,
                          const int32_t *active, const moe_nvfp4_experts &A, const moe_nvfp4_experts *B,
                          float *out, int N, int K, int P, int E, hipStream_t stream) {
    DecArgs a;
    a.act = act;
    a.sorted_tok = sorted_tok;
    a.offsets = offsets;
    a.active = active;
    a.pa = A.packed;
    a.sa = A.scale;
    a.s2a = A.scale2;
    a.pb = B ? B->packed : nullptr;
    a.sb = B ? B->scale : nullptr;
    a.s2b = B ? B->scale2 : nullptr;
    a.out = out;
    a.N = N;
    a.K = K;
    const int cols = gated ? kUnitRows / 2 : kUnitRows;
    const int cap = E < P ? E : P;
    dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)cap);
    size_t tail = (size_t)kRedBytes;                  // MFMA partial tiles
    if ((size_t)K * 2 > tail) tail = (size_t)K * 2;   // VALU activation row (bf16)
    const size_t lds = (size_t)K * 2 + tail;          // + the unit's scales
    if (lds > 160 * 1024) return MOE_NVFP4_ELIMIT;
    if (gated)
        hipLaunchKernelGGL(k_decode_row<true>, grid, dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(k_decode_row<false>, grid, dim3(kThreads), lds, stream, a);
    return moe_host::launch_status();
}
