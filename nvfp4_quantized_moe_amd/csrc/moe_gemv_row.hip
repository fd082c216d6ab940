// Decode path: grouped NVFP4 GEMV over row-major weights (packed [N, K/2],
// scales [N, K/16]) for the few tokens routed to each active expert.
//
// nvfp4_moe_grouped.rs, docs of moe_expert_gate_up_act_nvfp4_grouped and
// moe_expert_down_act_nvfp4_grouped: one block row per active expert slot
// (grid y = cap), blocks past the device-side active count exit, and each
// block walks its expert's sorted rows in passes.  Gate+up fuse the SiLU
// product and write fp32 h[position, n]; down reads h and writes fp32
// y[position, n].
//
// gfx950 mapping (the work is HBM-bound: every weight byte is read once):
//   * a wavefront is split into groups of LPR lanes (LPR = 8 or 16, one
//     DPP row or half-row); a group owns CPL output columns, and each lane
//     of the group owns the 16-byte chunks c = j, j + LPR, ... of the K axis
//     (32 E2M1 values, two scale groups), so one wave load instruction reads
//     LPR*16 contiguous bytes from each of 64/LPR weight rows;
//   * the next chunk's weights are loaded before the current one is used;
//   * E2M1 -> bf16 pairs with the hardware converter, products with the bf16
//     dot2 instruction into fp32, and the E4M3 block scale applied once per
//     16 products;
//   * the activation rows of a pass are staged once per block in LDS as bf16
//     (gate+up: x gathered by token id; down: h converted from fp32), in a
//     swizzled order so the group's 16-byte LDS reads hit distinct banks;
//   * the LPR partial sums of each (column, token) are combined with DPP.
#include "moe_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / moe::kWave;

struct GemvArgs {
    const void *act;              // gate+up: bf16 x [T, K]; down: fp32 h [P, K]
    const int32_t *sorted_tok;    // gate+up only
    const int32_t *offsets;
    const int32_t *active;
    const int32_t *nactive;
    const uint8_t *const *pa;     // gate (or down) tables
    const uint8_t *const *sa;
    const float *s2a;
    const uint8_t *const *pb;     // up tables (gate+up only)
    const uint8_t *const *sb;
    const float *s2b;
    float *out;                   // [P, N]
    int N, K;
};

// LDS position (in bf16 elements) of 16-byte sub-block s of chunk c.
__device__ __forceinline__ int swz(int c, int s) { return c * 32 + ((s ^ ((c >> 2) & 3)) << 3); }

__device__ __forceinline__ void decode32(const uint4 &w, bf16x2_t (&d)[16]) {
    d[0] = moe::e2m1x2_bf16<0>(w.x);
    d[1] = moe::e2m1x2_bf16<1>(w.x);
    d[2] = moe::e2m1x2_bf16<2>(w.x);
    d[3] = moe::e2m1x2_bf16<3>(w.x);
    d[4] = moe::e2m1x2_bf16<0>(w.y);
    d[5] = moe::e2m1x2_bf16<1>(w.y);
    d[6] = moe::e2m1x2_bf16<2>(w.y);
    d[7] = moe::e2m1x2_bf16<3>(w.y);
    d[8] = moe::e2m1x2_bf16<0>(w.z);
    d[9] = moe::e2m1x2_bf16<1>(w.z);
    d[10] = moe::e2m1x2_bf16<2>(w.z);
    d[11] = moe::e2m1x2_bf16<3>(w.z);
    d[12] = moe::e2m1x2_bf16<0>(w.w);
    d[13] = moe::e2m1x2_bf16<1>(w.w);
    d[14] = moe::e2m1x2_bf16<2>(w.w);
    d[15] = moe::e2m1x2_bf16<3>(w.w);
}

// acc += s0 * sum(first 16 products) + s1 * sum(last 16 products)
__device__ __forceinline__ float dot32(const bf16x2_t (&d)[16], const bf16x2_t (&xv)[16], float s0,
                                       float s1, float acc) {
    float p0 = 0.f, p1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0 = moe::dot2_bf16(d[i], xv[i], p0);
        q0 = moe::dot2_bf16(d[4 + i], xv[4 + i], q0);
        p1 = moe::dot2_bf16(d[8 + i], xv[8 + i], p1);
        q1 = moe::dot2_bf16(d[12 + i], xv[12 + i], q1);
    }
    return fmaf(s1, p1 + q1, fmaf(s0, p0 + q0, acc));
}

template <bool GATED>
__device__ __forceinline__ void stage_rows(const GemvArgs &a, uint16_t *xs, int start, int nt) {
    // nt rows of K activations -> LDS bf16, swizzled per 64-byte chunk.
    const int K = a.K;
    const int units_per_row = K >> 3;  // 16-byte units of bf16
    const int units = nt * units_per_row;
    for (int u = threadIdx.x; u < units; u += kThreads) {
        const int t = u / units_per_row;
        const int r = u - t * units_per_row;
        const int c = r >> 2, s = r & 3;
        uint4 v;
        if constexpr (GATED) {
            const int tok = a.sorted_tok[start + t];
            v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + (size_t)tok * K + r * 8);
        } else {
            const float *src = static_cast<const float *>(a.act) + (size_t)(start + t) * K + r * 8;
            const float4 f0 = *reinterpret_cast<const float4 *>(src);
            const float4 f1 = *reinterpret_cast<const float4 *>(src + 4);
            v.x = (uint32_t)moe::f32_to_bf16_rne(f0.x) | ((uint32_t)moe::f32_to_bf16_rne(f0.y) << 16);
            v.y = (uint32_t)moe::f32_to_bf16_rne(f0.z) | ((uint32_t)moe::f32_to_bf16_rne(f0.w) << 16);
            v.z = (uint32_t)moe::f32_to_bf16_rne(f1.x) | ((uint32_t)moe::f32_to_bf16_rne(f1.y) << 16);
            v.w = (uint32_t)moe::f32_to_bf16_rne(f1.z) | ((uint32_t)moe::f32_to_bf16_rne(f1.w) << 16);
        }
        *reinterpret_cast<uint4 *>(xs + (size_t)t * K + swz(c, s)) = v;
    }
}

// One pass over up to TT sorted rows [start, start + nt) of this block's expert.
template <bool GATED, int LPR, int CPL, int TT>
__device__ __forceinline__ void gemv_pass(const GemvArgs &a, uint16_t *xs, int start, int nt, bool grp_on,
                                          int col0, int j, const uint8_t *pA, const uint8_t *sA, float s2A,
                                          const uint8_t *pB, const uint8_t *sB, float s2B) {
    constexpr int R = GATED ? 2 : 1;  // weight matrices per column
    const int K = a.K, N = a.N;
    const int Kc = K >> 5;
    const size_t rbytes = (size_t)(K >> 1), sbytes = (size_t)(K >> 4);

    __syncthreads();  // the previous pass is done reading xs
    stage_rows<GATED>(a, xs, start, nt);
    __syncthreads();

    float acc[R][CPL][TT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < CPL; ++q)
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[r][q][t] = 0.f;

    if (grp_on && j < Kc) {
        const uint8_t *pbase[R], *sbase[R];
        pbase[0] = pA + (size_t)col0 * rbytes;
        sbase[0] = sA + (size_t)col0 * sbytes;
        if constexpr (GATED) {
            pbase[R - 1] = pB + (size_t)col0 * rbytes;
            sbase[R - 1] = sB + (size_t)col0 * sbytes;
        }
        uint4 w[R][CPL];
        uint32_t sc[R][CPL];
        auto load = [&](int c, uint4 (&wd)[R][CPL], uint32_t (&sd)[R][CPL]) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < CPL; ++q) {
                    wd[r][q] = *reinterpret_cast<const uint4 *>(pbase[r] + q * rbytes + (size_t)c * 16);
                    sd[r][q] = *reinterpret_cast<const uint16_t *>(sbase[r] + q * sbytes + (size_t)c * 2);
                }
        };
        load(j, w, sc);
        for (int c = j; c < Kc; c += LPR) {
            uint4 wn[R][CPL];
            uint32_t sn[R][CPL];
            const int cn = c + LPR;
            if (cn < Kc) load(cn, wn, sn);

            bf16x2_t d[R][CPL][16];
            float s0[R][CPL], s1[R][CPL];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < CPL; ++q) {
                    decode32(w[r][q], d[r][q]);
                    s0[r][q] = moe::e4m3_f32<0>(sc[r][q]);
                    s1[r][q] = moe::e4m3_f32<1>(sc[r][q]);
                }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                bf16x2_t xv[16];
                const uint16_t *xr = xs + (size_t)t * K;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(xr + swz(c, s));
                    xv[4 * s + 0] = moe::bitcast<bf16x2_t>(v.x);
                    xv[4 * s + 1] = moe::bitcast<bf16x2_t>(v.y);
                    xv[4 * s + 2] = moe::bitcast<bf16x2_t>(v.z);
                    xv[4 * s + 3] = moe::bitcast<bf16x2_t>(v.w);
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < CPL; ++q) acc[r][q][t] = dot32(d[r][q], xv, s0[r][q], s1[r][q], acc[r][q][t]);
            }
            if (cn < Kc) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < CPL; ++q) {
                        w[r][q] = wn[r][q];
                        sc[r][q] = sn[r][q];
                    }
            }
        }
    }
    // Combine the group's partial sums (every group runs this: DPP stays in-group).
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < CPL; ++q)
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[r][q][t] = moe::group_sum<LPR>(acc[r][q][t]);

    if (!grp_on) return;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < nt && ((q * TT + t) % LPR) == j) {
                float v;
                if constexpr (GATED)
                    v = moe::silu_f32(acc[0][q][t] * s2A) * (acc[R - 1][q][t] * s2B);
                else
                    v = acc[0][q][t] * s2A;
                a.out[(size_t)(start + t) * N + col0 + q] = v;
            }
        }
}

template <bool GATED, int LPR, int CPL, int TTMAX>
__global__ __launch_bounds__(kThreads) void k_gemv_row(GemvArgs a) {
    constexpr int GPW = moe::kWave / LPR;
    extern __shared__ uint4 lds_raw[];
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds_raw);

    const int slot = blockIdx.y;
    if (slot >= *a.nactive) return;  // uniform over the block
    const int e = a.active[slot];
    const int lo = a.offsets[e], hi = a.offsets[e + 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / LPR, j = lane % LPR;
    const int col0 = ((blockIdx.x * kWaves + wave) * GPW + grp) * CPL;
    const bool grp_on = col0 < a.N;

    const uint8_t *pA = a.pa[e];
    const uint8_t *pB = GATED ? a.pb[e] : pA;
    if (pA == nullptr || pB == nullptr) {  // absent expert: its rows are zero
        if (grp_on && j < CPL)
            for (int p = lo; p < hi; ++p) a.out[(size_t)p * a.N + col0 + j] = 0.f;
        return;
    }
    const uint8_t *sA = a.sa[e];
    const float s2A = a.s2a[e];
    const uint8_t *sB = GATED ? a.sb[e] : sA;
    const float s2B = GATED ? a.s2b[e] : s2A;

    for (int start = lo; start < hi;) {
        const int rem = hi - start;
        if (TTMAX >= 8 && rem > 4) {
            const int nt = rem < 8 ? rem : 8;
            gemv_pass<GATED, LPR, CPL, (TTMAX >= 8 ? 8 : 1)>(a, xs, start, nt, grp_on, col0, j, pA, sA, s2A, pB, sB, s2B);
            start += nt;
        } else if (TTMAX >= 4 && rem > 2) {
            const int nt = rem < 4 ? rem : 4;
            gemv_pass<GATED, LPR, CPL, (TTMAX >= 4 ? 4 : 1)>(a, xs, start, nt, grp_on, col0, j, pA, sA, s2A, pB, sB, s2B);
            start += nt;
        } else if (TTMAX >= 2 && rem >= 2) {
            gemv_pass<GATED, LPR, CPL, (TTMAX >= 2 ? 2 : 1)>(a, xs, start, 2, grp_on, col0, j, pA, sA, s2A, pB, sB, s2B);
            start += 2;
        } else {
            gemv_pass<GATED, LPR, CPL, 1>(a, xs, start, 1, grp_on, col0, j, pA, sA, s2A, pB, sB, s2B);
            start += 1;
        }
    }
}

using KernelFn = void (*)(GemvArgs);

template <bool GATED, int LPR>
KernelFn pick_tt(int ttmax) {
    constexpr int CPL = GATED ? 2 : 4;
    switch (ttmax) {
        case 8: return k_gemv_row<GATED, LPR, CPL, 8>;
        case 4: return k_gemv_row<GATED, LPR, CPL, 4>;
        case 2: return k_gemv_row<GATED, LPR, CPL, 2>;
        default: return k_gemv_row<GATED, LPR, CPL, 1>;
    }
}

// Lanes per column group: the LPR in {8, 16} that leaves the fewest idle
// chunk slots on the K axis (ties go to 16: wider contiguous reads).
int pick_lpr(int K) {
    const int kc = K / 32;
    const int w16 = ((kc + 15) / 16) * 16 - kc;
    const int w8 = ((kc + 7) / 8) * 8 - kc;
    return w8 < w16 ? 8 : 16;
}

constexpr size_t kLdsBudget = 64 * 1024;

}  // namespace

// Launch the row-major grouped GEMV (used by the two C-ABI entry points).
int moe_launch_gemv_row(bool gated, const void *act, const int32_t *sorted_tok, const int32_t *offsets,
                        const int32_t *active, const int32_t *nactive, const moe_nvfp4_experts &A,
                        const moe_nvfp4_experts *B, float *out, int N, int K, int P, int E,
                        hipStream_t stream) {
    GemvArgs a;
    a.act = act;
    a.sorted_tok = sorted_tok;
    a.offsets = offsets;
    a.active = active;
    a.nactive = nactive;
    a.pa = A.packed;
    a.sa = A.scale;
    a.s2a = A.scale2;
    a.pb = B ? B->packed : nullptr;
    a.sb = B ? B->scale : nullptr;
    a.s2b = B ? B->scale2 : nullptr;
    a.out = out;
    a.N = N;
    a.K = K;

    int ttmax = 8;
    while (ttmax > 1 && (ttmax > P || (size_t)ttmax * K * 2 > kLdsBudget)) ttmax >>= 1;
    const size_t lds = (size_t)ttmax * K * 2;
    const int lpr = pick_lpr(K);
    KernelFn fn;
    if (gated)
        fn = lpr == 8 ? pick_tt<true, 8>(ttmax) : pick_tt<true, 16>(ttmax);
    else
        fn = lpr == 8 ? pick_tt<false, 8>(ttmax) : pick_tt<false, 16>(ttmax);
    const int cpl = gated ? 2 : 4;
    const int cols_per_block = kWaves * (moe::kWave / lpr) * cpl;
    const int cap = E < P ? E : P;
    dim3 grid((unsigned)((N + cols_per_block - 1) / cols_per_block), (unsigned)cap);
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, stream, a);
    return moe_host::launch_status();
}
