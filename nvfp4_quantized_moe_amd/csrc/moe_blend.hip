// Weighted top-k blend: out[t, n] = bf16_rne(sum_j w[t, j] * y[pair_pos[t*k + j], n]).
//
// nvfp4_moe_grouped.rs, module doc: the grouped layout ends with a weighted
// sum over each token's top-k rows of the down output, which sit at sorted
// positions.  Sum in fp32, ascending j, one rounding to bf16 at the end.
// HBM-bound: each thread streams four consecutive columns of the k rows.
#include "moe_common.hpp"

namespace {

constexpr int kBlendThreads = 256;

__global__ __launch_bounds__(kBlendThreads) void k_moe_blend(const float *__restrict__ y,
                                                            const float *__restrict__ w,
                                                            const int32_t *__restrict__ pair_pos, int k,
                                                            int H, int nb, uint16_t *__restrict__ out) {
    const int t = blockIdx.x / nb;
    const int n = ((blockIdx.x - t * nb) * kBlendThreads + threadIdx.x) * 4;
    if (n >= H) return;
    const int32_t *pp = pair_pos + (size_t)t * k;
    const float *wt = w + (size_t)t * k;
    uint16_t *o = out + (size_t)t * H;
    if ((H & 3) == 0) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        // Eight pairs at a time: their positions and weights first, then all
        // eight rows of y, so the loads of a token overlap instead of chaining.
        for (int j0 = 0; j0 < k; j0 += 8) {
            int p[8];
            float wj[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = j0 + i < k;
                p[i] = in ? pp[j0 + i] : -1;
                wj[i] = in ? wt[j0 + i] : 0.f;
            }
            float4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)  // a pair of no expert reads row 0 and adds nothing
                v[i] = *reinterpret_cast<const float4 *>(y + (size_t)(p[i] < 0 ? 0 : p[i]) * H + n);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (p[i] < 0) continue;
                a0 = fmaf(wj[i], v[i].x, a0);
                a1 = fmaf(wj[i], v[i].y, a1);
                a2 = fmaf(wj[i], v[i].z, a2);
                a3 = fmaf(wj[i], v[i].w, a3);
            }
        }
        uint2 r;
        r.x = (uint32_t)moe::f32_to_bf16_rne(a0) | ((uint32_t)moe::f32_to_bf16_rne(a1) << 16);
        r.y = (uint32_t)moe::f32_to_bf16_rne(a2) | ((uint32_t)moe::f32_to_bf16_rne(a3) << 16);
        *reinterpret_cast<uint2 *>(o + n) = r;
    } else {
        for (int c = n; c < min(n + 4, H); ++c) {
            float a = 0.f;
            for (int j = 0; j < k; ++j) {
                const int p = pp[j];
                if (p >= 0) a = fmaf(wt[j], y[(size_t)p * H + c], a);
            }
            o[c] = moe::f32_to_bf16_rne(a);
        }
    }
}

}  // namespace

extern "C" int moe_nvfp4_blend(const float *y, const float *topk_weights, const int32_t *pair_pos,
                               int32_t T, int32_t k, int32_t H, uint16_t *out, void *stream) {
    if (!y || !topk_weights || !pair_pos || !out) return MOE_NVFP4_ENULL;
    if (T < 1 || k < 1 || H < 1) return MOE_NVFP4_ESHAPE;
    if ((int64_t)T * k > MOE_NVFP4_MAX_PAIRS || H > MOE_NVFP4_MAX_WIDTH) return MOE_NVFP4_ELIMIT;
    const int nb = (H + 4 * kBlendThreads - 1) / (4 * kBlendThreads);
    hipLaunchKernelGGL(k_moe_blend, dim3((unsigned)(nb * T)), dim3(kBlendThreads), 0, (hipStream_t)stream, y,
                       topk_weights, pair_pos, k, H, nb, out);
    return moe_host::launch_status();
}
