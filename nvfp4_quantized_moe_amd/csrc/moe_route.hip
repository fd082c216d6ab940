// Router ahead of the path: for each token, the k experts with the largest
// logits and their softmax weights renormalised over those k.  The pages show
// only the router's logit GEMM (prefill_weights.rs, doc of dense_gemm_prefill:
// the gate GEMM); the selection and weights are the routing the workloads are
// defined by, and the output feeds moe_nvfp4_sort and moe_nvfp4_blend.
//
// One wavefront per token: each lane holds up to 16 of the E logits (expert
// lane + 64 i) as order keys; k rounds of a wave-wide argmax (larger key
// first, then lower expert id; a DPP maximum of the keys, then a DPP minimum
// of the ids holding it) pick the experts in descending order.  The
// softmax denominator over all E cancels in the renormalisation, so the
// weights are exp(l_j - l_max) over the k selected, summed across the wave.
#include "moe_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kPerLane = MOE_NVFP4_MAX_EXPERTS / moe::kWave;  // logits held per lane
constexpr int kMaxK = moe::kWave;                             // one selected expert per lane

// Order key of a logit: larger logit, larger key; -0.0 equals +0.0; NaN has
// key 0, below every number (whose keys are at least 0x007FFFFF).
__device__ __forceinline__ uint32_t rank_key(float x) {
    if (x != x) return 0u;
    const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int PER>  // logits held per lane: E <= 64 * PER
__global__ __launch_bounds__(kThreads) void k_route(const float *__restrict__ logits, int T, int E, int k,
                                                    int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (kThreads / moe::kWave) + (threadIdx.x >> 6);
    if (t >= T) return;  // the whole wavefront
    const float *row = logits + (size_t)t * E;

    uint32_t key[PER];
    float val[PER];
    uint32_t taken = 0;  // bit i: candidate lane + 64 i selected already, or beyond E
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + moe::kWave * i;
        if (e < E) {
            val[i] = row[e];
            key[i] = rank_key(val[i]);
        } else {
            val[i] = 0.f;
            key[i] = 0u;
            taken |= 1u << i;
        }
    }

    float mine = 0.f;  // logit selected in round `lane`
    for (int r = 0; r < k; ++r) {
        // This lane's best remaining candidate (largest key, lowest id on
        // equal keys: candidates are visited in ascending id); "none" has id
        // 0xffffffff, so it loses to any candidate, NaN ones included.
        uint32_t bk = 0u, be = 0xffffffffu;
        float bv = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!((taken >> i) & 1u) && (key[i] > bk || be == 0xffffffffu)) {
                bk = key[i];
                be = (uint32_t)(lane + moe::kWave * i);
                bv = val[i];
            }
        }
        // Wave-wide winner: the largest key, then the lowest id holding it.
        const uint32_t mk = moe::wave_max_u32(bk);
        const uint32_t me = moe::wave_min_u32(bk == mk ? be : 0xffffffffu);
        const float mv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), me & 63));
        if ((int)(me & 63) == lane) taken |= 1u << (me >> 6);
        if (lane == r) mine = mv;
        if (lane == 0) ids[(size_t)t * k + r] = (int32_t)me;
    }

    // Renormalised softmax over the k selected (round 0 holds the largest).
    const float lmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mine)));
    const float ex = lane < k ? expf(mine - lmax) : 0.f;
    float sum = ex;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
    if (lane < k) w[(size_t)t * k + lane] = ex / sum;
}

}  // namespace

extern "C" int moe_nvfp4_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                               float *topk_weights, void *stream) {
    if (!logits || !topk_ids || !topk_weights) return MOE_NVFP4_ENULL;
    if (T < 1 || E < 1 || k < 1 || k > E) return MOE_NVFP4_ESHAPE;
    if (E > MOE_NVFP4_MAX_EXPERTS || k > kMaxK || (int64_t)T * k > MOE_NVFP4_MAX_PAIRS) return MOE_NVFP4_ELIMIT;
    const int per_block = kThreads / moe::kWave;
    const unsigned grid = (unsigned)((T + per_block - 1) / per_block);
    const hipStream_t st = (hipStream_t)stream;
    if (E <= 64)
        hipLaunchKernelGGL(k_route<1>, dim3(grid), dim3(kThreads), 0, st, logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 128)
        hipLaunchKernelGGL(k_route<2>, dim3(grid), dim3(kThreads), 0, st, logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 256)
        hipLaunchKernelGGL(k_route<4>, dim3(grid), dim3(kThreads), 0, st, logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 512)
        hipLaunchKernelGGL(k_route<8>, dim3(grid), dim3(kThreads), 0, st, logits, T, E, k, topk_ids, topk_weights);
    else
        hipLaunchKernelGGL(k_route<kPerLane>, dim3(grid), dim3(kThreads), 0, st, logits, T, E, k, topk_ids,
                           topk_weights);
    return moe_host::launch_status();
}
