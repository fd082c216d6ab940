// Router ahead of the path: for each token, the k experts with the largest
// logits and their softmax weights renormalised over those k.  The pages show
// only the router's logit GEMM (prefill_weights.rs, doc of dense_gemm_prefill:
// the gate GEMM); the selection and weights are the routing the workloads are
// defined by, and the output feeds moe_nvfp4_sort and moe_nvfp4_blend.
//
// One wavefront per token: each lane holds up to 16 of the E logits (expert
// lane + 64 i) as order keys; k rounds of a wave-wide argmax (larger key
// first, then lower expert id) pick the experts in descending order.  The
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

__global__ __launch_bounds__(kThreads) void k_route(const float *__restrict__ logits, int T, int E, int k,
                                                    int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (kThreads / moe::kWave) + (threadIdx.x >> 6);
    if (t >= T) return;  // the whole wavefront
    const float *row = logits + (size_t)t * E;

    uint32_t key[kPerLane];
    float val[kPerLane];
    uint32_t taken = 0;  // bit i: candidate lane + 64 i selected already, or beyond E
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
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
        // This lane's best remaining candidate; "none" is (0, INT_MAX), below
        // a NaN candidate (0, e).  Candidates are visited in ascending id, so
        // a strict comparison keeps the lower id on equal keys.
        uint32_t bk = 0u;
        int be = 0x7fffffff;
        float bv = 0.f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane + moe::kWave * i;
            if (!((taken >> i) & 1u) && (key[i] > bk || be == 0x7fffffff)) {
                bk = key[i];
                be = e;
                bv = val[i];
            }
        }
        // Wave-wide argmax over (key descending, id ascending): a total order,
        // so every lane ends with the same winner.
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t ok = __shfl_xor(bk, d, 64);
            const int oe = __shfl_xor(be, d, 64);
            const float ov = __shfl_xor(bv, d, 64);
            if (ok > bk || (ok == bk && oe < be)) {
                bk = ok;
                be = oe;
                bv = ov;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == r) mine = bv;
        if (lane == 0) ids[(size_t)t * k + r] = be;
    }

    // Renormalised softmax over the k selected (round 0 holds the largest).
    const float lmax = __shfl(mine, 0, 64);
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
    hipLaunchKernelGGL(k_route, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, logits, T, E, k, topk_ids,
                       topk_weights);
    return moe_host::launch_status();
}
