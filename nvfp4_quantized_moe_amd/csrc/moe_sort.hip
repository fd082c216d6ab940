// Routing sort: group the T*k routed (token, expert) pairs by expert.
//
// nvfp4_moe_grouped.rs, module doc: the grouped decode lays rows out grouped
// by expert, lists the active experts, and indexes intermediates by sorted
// position.  Here the order inside an expert is the flat pair index, so the
// result is unique; the kernel is a stable counting sort in one workgroup:
//   pass 1  each wave counts the ids of its contiguous slice of pairs into its
//           own LDS histogram (order-free atomics);
//   scan    per-expert totals -> exclusive offsets; each wave's running base
//           per expert = offset + counts of the waves before it;
//   pass 2  each wave re-walks its slice 64 pairs at a time; a pair's rank
//           among equal ids in the same 64 is found with ballots, so ranks
//           follow the flat index; the last lane of each id advances the base.
// No global atomics touch the ordering, so the output is deterministic.
// Lanes holding equal ids are found by one ballot per bit of the id
// (ceil(log2 E) ballots per 64 pairs, whatever the number of distinct ids).
#include "moe_common.hpp"

namespace {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / moe::kWave;
constexpr int kIdsPerLane = 8;

// Exclusive scan of one int per thread over the whole 1024-thread block.
__device__ int block_exclusive_scan(int v, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kSortWaves ? wave_tot[lane] : 0;
        int wi = w;
#pragma unroll
        for (int d = 1; d < kSortWaves; d <<= 1) {
            int o = __shfl_up(wi, d, 64);
            if (lane >= d) wi += o;
        }
        if (lane < kSortWaves) wave_tot[kSortWaves + lane] = wi - w;  // exclusive wave base
        if (lane == kSortWaves - 1) *total = wi;
    }
    __syncthreads();
    int r = wave_tot[kSortWaves + wave] + incl - v;
    __syncthreads();  // wave_tot is reused by the next scan
    return r;
}

__global__ __launch_bounds__(kSortThreads) void k_moe_sort(
    const int32_t *__restrict__ ids, int P, int k, int E, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_tok, int32_t *__restrict__ pair_pos, int32_t *__restrict__ active,
    int32_t *__restrict__ active_count, uint32_t *__restrict__ err_flag) {
    extern __shared__ int cnt[];  // [kSortWaves][E]
    __shared__ int wave_tot[2 * kSortWaves];
    __shared__ int s_total, s_nact;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kSortWaves * E; i += kSortThreads) cnt[i] = 0;
    __syncthreads();

    const int per_wave = ((P + kSortWaves * 64 - 1) / (kSortWaves * 64)) * 64;
    const int f0 = wave * per_wave;
    const int f1 = min(P, f0 + per_wave);
    int *my = cnt + wave * E;

    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const unsigned long long lt = (1ull << lane) - 1ull;
    // The slice is read kIdsPerLane chunks of 64 at a time, all loads of a
    // group issued together; a slice of one group stays in registers for
    // pass 2.
    const int ngroups = (f1 - f0 + 64 * kIdsPerLane - 1) / (64 * kIdsPerLane);
    int ev[kIdsPerLane];
    auto load_group = [&](int g) {
#pragma unroll
        for (int j = 0; j < kIdsPerLane; ++j) {
            const int f = f0 + 64 * (kIdsPerLane * g + j) + lane;
            ev[j] = f < f1 ? ids[f] : -1;
        }
    };
    bool bad = false;
    for (int g = 0; g < ngroups; ++g) {
        load_group(g);
#pragma unroll
        for (int j = 0; j < kIdsPerLane; ++j) {
            const int f = f0 + 64 * (kIdsPerLane * g + j) + lane;
            if (f - lane >= f1) break;  // uniform: past the slice
            const int e = ev[j];
            const bool valid = f < f1 && e >= 0 && e < E;
            bad |= f < f1 && !valid;
            // The first lane of each id adds the group's count.
            const unsigned long long eq = moe::match_lanes(e, valid, nbits);
            if (valid && (eq & lt) == 0ull) my[e] += __popcll(eq);
        }
    }
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(err_flag, MOE_NVFP4_FLAG_BAD_EXPERT_ID);
    __syncthreads();

    // Per-expert totals (E <= kSortThreads, one expert per thread).
    int tot = 0;
    if (tid < E)
        for (int w = 0; w < kSortWaves; ++w) tot += cnt[w * E + tid];
    int off = block_exclusive_scan(tot, wave_tot, &s_total);
    if (tid < E) {
        offsets[tid] = off;
        int run = off;
        for (int w = 0; w < kSortWaves; ++w) {
            int c = cnt[w * E + tid];
            cnt[w * E + tid] = run;
            run += c;
        }
    }
    const int flag = (tid < E && tot > 0) ? 1 : 0;
    int aidx = block_exclusive_scan(flag, wave_tot, &s_nact);
    const int total = s_total, nact = s_nact;
    if (tid == 0) {
        offsets[E] = total;
        *active_count = nact;
    }
    if (tid < E) {
        if (flag) active[aidx] = tid;
        if (tid >= nact) active[tid] = -1;
    }
    __syncthreads();

    // Pass 2: stable positions.
    for (int g = 0; g < ngroups; ++g) {
        if (ngroups > 1) load_group(g);
#pragma unroll
        for (int j = 0; j < kIdsPerLane; ++j) {
            const int f = f0 + 64 * (kIdsPerLane * g + j) + lane;
            if (f - lane >= f1) break;  // uniform: past the slice
            const bool in = f < f1;
            const int e = ev[j];
            const bool valid = in && e >= 0 && e < E;
            const unsigned long long eq = moe::match_lanes(e, valid, nbits);
            const int rank = __popcll(eq & lt), same = __popcll(eq);
            int pos = -1;
            if (valid) pos = my[e] + rank;
            // All lanes of this wave have read their base before any lane
            // writes it (LDS operations of one wave complete in order).
            if (valid && rank == same - 1) my[e] = pos + 1;
            if (in) {
                pair_pos[f] = pos;
                if (valid) sorted_tok[pos] = f / k;
            }
        }
    }
    for (int p = total + tid; p < P; p += kSortThreads) sorted_tok[p] = -1;
}

// Few pairs (P <= 256): one pair per thread, an LDS histogram of all pairs
// and one per wave, no second read of the ids.  A pair's position is its
// expert's offset, plus the pairs of its id in earlier waves, plus those in
// earlier lanes of its own wave.  Same results as k_moe_sort.
constexpr int kSmallThreads = 256;
constexpr int kSmallPairs = moe::kBlockSortPairs;
constexpr int kSmallWaves = kSmallThreads / 64;

__global__ __launch_bounds__(kSmallThreads) void k_moe_sort_small(
    const int32_t *__restrict__ ids, int P, int k, int E, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_tok, int32_t *__restrict__ pair_pos, int32_t *__restrict__ active,
    int32_t *__restrict__ active_count, uint32_t *__restrict__ err_flag) {
    __shared__ int offs[MOE_NVFP4_MAX_EXPERTS + 1];
    __shared__ int cntw[kSmallWaves * MOE_NVFP4_MAX_EXPERTS];  // per-wave histograms
    __shared__ int act[MOE_NVFP4_MAX_EXPERTS];
    __shared__ int stok[kSmallPairs];
    const moe::SortOutputs out{offsets, sorted_tok, pair_pos, active, active_count, err_flag};
    moe::block_sort_256(ids, P, k, E, offs, cntw, act, stok, out, true);
}

}  // namespace

// The sort launch itself (arguments already checked).
int moe_launch_sort(const int32_t *topk_ids, int T, int k, int E, int32_t *expert_offsets,
                    int32_t *sorted_token_ids, int32_t *pair_pos, int32_t *active_experts, int32_t *active_count,
                    uint32_t *err_flag, hipStream_t stream) {
    const int P = T * k;
    if (P <= kSmallPairs) {
        hipLaunchKernelGGL(k_moe_sort_small, dim3(1), dim3(kSmallThreads), 0, stream, topk_ids, P, k, E,
                           expert_offsets, sorted_token_ids, pair_pos, active_experts, active_count, err_flag);
        return moe_host::launch_status();
    }
    const size_t lds = (size_t)kSortWaves * E * sizeof(int);
    hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(kSortThreads), lds, stream, topk_ids, P, k, E, expert_offsets,
                       sorted_token_ids, pair_pos, active_experts, active_count, err_flag);
    return moe_host::launch_status();
}

extern "C" int moe_nvfp4_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                              int32_t *expert_offsets, int32_t *sorted_token_ids, int32_t *pair_pos,
                              int32_t *active_experts, int32_t *active_count, uint32_t *err_flag,
                              void *stream) {
    if (!topk_ids || !expert_offsets || !sorted_token_ids || !pair_pos || !active_experts ||
        !active_count || !err_flag)
        return MOE_NVFP4_ENULL;
    if (T < 1 || k < 1 || E < 1 || k > E) return MOE_NVFP4_ESHAPE;
    if (E > MOE_NVFP4_MAX_EXPERTS || (int64_t)T * k > MOE_NVFP4_MAX_PAIRS) return MOE_NVFP4_ELIMIT;
    return moe_launch_sort(topk_ids, T, k, E, expert_offsets, sorted_token_ids, pair_pos, active_experts,
                           active_count, err_flag, (hipStream_t)stream);
}

extern "C" int moe_nvfp4_abi_version(void) { return MOE_NVFP4_ABI_VERSION; }
