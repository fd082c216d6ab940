// Shared device helpers and host argument checks for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Format decode.  gfx950's scaled converters apply only the exponent of the
// f32 scale operand, so they are called with 1.0 and the E4M3 block scale is
// applied separately.  Both conversions are exact: every E2M1 value is a
// bf16/fp16 number and the OCP E4M3 codes convert exactly to f32.
// ---------------------------------------------------------------------------

// Byte B of w holds two E2M1 codes; low nibble -> .x (even k), high -> .y.
template <int B>
__device__ __forceinline__ bf16x2_t e2m1x2_bf16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f16x2_t e2m1x2_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}
// Byte B of w as an E4M3 (OCP FN) code, widened to f32.
template <int B>
__device__ __forceinline__ float e4m3_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(w, B);
}

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Loads through pointers known to be in global memory.  Pointers read from a
// table (the per-expert weight pointers) are generic to the compiler, which
// would otherwise emit flat loads; those count against both the vector-memory
// and the LDS counters and force conservative waits.
// (HIP's uint4/float4 are structs whose copies go through a generic memcpy,
// so 16-byte values move as a native 4 x u32 vector.)
#define MOE_GLOBAL __attribute__((address_space(1)))
#define MOE_LDS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
template <typename T>
__device__ __forceinline__ T gload(const void *p) {
    if constexpr (sizeof(T) == 16) {
        const u32x4_t v = *(const MOE_GLOBAL u32x4_t *)p;
        T t;
        __builtin_memcpy(&t, &v, 16);
        return t;
    } else if constexpr (sizeof(T) == 8) {
        const u32x2_t v = *(const MOE_GLOBAL u32x2_t *)p;
        T t;
        __builtin_memcpy(&t, &v, 8);
        return t;
    } else {
        return *(const MOE_GLOBAL T *)p;
    }
}

// 16-byte load with the nontemporal hint, for weight bytes that are streamed
// once: they then do not displace reused data (activations, weights that a
// later pass reads again) from the caches.
template <typename T>
__device__ __forceinline__ T gload_nt(const void *p) {
    static_assert(sizeof(T) == 16, "16-byte loads only");
    const u32x4_t v = __builtin_nontemporal_load((const MOE_GLOBAL u32x4_t *)p);
    T t;
    __builtin_memcpy(&t, &v, 16);
    return t;
}

// Index of this wavefront in the block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
    static_assert(sizeof(T) == sizeof(U), "size");
    T t;
    __builtin_memcpy(&t, &u, sizeof(T));
    return t;
}

// ---------------------------------------------------------------------------
// Cross-lane sums with DPP (within 16-lane rows).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes

// Sum over aligned groups of L lanes (L in {1,2,4,8,16}); every lane of the
// group receives the group total.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 2) v += dpp<kDppXor1>(v);
    if constexpr (L >= 4) v += dpp<kDppXor2>(v);
    if constexpr (L >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (L >= 16) v += dpp<kDppMirror>(v);
    return v;
}

// Wave-wide extrema of a 32-bit unsigned value: DPP within each 16-lane row
// (every lane of a row reads a valid source in these patterns), then the
// four row results through readlane, so the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_u32<kDppXor1>(v));
    v = min(v, dpp_u32<kDppXor2>(v));
    v = min(v, dpp_u32<kDppHalfMirror>(v));
    v = min(v, dpp_u32<kDppMirror>(v));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return min(min(a, b), min(c, d));
}

// Mask of the lanes whose id equals this lane's (among lanes with valid set),
// from one ballot per id bit.
__device__ __forceinline__ unsigned long long match_lanes(int e, bool valid, int nbits) {
    unsigned long long eq = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long m = __ballot(valid && bit);
        eq &= bit ? m : ~m;
    }
    return eq;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt in bits 3:0 and 15:14; the LDS/scalar and
// export counters left at their maxima, i.e. not waited for).  Loads count
// down in issue order, so this waits for every load but the newest n.
constexpr int waitcnt_vm(int n) { return (((n >> 4) & 3) << 14) | 0x0F70 | (n & 15); }

// Workgroup barrier that waits for this wave's LDS operations only.  Direct
// global-to-LDS loads count as vector-memory operations: a wave waits for its
// own (waitcnt_vm) before the barrier that publishes them.  The asm fences
// keep memory operations on their side.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float silu_f32(float z) {
    return z / (1.0f + __expf(-z));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Routing sort of P <= 256 pairs by one 256-thread block, in LDS: one pair per
// thread; an LDS histogram of all pairs and one per wave; a pair's sorted
// position is its expert's offset, plus the pairs of its id in earlier
// waves, plus those in earlier lanes of its own wave (so positions follow the
// flat pair index and the result is unique).  LDS (caller's): offs[E + 1]
// (on return the exclusive offsets, offs[E] = valid pairs), cntw[4 * E],
// act[E] (on return the active experts ascending), stok[P] (on return the
// token of each sorted position below offs[E]).  Returns the active count.
// With `wr` set, also writes every output of moe_nvfp4_sort to memory.  (The
// outputs come by value with a flag, not as a pointer that may be null: a
// select between the address of a local and null kept the struct on the
// stack, a private-memory write by every lane of every block.)  Ends with a
// barrier.
struct SortOutputs {
    int32_t *offsets, *sorted_tok, *pair_pos, *active, *active_count;
    uint32_t *err_flag;
};
constexpr int kBlockSortPairs = 256;
__device__ __forceinline__ int block_sort_256(const int32_t *ids, int P, int k, int E, int *offs, int *cntw,
                                              int *act, int *stok, const SortOutputs out, const bool wr) {
    __shared__ int wsum[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = tid < P ? ids[tid] : -1;
    const bool valid = tid < P && e >= 0 && e < E;
    for (int i = tid; i < E; i += 256) {
        offs[i] = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) cntw[w * E + i] = 0;
    }
    if (wr && __ballot(tid < P && !valid) != 0ull && lane == 0)
        atomicOr(out.err_flag, MOE_NVFP4_FLAG_BAD_EXPERT_ID);
    __syncthreads();
    if (valid) {
        atomicAdd(&offs[e], 1);
        atomicAdd(&cntw[wave * E + e], 1);
    }
    __syncthreads();

    // Exclusive scans over the experts (4 consecutive per thread) of the
    // counts and of the active flags.
    int c[4], s0 = 0, s1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ex = 4 * tid + i;
        c[i] = ex < E ? offs[ex] : 0;
        s0 += c[i];
        s1 += c[i] > 0 ? 1 : 0;
    }
    int i0 = s0, i1 = s1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o0 = __shfl_up(i0, d, 64), o1 = __shfl_up(i1, d, 64);
        if (lane >= d) {
            i0 += o0;
            i1 += o1;
        }
    }
    if (lane == 63) {
        wsum[0][wave] = i0;
        wsum[1][wave] = i1;
    }
    __syncthreads();
    int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (w < wave) {
            b0 += wsum[0][w];
            b1 += wsum[1][w];
        }
        t0 += wsum[0][w];
        t1 += wsum[1][w];
    }
    int off = b0 + i0 - s0, aidx = b1 + i1 - s1;
    __syncthreads();  // every count is read before the offsets replace them
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ex = 4 * tid + i;
        if (ex < E) {
            offs[ex] = off;
            if (c[i] > 0) act[aidx] = ex;
            if (wr) {
                out.offsets[ex] = off;
                if (c[i] > 0) out.active[aidx] = ex;
                if (ex >= t1) out.active[ex] = -1;
            }
            aidx += c[i] > 0 ? 1 : 0;
        }
        off += c[i];
    }
    if (tid == 0) {
        offs[E] = t0;
        if (wr) {
            out.offsets[E] = t0;
            *out.active_count = t1;
        }
    }
    __syncthreads();

    if (wave * 64 < P) {
        const unsigned long long lt = (1ull << lane) - 1ull;
        int rank = __popcll(match_lanes(e, valid, E > 1 ? 32 - __clz(E - 1) : 0) & lt);
        if (valid)
            for (int w = 0; w < wave; ++w) rank += cntw[w * E + e];
        if (tid < P) {
            const int pos = valid ? offs[e] + rank : -1;
            if (valid) stok[pos] = tid / k;
            if (wr) {
                out.pair_pos[tid] = pos;
                if (valid) out.sorted_tok[pos] = tid / k;
            }
        }
    }
    if (wr)
        for (int q = t0 + tid; q < P; q += 256) out.sorted_tok[q] = -1;
    __syncthreads();
    return t1;
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Host-side helpers.
// ---------------------------------------------------------------------------
// Routing-sort arguments handed to a gate+up launch that may run the sort
// itself (moe_nvfp4_sort_gate_up_silu).
struct MoeSortFuse {
    const int32_t *topk_ids;
    int k;
    int32_t *offsets, *sorted_tok, *pair_pos, *active, *active_count;
    uint32_t *err_flag;
};

namespace moe_host {

inline bool experts_null(const moe_nvfp4_experts &w) {
    return w.packed == nullptr || w.scale == nullptr || w.scale2 == nullptr;
}

// Compute units of the current device (cached per device).
inline int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_NVFP4_OK : (int)e;
}

}  // namespace moe_host
