// Decode path: grouped NVFP4 projection over row-major weights (packed
// [N, K/2], scales [N, K/16]) for the few tokens routed to each expert.
//
// Grouped NVFP4 MoE decode kernels (moe_expert_gate_up_act_nvfp4_grouped and
// moe_expert_down_act_nvfp4_grouped): one block row per active-expert slot
// (grid y = cap = min(E, P)); blocks past the device-side active count exit;
// gate+up fuse the SiLU product into fp32 h[position, n]; down reads h and
// writes fp32 y[position, n].
//
// gfx950 mapping.  The projection is bound by streaming the expert weights
// from HBM, so the kernel is laid out around one rule: in the steady state
// the only global loads are the weight stream itself, each instruction
// covering 4 rows x 256 contiguous bytes, plus one 16-byte-per-lane load of
// the matching E4M3 scales every four steps.  Everything else a step needs
// comes from LDS.
//
//   * Work split.  The weight rows of an expert are cut into units of 32 rows
//     (gate+up: 16 output columns of each matrix; down: 32 output columns); a
//     block streams G consecutive units (G from the shape on the host).  Wave
//     w of the block owns 8 rows of every unit, as two groups of 4 (gate+up:
//     the gate rows and the up rows of the same 4 columns), over the whole K
//     axis, so no partial sums cross waves.
//   * Ring.  A wave walks its rows segment by segment (512 k = 256 bytes per
//     row): per segment ("step"), two 16-byte loads per lane, one per row
//     group.  Steps flow through a register ring of depth D that is refilled
//     without any branch around the loads and in a pinned issue order, so the
//     waits on it stay partial and the ring runs on across unit boundaries.
//     Steps past the end of the stream repeat the last real address (a cache
//     hit) and contribute nothing; lanes of a ragged last segment read a
//     valid chunk of the same row and contribute zero.
//   * Scales.  Every fourth step also loads the scale slices of the next four
//     steps, 16 bytes per lane (8 rows x 4 steps x 32 bytes), into a 1 KiB
//     LDS area of the wave; each step reads its two scale bytes per lane from
//     there.
//   * Matrix cores.  16x16x32 fp16 MFMA.  Lane (n, q) (n = lane & 15, q =
//     lane >> 4) holds 16 bytes of row n >> 2 at byte 64q + 16(n & 3) of the
//     segment: each B column is one (row, quarter) pair, so an instruction
//     reads 256 contiguous bytes per row.  The A rows are (token, quarter)
//     pairs, 4 tokens per MFMA, fed with the activation at the same k.  Only
//     the blocks where the two quarters agree are kept, and the 4 quarters are
//     summed across a quad of lanes at the end of the unit.  The E2M1 codes
//     are widened to fp16 pairs and multiplied by the E4M3 scale in fp16
//     (exact: at most 6 significant bits, range 2^-10 .. 2688).  This layout
//     serves passes of up to 4 routed rows (one MFMA token group); longer
//     passes, up to 16 rows sharing each decoded weight, take the
//     token-dense form (run_pass_dense): 16 rows x 64 bytes per load, one
//     weight row per B column, all 16 rows of the pass in one MFMA.  Experts
//     with more rows than the staged activation holds take further passes.
//   * Routing sort fused in (k_decode_row<true, true>): with few pairs, every
//     wave ranks them itself and block (0, 0) writes the sort outputs.
//   * Activations.  LDS holds the pass's activation rows (x rows for gate+up,
//     h rows for down) as fp16, each row scaled by a power of two that brings
//     its largest magnitude into [2^14, 2^15): x (bf16) is then exact for
//     every element down to 2^-29 of the row maximum and h keeps 11
//     significant bits, whatever the row's range.  The factor is undone in
//     the epilogue.  The row stride is padded so the A-operand reads are free
//     of bank conflicts.
#include "moe_common.hpp"

#include <algorithm>
#include <type_traits>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / moe::kWave;
constexpr int kDepth = 4;          // ring: steps in flight per wave (a multiple of kGroup)
constexpr int kGroup = 4;          // steps per scale load
constexpr int kSegBytes = 256;     // bytes of one weight row per step (512 k)
constexpr int kMaxTG = 4;          // token groups of 4 per pass (16 rows, token-dense above 4)
constexpr int kLdsBudget = 72 * 1024;  // staged activation rows per block (two blocks per CU)
constexpr int kScaleLds = 1024;        // per wave: 4 steps x 8 rows x 32 bytes
constexpr int kPreLds = 4 * (MOE_NVFP4_MAX_EXPERTS + 4);  // per-slot prefix sums of passes (or the fused sort)
constexpr int kRmaxOff = kWaves * kScaleLds;                    // per-row maxima (16 x u32)
constexpr int kTokOff = kRmaxOff + 64;                          // tokens of the pass's rows (16 x i32)
constexpr int kPreOff = kTokOff + 64;
constexpr int kHdrLds = kPreOff + kPreLds;  // scale areas + row maxima + pass prefix; then the rows
constexpr int kRingFillLoads = 2 * kDepth + kDepth / kGroup;  // vector-memory loads that fill the ring

using moe::u32x2_t;
using moe::u32x4_t;
// sched_barrier mask: ALU, VALU, SALU, MFMA, LDS and transcendental
// instructions may be scheduled across; global memory instructions may not.
constexpr int kMoveAcrossLoads = 0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0080 | 0x0400;

struct DecArgs {
    const void *act;            // gate+up: bf16 x [T, K]; down: fp32 h [P, K]
    const int32_t *sorted_tok;  // gate+up only
    const int32_t *offsets;
    const int32_t *active;
    const int32_t *nactive;
    const uint8_t *const *pa;   // gate (or down)
    const uint8_t *const *sa;
    const float *s2a;
    const uint8_t *const *pb;   // up (gate+up only)
    const uint8_t *const *sb;
    const float *s2b;
    float *out;                 // [P, N]
    int N, K;
    int G;                      // units per block
    int units;                  // units along N
    int pass_rows;              // activation rows staged per pass
    int ldx;                    // staged row stride, fp16 elements
    int extra;                  // block rows for passes beyond each expert's first
    int single_token;           // gate+up with T == 1: every routed row is token 0
    int nt_min_active;          // nontemporal weight loads from this many active experts on
    int cap;                    // active-slot capacity, min(E, P)
    // Routing sort fused into the gate+up launch (few pairs, one pass per
    // expert): the routed ids, and the sort outputs that block (0, 0) writes.
    int fused_sort;
    int P, topk, E;
    const int32_t *topk_ids;
    int32_t *sort_offsets, *sort_tok, *sort_pos, *sort_active, *sort_count;
    uint32_t *err_flag;
    // Down projection with the blend fused in (k_decode_down_blend): the
    // routing weights, each pair's sorted position, and the bf16 output.
    const float *blend_w;
    const int32_t *blend_pos;
    uint16_t *blend_out;
};

// The fused sort's tables, in the LDS area the pass prefix would otherwise
// use: the token of every sorted position, and (for the block that writes
// the sort outputs) the active experts in ascending order with, for each,
// the number of routed pairs with a smaller id (its first sorted position).
constexpr int kSortPairs = 64;
struct SortLds {
    int active[kSortPairs];
    int lo[kSortPairs];
    int tok[kSortPairs];
};

// 8 E2M1 codes (one 32-bit word: k .. k+7) times the block scale, as fp16.
__device__ __forceinline__ f16x8_t decode_b(uint32_t w, f16x2_t s) {
    const f16x2_t v0 = moe::e2m1x2_f16<0>(w) * s, v1 = moe::e2m1x2_f16<1>(w) * s;
    const f16x2_t v2 = moe::e2m1x2_f16<2>(w) * s, v3 = moe::e2m1x2_f16<3>(w) * s;
    f16x8_t r;
    r[0] = v0.x;
    r[1] = v0.y;
    r[2] = v1.x;
    r[3] = v1.y;
    r[4] = v2.x;
    r[5] = v2.y;
    r[6] = v3.x;
    r[7] = v3.y;
    return r;
}

__device__ __forceinline__ float pick(const f32x4_t &v, int i) {
    float r = v[0];
    r = i == 1 ? v[1] : r;
    r = i == 2 ? v[2] : r;
    r = i == 3 ? v[3] : r;
    return r;
}

// A 16-byte weight load; NT: the nontemporal hint.  It is used when the
// launch streams more expert weights than the 256 MB Infinity Cache holds
// (caching them cannot pay off), only for experts read by one pass (a later
// pass finds the weights of a busy expert in the cache), and only in the
// (row, quarter) pass: 64 tokens x 256 experts (3.7 GB of gate+up weights)
// ran 8% faster in gate+up and 5% in down so, while the hint in the
// token-dense pass as well gave back most of the gate+up gain, and 32 tokens
// (170 MB) ran 4-6% slower with it, hence the size bound.
template <bool NT>
__device__ __forceinline__ u32x4_t wload(const void *p) {
    if constexpr (NT)
        return moe::gload_nt<u32x4_t>(p);
    else
        return moe::gload<u32x4_t>(p);
}

// Power-of-two exponent e that brings a row maximum (bits of a non-negative
// float) into [2^14, 2^15) after scaling by 2^-e; 0 for zero, inf or NaN.
__device__ __forceinline__ int row_exp(uint32_t mbits) {
    const int ef = (int)(mbits >> 23);
    if (mbits == 0u || ef >= 255) return 0;
    const int e = (ef == 0 ? -126 : ef - 127) - 14;
    return e < -126 ? -126 : (e > 126 ? 126 : e);
}
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// Largest magnitude of 8 bf16 values, as two 16-bit halves: with the sign
// bit cleared, bf16 bits order as their magnitudes do (NaN above inf).
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;
__device__ __forceinline__ u16x2_t absmax8_bf16(uint4 v) {
    auto m = [](uint32_t u) { return __builtin_bit_cast(u16x2_t, u & 0x7fff7fffu); };
    return __builtin_elementwise_max(__builtin_elementwise_max(m(v.x), m(v.y)),
                                     __builtin_elementwise_max(m(v.z), m(v.w)));
}

__device__ __forceinline__ float absmax8f(const f32x4_t &a, const f32x4_t &b) {
    const float u = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3])));
    const float v = fmaxf(fmaxf(fabsf(b[0]), fabsf(b[1])), fmaxf(fabsf(b[2]), fabsf(b[3])));
    return fmaxf(u, v);
}

// 8 fp32 values times f -> fp16, written as one 16-byte LDS chunk.
__device__ __forceinline__ void put_f16x8(uint16_t *dst, const f32x4_t &a, const f32x4_t &b, float f) {
    f16x8_t h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = (_Float16)(a[j] * f);
        h[4 + j] = (_Float16)(b[j] * f);
    }
    *reinterpret_cast<f16x8_t *>(dst) = h;
}

// Row maxima with 2^lgt threads per row (lgt >= 2): the groups are
// aligned runs of lanes, so a row's threads share a wave (up to 16 lanes)
// or span whole 16-lane runs.  v is a non-negative float's bits; each run's
// first lane merges the run's maximum into rmax[m] (rows m < pr only).
__device__ __forceinline__ uint32_t threads_per_row_log2(int rows) {  // rows <= 64: 2^lgt >= 4
    return rows <= 1 ? 8u : 8u - (32u - (uint32_t)__builtin_clz((uint32_t)(rows - 1)));
}
__device__ __forceinline__ void row_group_max(uint32_t *rmax, int m, bool in, uint32_t v, int lgt) {
    const int lane = threadIdx.x & 63;
    v = max(v, moe::dpp_u32<moe::kDppXor1>(v));
    v = max(v, moe::dpp_u32<moe::kDppXor2>(v));
    if (lgt >= 3) v = max(v, moe::dpp_u32<moe::kDppHalfMirror>(v));
    if (lgt >= 4) v = max(v, moe::dpp_u32<moe::kDppMirror>(v));
    const int run = lgt >= 4 ? 15 : (1 << lgt) - 1;
    if (in && (lane & run) == 0) atomicMax(rmax + m, v);
}

// Stage rows [row0, row0 + pr) of the activation into LDS as fp16 (stride
// ldx), row m scaled by 2^-e(m) where e(m) comes from the row's largest
// magnitude (kept in rmax[m] as float bits; rmax is zero on entry).  Gate+up
// gathers x rows by token (row m's token in ptok[m], LDS); down reads h rows
// in order, or (GATHER) row gpos[m] for row m.
// mid() issues the weight ring: gate+up after every x load (mid() must issue
// exactly kRingFillLoads loads); down once the first h loads are in flight
// (rows read in one batch) or once the maxima are known and the first two
// conversion batches are in flight (rows read in several).
// Ends with the rows visible to the whole block.
template <bool GATED, bool GATHER = false, typename Mid>
__device__ __forceinline__ void stage(const DecArgs &a, int row0, int pr, const int *ptok, uint16_t *xs,
                                      uint32_t *rmax, Mid &&mid, const int *gpos = nullptr) {
    const int K = a.K, ldx = a.ldx;
    auto hrow = [&](int m) -> size_t { return GATHER ? (size_t)gpos[m] : (size_t)(row0 + m); };
    const int cpr = K >> 3;  // 8-element chunks per row
    constexpr int SB = 4;  // h: chunks per thread per batch
    // pr <= 64 rows.  No load sits behind a branch, so none is left in
    // flight on any path.
    if constexpr (GATED) {
        // x rows (bf16 bytes) straight into their LDS slots by direct loads,
        // issued ahead of the weight ring (mid()): loads complete in issue
        // order, so waiting for x then waits for no weight load.  One 16-byte
        // slot per lane, 64 consecutive slots of one padded row per
        // instruction (a pad slot loads its row's first chunk, never read).
        // The (row, 64-slot group) items go round-robin over the waves; each
        // wave holds the pass's tokens in one register (lane r: row r,
        // pr <= 16) and picks an item's token with a lane read, so no item
        // waits on a memory read.
        const uint16_t *x = static_cast<const uint16_t *>(a.act);
        const int spr = ldx >> 3;          // 16-byte slots per staged row (chunks and pad)
        const int nit = (spr + 63) >> 6;   // 64-slot groups per row
        const int lane = threadIdx.x & 63, w = moe::wave_id();
        uint8_t *xb = reinterpret_cast<uint8_t *>(xs);
        const int tokv = ptok[lane & 15];
        int row = 0, i = w;  // item w: group i of row `row`
        while (i >= nit) {
            i -= nit;
            ++row;
        }
        for (; row < pr;) {
            const int tok = __builtin_amdgcn_readlane(tokv, row);
            const int kc = 64 * i + lane;
            if (kc < spr)
                __builtin_amdgcn_global_load_lds(
                    (const MOE_GLOBAL void *)(x + (size_t)tok * K + 8 * (kc < cpr ? kc : 0)),
                    (MOE_LDS void *)(xb + 16 * (row * spr + 64 * i)), 16, 0, 0);
            i += kWaves;
            while (i >= nit) {
                i -= nit;
                ++row;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        mid();
        __builtin_amdgcn_s_waitcnt(moe::waitcnt_vm(kRingFillLoads));  // this wave's x slots have landed
        moe::lds_barrier();
        // Maxima and conversion: 2^lgt threads per row, thread t on row
        // t >> lgt and every 2^lgt-th chunk of it from t mod 2^lgt.
        const int lgt = (int)threads_per_row_log2(pr);
        const int tm = (int)threadIdx.x >> lgt, tj = (int)threadIdx.x & ((1 << lgt) - 1);
        const bool rin = tm < pr;
        uint16_t *xr = xs + (rin ? tm : 0) * ldx;
        // kIlp chunks per iteration, their LDS reads issued together (a
        // chunk past the row's end reads the iteration's first again).
        constexpr int kIlp = 8;
        const int cst = 1 << lgt;
        u16x2_t mx = {0, 0};
        if (rin)
            for (int c = tj; c < cpr; c += kIlp * cst) {
                uint4 v[kIlp];
#pragma unroll
                for (int u = 0; u < kIlp; ++u) {
                    const int cc = c + u * cst;
                    v[u] = *reinterpret_cast<const uint4 *>(xr + 8 * (cc < cpr ? cc : c));
                }
#pragma unroll
                for (int u = 0; u < kIlp; ++u) mx = __builtin_elementwise_max(mx, absmax8_bf16(v[u]));
            }
        // float bits of the largest magnitude
        row_group_max(rmax, tm, rin, (uint32_t)(mx.x > mx.y ? mx.x : mx.y) << 16, lgt);
        moe::lds_barrier();  // maxima complete
        if (rin) {  // bf16 -> scaled fp16 in place, kIlp chunks per iteration
            const float f = exp2i(-row_exp(rmax[tm]));
            for (int c = tj; c < cpr; c += kIlp * cst) {
                uint4 v[kIlp];
#pragma unroll
                for (int u = 0; u < kIlp; ++u) {
                    const int cc = c + u * cst;
                    v[u] = *reinterpret_cast<const uint4 *>(xr + 8 * (cc < cpr ? cc : c));
                }
#pragma unroll
                for (int u = 0; u < kIlp; ++u) {
                    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    f16x8_t h;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        h[2 * j] = (_Float16)(bf16_lo(w4[j]) * f);
                        h[2 * j + 1] = (_Float16)(bf16_hi(w4[j]) * f);
                    }
                    if (c + u * cst < cpr) *reinterpret_cast<f16x8_t *>(xr + 8 * (c + u * cst)) = h;
                }
            }
        }
        moe::lds_barrier();
    } else {
        const float *h = static_cast<const float *>(a.act);
        // 2^lgt threads per row, thread t on row t >> lgt and its chunks
        // t mod 2^lgt + 2^lgt i.  Every thread issues the same loads (a chunk
        // past its row's end, or a thread past the last row, re-reads a valid
        // chunk that is not used), so the ring's waits stay exact.
        const int lgt = (int)threads_per_row_log2(pr);
        const int tm = (int)threadIdx.x >> lgt, tj = (int)threadIdx.x & ((1 << lgt) - 1);
        const bool rin = tm < pr;
        const float *src = h + hrow(rin ? tm : 0) * K;
        uint16_t *dst = xs + (rin ? tm : 0) * ldx;
        const int nct = (cpr + (1 << lgt) - 1) >> lgt;  // chunks per thread, at most
        auto ld = [&](int i, f32x4_t &f0, f32x4_t &f1) {
            const int c = min(tj + (i << lgt), cpr - 1);
            f0 = moe::gload<f32x4_t>(src + 8 * c);
            f1 = moe::gload<f32x4_t>(src + 8 * c + 4);
        };
        auto valid = [&](int i) { return rin && tj + (i << lgt) < cpr; };
        uint32_t mx = 0u;
        if (nct <= SB) {
            // One batch: the rows stay in registers between the two phases.
            f32x4_t f0[SB], f1[SB];
#pragma unroll
            for (int i = 0; i < SB; ++i) ld(i, f0[i], f1[i]);
            mid();
#pragma unroll
            for (int i = 0; i < SB; ++i)
                if (valid(i)) mx = max(mx, __float_as_uint(absmax8f(f0[i], f1[i])));
            row_group_max(rmax, tm, rin, mx, lgt);
            __syncthreads();  // maxima complete
            const float f = exp2i(-row_exp(rmax[rin ? tm : 0]));
#pragma unroll
            for (int i = 0; i < SB; ++i)
                if (valid(i)) put_f16x8(dst + 8 * (tj + (i << lgt)), f0[i], f1[i], f);
        } else {
            // Several batches, read once.  Each row's scale comes from the
            // largest magnitude of its threads' first batch (a lower bound on
            // the row's), doubled: the estimate lands in [2^13, 2^14), so any
            // element up to 4x it still converts to a finite fp16 number.
            // Scaling by a power of two leaves the fp16 rounding of a normal
            // number unchanged, so the staged values (and every sum over
            // them) are those of the exact row maximum's scale, up to that
            // power of two, which the epilogue undoes from rmax.  Every
            // thread tracks the largest magnitude it converts; a row with an
            // element at or past the fp16 limit at this scale (or not
            // finite), or whose estimate is zero, makes the whole block stage
            // again from exact maxima: the rows read twice, maxima first.
            // Two register sets: each batch's loads go out before the
            // previous batch is used, so the batches' round trips overlap
            // (the loads past the last batch re-read valid chunks, unused).
            // The weight ring goes out once the estimates are known: loads
            // complete in issue order, so the wait for the first batch does
            // not wait for weights.
            f32x4_t a0[SB], a1[SB], b0[SB], b1[SB];
            auto ldb = [&](int b, f32x4_t *f0, f32x4_t *f1) {
#pragma unroll
                for (int i = 0; i < SB; ++i) ld(b + i, f0[i], f1[i]);
            };
            auto mxb = [&](int b, const f32x4_t *f0, const f32x4_t *f1) {
#pragma unroll
                for (int i = 0; i < SB; ++i)
                    if (valid(b + i)) mx = max(mx, __float_as_uint(absmax8f(f0[i], f1[i])));
            };
            auto cvb = [&](int b, const f32x4_t *f0, const f32x4_t *f1, float f) {
#pragma unroll
                for (int i = 0; i < SB; ++i)
                    if (valid(b + i)) put_f16x8(dst + 8 * (tj + ((b + i) << lgt)), f0[i], f1[i], f);
            };
            // (The gathered staging of the fused down+blend launch keeps the
            // two reads: its few rows mostly take the one-batch path, and the
            // single-read code would cost it a wave per SIMD.)
            bool twice = GATHER;
            if constexpr (!GATHER) {
            ldb(0, a0, a1);
            ldb(SB, b0, b1);
            mxb(0, a0, a1);
            row_group_max(rmax, tm, rin, mx, lgt);
            __syncthreads();  // first-batch maxima complete
            const uint32_t est = rmax[rin ? tm : 0];
            __syncthreads();  // every estimate is read before the rows' scales replace them
            const uint32_t sc = est + (1u << 23);  // the estimate doubled (non-finite: row_exp gives 0)
            if (rin && tj == 0) rmax[tm] = sc;
            const int es = row_exp(sc);
            const float f = exp2i(-es);
            const uint32_t lim = __float_as_uint(65504.f * exp2i(es));  // largest magnitude that stays finite
            mid();
            for (int b = 0; b < nct; b += 2 * SB) {
                if (b > 0) mxb(b, a0, a1);  // the first batch's maximum is in mx already
                cvb(b, a0, a1, f);
                ldb(b + 2 * SB, a0, a1);
                mxb(b + SB, b0, b1);
                cvb(b + SB, b0, b1, f);
                ldb(b + 3 * SB, b0, b1);
            }
            twice = __syncthreads_or(rin && (est == 0u || mx >= lim));
            if (twice) {
                if ((int)threadIdx.x < pr) rmax[threadIdx.x] = 0u;
                __syncthreads();
                mx = 0u;
            }
            }
            if (twice) {
                ldb(0, a0, a1);
                for (int b = 0; b < nct; b += 2 * SB) {
                    ldb(b + SB, b0, b1);
                    mxb(b, a0, a1);
                    ldb(b + 2 * SB, a0, a1);
                    mxb(b + SB, b0, b1);
                }
                row_group_max(rmax, tm, rin, mx, lgt);
                __syncthreads();  // exact maxima complete
                const float fx = exp2i(-row_exp(rmax[rin ? tm : 0]));
                ldb(0, a0, a1);
                ldb(SB, b0, b1);
                if constexpr (GATHER) mid();  // (single read: the ring is out already)
                for (int b = 0; b < nct; b += 2 * SB) {
                    cvb(b, a0, a1, fx);
                    ldb(b + 2 * SB, a0, a1);
                    cvb(b + SB, b0, b1, fx);
                    ldb(b + 3 * SB, b0, b1);
                }
            }
        }
        __syncthreads();
    }
}

// One pass: rows [row0, row0 + pr) of the expert against units
// u_first + us i, i in [0, nu), of its weights (us = 1: a contiguous range).
// A pass of up to 4 rows in the (row, quarter) layout.
template <bool GATED, int D, bool TOK_LDS, bool NT>  // TOK_LDS: tokens from the fused sort's LDS table tokl
__device__ __forceinline__ void run_pass(const DecArgs &a, int row0, int pr, int u_first, int nu, int us,
                                         const uint8_t *pA, const uint8_t *sA, const uint8_t *pB,
                                         const uint8_t *sB, float s2A, float s2B, uint8_t *lds,
                                         const int *tokl) {
    static_assert(D % kGroup == 0, "ring depth");
    const int K = a.K, N = a.N, ldx = a.ldx;
    const int rowbytes = K >> 1, sbytes = K >> 4;
    const int nseg = (rowbytes + kSegBytes - 1) / kSegBytes;
    const int total = nu * nseg;
    const int lane = threadIdx.x & 63, w = moe::wave_id();
    const int n = lane & 15, q = lane >> 4;
    const int rho = n >> 2, c = n & 3;
    const int choff = 64 * q + 16 * c;  // this lane's chunk within a row segment
    // Scale-load role: step s4 of the group, row r8 of the wave, half hh of the 32-byte slice.
    const int s4 = lane >> 4, r8 = (lane >> 1) & 7, hh = lane & 1;

    uint8_t *sc_lds = lds + w * kScaleLds;
    uint32_t *rmax = reinterpret_cast<uint32_t *>(lds + kRmaxOff);
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds + kHdrLds);

    // Row bases (bytes) of this lane's two weight rows and its scale row, in unit 0.
    const uint8_t *wb0, *wb1, *sbase;
    size_t ustride, sustride;  // advance per unit
    if constexpr (GATED) {
        wb0 = pA + (size_t)(4 * w + rho) * rowbytes;
        wb1 = pB + (size_t)(4 * w + rho) * rowbytes;
        sbase = (r8 < 4 ? sA : sB) + (size_t)(4 * w + (r8 & 3)) * sbytes;
        ustride = (size_t)16 * rowbytes;
        sustride = (size_t)16 * sbytes;
    } else {
        wb0 = pA + (size_t)(8 * w + rho) * rowbytes;
        wb1 = wb0 + (size_t)4 * rowbytes;
        sbase = sA + (size_t)(8 * w + r8) * sbytes;
        ustride = (size_t)32 * rowbytes;
        sustride = (size_t)32 * sbytes;
    }

    u32x4_t w0[D], w1[D], sv[D / kGroup];
    int ssh[D / kGroup];  // dword shift of a scale slice loaded from a clamped address
    int lu = 0, li = 0;   // stream position of the next load (unit, segment)
    auto load = [&](int d) {
        if (d % kGroup == 0) {
            // Scale slice of step (lu, li) + s4 for row r8 (16 bytes, half hh).
            int l = li + s4, u = lu;
#pragma unroll
            for (int i = 0; i < kGroup - 1; ++i) {
                const bool wrap = l >= nseg;
                l = wrap ? l - nseg : l;
                u = wrap ? u + 1 : u;
            }
            const bool real = u < nu;
            u = real ? u : nu - 1;
            l = real ? l : nseg - 1;
            const int want = 32 * l + 16 * hh;
            const int got = min(want, sbytes - 16);
            ssh[d / kGroup] = (want - got) >> 2;
            sv[d / kGroup] = moe::gload<u32x4_t>(sbase + (size_t)(u_first + us * u) * sustride + got);
        }
        const bool real = lu < nu;  // past the end: the last real step again
        const int unit = u_first + us * (real ? lu : nu - 1);
        const int off = min(kSegBytes * (real ? li : nseg - 1) + choff, rowbytes - 16);
        w0[d] = wload<NT>(wb0 + (size_t)unit * ustride + off);
        w1[d] = wload<NT>(wb1 + (size_t)unit * ustride + off);
        if (++li == nseg) {
            li = 0;
            ++lu;
        }
    };

    // The pass's row maxima are cleared and its tokens published in LDS
    // (read there, no load result is pending when the activation loads go
    // out).
    // The activation rows are loaded before the ring (gate+up after the
    // lookup of the pass's tokens, except with one token, whose row is x row
    // 0), so waiting for them waits for no weight; the ring then fills while
    // they are converted.
    int *ptok = reinterpret_cast<int *>(lds + kTokOff);
    if (threadIdx.x < 16) {
        rmax[threadIdx.x] = 0u;
        int tk = 0;  // one token: x row 0
        if (GATED && !a.single_token) {
            const int r = row0 + min((int)threadIdx.x, pr - 1);
            if constexpr (TOK_LDS)
                tk = tokl[r];
            else
                tk = moe::gload<int32_t>(a.sorted_tok + r);
        }
        ptok[threadIdx.x] = tk;
    }
    __syncthreads();  // rmax cleared, tokens published
    __builtin_amdgcn_sched_barrier(0);
    stage<GATED>(a, row0, pr, ptok, xs, rmax, [&]() {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(d);
            __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
        }
    });

    // One token group (pr <= 4): lane (n, q) feeds A row (token n >> 2,
    // quarter n & 3) and its output row is token q.
    const int tA = n >> 2, cA = n & 3;
    const int arow = (tA < pr ? tA : 0) * ldx;  // rows past the pass read row 0: dropped outputs
    const float oscale = exp2i(row_exp(rmax[q < pr ? q : 0]));  // undoes the row scaling of token q
    const int sread0 = 32 * rho + 8 * q + 2 * c;  // this lane's scale bytes in a step's slice (group 0)

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

    int cu = 0, ci = 0;  // stream position being computed
    // One step of the ring: compute slot d, then (refill) load the step D
    // ahead into it.  Every iteration but the last refills all of its slots,
    // so the loop body has no branch around a load; the last iteration, whose
    // refills would all lie past the end, has none.
    auto step = [&](const int d, auto refill) {
        if (d % kGroup == 0) {
            // This group's scale slices -> LDS (undoing a clamped load's shift).
            const u32x4_t v = sv[d / kGroup];
            const int s = ssh[d / kGroup];
            u32x4_t r;
            r[0] = s == 0 ? v[0] : (s == 1 ? v[1] : (s == 2 ? v[2] : v[3]));
            r[1] = s == 0 ? v[1] : (s == 1 ? v[2] : v[3]);
            r[2] = s == 0 ? v[2] : v[3];
            r[3] = v[3];
            *reinterpret_cast<u32x4_t *>(sc_lds + 16 * lane) = r;
        }
        // A fragments, read first so the LDS latency hides behind the decode.
        const int ka = 512 * ci + 128 * q + 32 * cA;  // first k of this lane's A fragment
        const int kac = ka < K ? ka : 0;              // past the end: any finite row data
        f16x8_t a0[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a0[ks] = *reinterpret_cast<const f16x8_t *>(xs + arow + kac + 8 * ks);
        const int kq = 512 * ci + 128 * q + 32 * c;  // first k of this lane's B chunk
        const bool kin = cu < nu && kq < K;
        const uint8_t *sp = sc_lds + 256 * (d % kGroup) + sread0;
        const uint32_t v0 = *reinterpret_cast<const uint16_t *>(sp);
        const uint32_t v1 = *reinterpret_cast<const uint16_t *>(sp + 128);
        const f16x2_t zero2 = {(_Float16)0.f, (_Float16)0.f};
        const f16x2_t sf0 = kin ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v0, 1.0f, false) : zero2;
        const f16x2_t sf1 = kin ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v1, 1.0f, false) : zero2;
        const f16x2_t sl0 = {sf0.x, sf0.x}, sh0 = {sf0.y, sf0.y};
        const f16x2_t sl1 = {sf1.x, sf1.x}, sh1 = {sf1.y, sf1.y};
        f16x8_t b0[4], b1[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            b0[ks] = decode_b(w0[d][ks], ks < 2 ? sl0 : sh0);
            b1[ks] = decode_b(w1[d][ks], ks < 2 ? sl1 : sh1);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[ks], b0[ks], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[ks], b1[ks], acc1, 0, 0, 0);
        }
        if (cu < nu && ci == nseg - 1) {  // uniform: this unit is complete
            const int unit = u_first + us * cu;
            // Lane (n, q) holds rows 4q..4q+3 of column n; the kept block is
            // row 4q + (n & 3), i.e. token q.  Sum the quarters of a quad.
            const float g0 = moe::group_sum<4>(pick(acc0, c)) * oscale;
            const float g1 = moe::group_sum<4>(pick(acc1, c)) * oscale;
            if (c == 0 && q < pr) {
                float *o = a.out + (size_t)(row0 + q) * N;
                if constexpr (GATED) {
                    o[16 * unit + 4 * w + rho] = moe::silu_f32(g0 * s2A) * (g1 * s2B);
                } else {
                    o[32 * unit + 8 * w + rho] = g0 * s2A;
                    o[32 * unit + 8 * w + 4 + rho] = g1 * s2A;
                }
            }
            acc0 = acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (++ci == nseg) {
            ci = 0;
            ++cu;
        }
        if constexpr (decltype(refill)::value) {
            // Loads keep their order; arithmetic and LDS work may move across.
            __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
            load(d);
            __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
        }
    };
    int base = 0;
    for (; base + D < total; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) step(d, std::true_type{});
    }
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, std::false_type{});
}

// Token-dense pass, for passes of more than 4 rows.  The (row, quarter)
// layout above feeds 4 tokens per MFMA and keeps a quarter of each result,
// so a pass of 16 rows costs 4 MFMAs per decoded operand; here one MFMA
// takes all 16 rows of the pass.  Each B column is one weight row: lane
// (n, q) loads 16 bytes (32 k) of row n at byte 64 window + 16 q, so a load
// instruction reads 16 rows x 64 contiguous bytes (streams within a few
// percent of 4 rows x 256 bytes).  MFMA d of a window takes dword d of every
// lane, i.e. k = 128 window + 32 q + 8 d + i in B slot (q, i); the A operand
// (x rows of the pass, staged as above) is read at the same k.  The k order
// inside the sum differs from the plain order; the products do not.
//   * Work items of 16 weight rows, two per unit, taken round-robin by the
//     waves: gate+up, 8 gate rows and the 8 up rows of the same 8 output
//     columns (lane n and lane n + 8 meet through a lane swap for the SiLU
//     product); down, 16 output rows.  A step is two 64-byte windows of the
//     item's rows.
//   * Scales: every 4 steps each lane loads 16 scale bytes (one row, one
//     step: two windows) into the wave's 1 KiB LDS area; a step reads its
//     two bytes per window per lane from there.
template <bool GATED, int D, bool TOK_LDS>
__device__ __forceinline__ void run_pass_dense(const DecArgs &a, int row0, int pr, int u_first, int nu, int us,
                                               const uint8_t *pA, const uint8_t *sA, const uint8_t *pB,
                                               const uint8_t *sB, float s2A, float s2B, uint8_t *lds,
                                               const int *tokl) {
    static_assert(D % kGroup == 0, "ring depth");
    const int K = a.K, N = a.N, ldx = a.ldx;
    const int rowbytes = K >> 1, sbytes = K >> 4;
    const int nwin = (rowbytes + 63) >> 6;  // 64-byte windows (128 k) per row
    const int nstep = (nwin + 1) >> 1;      // two windows per step
    const int lane = threadIdx.x & 63, w = moe::wave_id();
    const int n = lane & 15, q = lane >> 4;
    const int nit = 2 * nu;  // items of the block: item b is half b & 1 of unit u_first + us (b >> 1)
    auto item_of = [&](int b) { return 2 * (u_first + us * (b >> 1)) + (b & 1); };
    const int niw = nit > w ? (nit - w + 3) >> 2 : 0;  // items of this wave: item_of(w + 4 j)
    const int total = niw * nstep;
    // Item read past the end of this wave's list (a wave with none reads the
    // block's first item): the addresses stay inside the expert's weights.
    const int last_item = item_of(niw > 0 ? w + 4 * (niw - 1) : 0);

    uint8_t *sc_lds = lds + w * kScaleLds;
    uint32_t *rmax = reinterpret_cast<uint32_t *>(lds + kRmaxOff);
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds + kHdrLds);

    // Weight row of lane n in item 0, and the item stride (rows).
    //   gate+up: rows 8 i + n of gate (n < 8) or 8 i + n - 8 of up;
    //   down:    rows 16 i + n.
    const bool upl = GATED && n >= 8;
    const uint8_t *wb = (upl ? pB : pA) + (size_t)(GATED ? (n & 7) : n) * rowbytes;
    const size_t istride = (size_t)(GATED ? 8 : 16) * rowbytes;
    // Scale role: row r = lane >> 2 of the item, step s4 = lane & 3 of the group.
    const int r = lane >> 2, s4 = lane & 3;
    const bool upr = GATED && r >= 8;
    const uint8_t *sb = (upr ? sB : sA) + (size_t)(GATED ? (r & 7) : r) * sbytes;
    const size_t sistride = (size_t)(GATED ? 8 : 16) * sbytes;

    u32x4_t w0[D], w1[D], sv[D / kGroup];
    int ssh[D / kGroup];  // dword shift of a clamped scale load
    int lj = 0, ls = 0;   // stream position of the next load (item, step)
    auto load = [&](int d) {
        if (d % kGroup == 0) {
            // Scales of step (lj, ls) + s4 for row r: 16 bytes at 16 step.
            int l = ls + s4, j = lj;
#pragma unroll
            for (int i = 0; i < kGroup - 1; ++i) {
                const bool wrap = l >= nstep;
                l = wrap ? l - nstep : l;
                j = wrap ? j + 1 : j;
            }
            const bool real = j < niw;
            const int item = real ? item_of(w + 4 * j) : last_item;
            l = real ? l : nstep - 1;
            const int want = 16 * l;
            const int got = min(want, sbytes - 16);
            ssh[d / kGroup] = (want - got) >> 2;
            sv[d / kGroup] = moe::gload<u32x4_t>(sb + (size_t)item * sistride + got);
        }
        const bool real = lj < niw;  // past the end: the last real step again
        const int item = real ? item_of(w + 4 * lj) : last_item;
        const int st = real ? ls : nstep - 1;
        const uint8_t *rb = wb + (size_t)item * istride;
        w0[d] = moe::gload<u32x4_t>(rb + min(128 * st + 16 * q, rowbytes - 16));
        w1[d] = moe::gload<u32x4_t>(rb + min(128 * st + 64 + 16 * q, rowbytes - 16));
        if (++ls == nstep) {
            ls = 0;
            ++lj;
        }
    };

    int *ptok = reinterpret_cast<int *>(lds + kTokOff);
    if (threadIdx.x < 16) {
        rmax[threadIdx.x] = 0u;
        int tk = 0;  // one token: x row 0
        if (GATED && !a.single_token) {
            const int r = row0 + min((int)threadIdx.x, pr - 1);
            if constexpr (TOK_LDS)
                tk = tokl[r];
            else
                tk = moe::gload<int32_t>(a.sorted_tok + r);
        }
        ptok[threadIdx.x] = tk;
    }
    __syncthreads();  // rmax cleared, tokens published
    __builtin_amdgcn_sched_barrier(0);
    stage<GATED>(a, row0, pr, ptok, xs, rmax, [&]() {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(d);
            __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
        }
    });

    // A operand: row n of the pass (rows past it read row 0: dropped outputs).
    const int arow = (n < pr ? n : 0) * ldx;
    float oscale[4];  // undoes the row scaling of this lane's output rows 4 q + v
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int t = 4 * q + v;
        oscale[v] = exp2i(row_exp(rmax[t < pr ? t : 0]));
    }
    const float s2l = upl ? s2B : s2A;  // scale_2 of this lane's weight row

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int cj = 0, cs = 0;  // stream position being computed
    auto step = [&](const int d, auto refill) {
        if (d % kGroup == 0) {
            // This group's scales -> LDS at [step s4][row r][16 bytes] (undoing a clamped load's shift).
            const u32x4_t v = sv[d / kGroup];
            const int sh = ssh[d / kGroup];
            u32x4_t t;
            t[0] = sh == 0 ? v[0] : (sh == 1 ? v[1] : (sh == 2 ? v[2] : v[3]));
            t[1] = sh == 0 ? v[1] : (sh == 1 ? v[2] : v[3]);
            t[2] = sh == 0 ? v[2] : v[3];
            t[3] = v[3];
            *reinterpret_cast<u32x4_t *>(sc_lds + 256 * s4 + 16 * r) = t;
        }
        const uint8_t *sp = sc_lds + 256 * (d % kGroup) + 16 * n + 2 * q;
        const uint32_t u0 = *reinterpret_cast<const uint16_t *>(sp);      // window 2 step
        const uint32_t u1 = *reinterpret_cast<const uint16_t *>(sp + 8);  // window 2 step + 1
        const f16x2_t zero2 = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k0 = 128 * (2 * cs + h) + 32 * q;  // first k of this lane's chunk
            const bool kin = cj < niw && k0 < K;
            const int kac = k0 < K ? k0 : 0;  // past the end: any finite row data
            const f16x2_t sf = kin ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h ? u1 : u0, 1.0f, false) : zero2;
            const f16x2_t sl = {sf.x, sf.x}, sh = {sf.y, sf.y};
            const u32x4_t wv = h ? w1[d] : w0[d];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f16x8_t av = *reinterpret_cast<const f16x8_t *>(xs + arow + kac + 8 * i);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, decode_b(wv[i], i < 2 ? sl : sh), acc, 0, 0, 0);
            }
        }
        if (cj < niw && cs == nstep - 1) {  // uniform: this item is complete
            const int item = item_of(w + 4 * cj);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * q + v;  // C row (pass row) of acc[v]; column n
                const float val = acc[v] * oscale[v] * s2l;
                if constexpr (GATED) {
                    const float other = __shfl_xor(val, 8, 16);  // lane n <-> n + 8: gate <-> up
                    if (t < pr && !upl)
                        a.out[(size_t)(row0 + t) * N + 8 * item + n] = moe::silu_f32(val) * other;
                } else {
                    if (t < pr) a.out[(size_t)(row0 + t) * N + 16 * item + n] = val;
                }
            }
            acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (++cs == nstep) {
            cs = 0;
            ++cj;
        }
        if constexpr (decltype(refill)::value) {
            __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
            load(d);
            __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
        }
    };
    int base = 0;
    for (; base + D < total; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) step(d, std::true_type{});
    }
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, std::false_type{});
}

// Passes beyond the first of an expert with r routed rows.
__device__ __forceinline__ int further_passes(int r, int pr) { return r <= 0 ? 0 : (r - 1) / pr; }

// Block-wide exclusive prefix sum over the active slots of further_passes:
// pre[s] for s < n, pre[n] = total.  n <= 1024.
__device__ __forceinline__ void pass_prefix(const DecArgs &a, int n, int *pre) {
    __shared__ int wsum[kWaves];
    const int t = threadIdx.x, lane = t & 63, w = moe::wave_id();
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * t + i;
        int r = 0;
        if (sl < n) {
            const int e = a.active[sl];
            r = a.offsets[e + 1] - a.offsets[e];
        }
        c[i] = further_passes(r, a.pass_rows);
        sum += c[i];
    }
    int incl = sum;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    int run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * t + i;
        if (sl < n) pre[sl] = run;
        run += c[i];
    }
    if (t == kThreads - 1) pre[n] = run;  // the total
    __syncthreads();
}

// Last slot s < n with pre[s] <= g (pre non-decreasing, pre[0] = 0 <= g),
// found by the lanes of the calling wave together: lane l tests slot
// base + l, and the qualifying slots form a prefix, so the answer is the
// highest qualifying lane of the first chunk of 64 slots that does not
// qualify whole (one LDS read per lane per chunk, not a chain of dependent
// reads).  Wave-uniform.
__device__ __forceinline__ int find_slot(const int *pre, int n, int g) {
    const int lane = threadIdx.x & 63;
    int best = 0;
    for (int base = 0; base < n; base += 64) {
        const int s = base + lane;
        const unsigned long long m = __ballot(s < n && pre[s] <= g);
        if (m == 0ull) break;
        best = base + 63 - __clzll((long long)m);
        if (m != ~0ull) break;
    }
    return best;
}

// One pass of expert e, whose rows are the sorted positions [lo, hi).
// Units u_first + us i, i in [0, nu).
template <bool GATED, bool TOK_LDS, bool NT_OK>  // NT_OK: built with the nontemporal variant
__device__ __forceinline__ void do_pass_rows(const DecArgs &a, int e, int lo, int hi, int pass, int u_first,
                                             int nu, bool nt_ok, uint8_t *lds, const int *tokl = nullptr,
                                             int us = 1) {
    // Every table entry of expert e is read at once (e < E, so each read is
    // in bounds): one round of dependent loads, not one per table.
    const uint8_t *pA = a.pa[e];
    const uint8_t *pB = GATED ? a.pb[e] : pA;
    const uint8_t *sA = a.sa[e];
    const uint8_t *sB = GATED ? a.sb[e] : sA;
    const float s2A = a.s2a[e];
    const float s2B = GATED ? a.s2b[e] : s2A;
    // Hold the reads here: otherwise they sink below the branches that follow.
    asm volatile("" ::"s"(lo), "s"(hi), "s"(pA), "s"(pB), "s"(sA), "s"(sB), "s"(s2A), "s"(s2B));
    const int rows = hi - lo;
    const int m0 = pass * a.pass_rows;
    if (m0 >= rows) return;
    const int pr = min(a.pass_rows, rows - m0);
    constexpr int ucols = GATED ? 16 : 32;
    if (pA == nullptr || pB == nullptr || sA == nullptr || sB == nullptr) {  // absent expert: its rows are zero
        const int ncols = nu * ucols;
        for (int i = threadIdx.x; i < pr * ncols; i += kThreads) {
            const int m = i / ncols, c = i - m * ncols, k = c / ucols;
            a.out[(size_t)(lo + m0 + m) * a.N + (u_first + us * k) * ucols + (c - k * ucols)] = 0.f;
        }
        return;
    }
    // Passes of more than 4 rows (more than one token group) run token-dense:
    // one MFMA per 16 rows instead of one per 4.
    // Nontemporal weight loads: a large launch, and an expert read by this
    // pass alone.
    if (pr > 4)
        run_pass_dense<GATED, kDepth, TOK_LDS>(a, lo + m0, pr, u_first, nu, us, pA, sA, pB, sB, s2A, s2B, lds, tokl);
    else if (NT_OK && nt_ok && rows <= a.pass_rows)
        run_pass<GATED, kDepth, TOK_LDS, NT_OK>(a, lo + m0, pr, u_first, nu, us, pA, sA, pB, sB, s2A, s2B, lds, tokl);
    else
        run_pass<GATED, kDepth, TOK_LDS, false>(a, lo + m0, pr, u_first, nu, us, pA, sA, pB, sB, s2A, s2B, lds, tokl);
}

template <bool GATED, bool NT_OK>
__device__ __forceinline__ void do_pass(const DecArgs &a, int slot, int pass, int u_first, int nu, int us,
                                        int nactive, uint8_t *lds) {
    const int e = a.active[slot];  // -1 past the active count
    if (e < 0) return;
    const bool nt_ok = a.nt_min_active > 0 && nactive >= a.nt_min_active;
    do_pass_rows<GATED, false, NT_OK>(a, e, a.offsets[e], a.offsets[e + 1], pass, u_first, nu, nt_ok, lds, nullptr,
                                      us);
}

// Routing sort of P <= 64 pairs inside the block (the sort step fused into
// the gate+up launch when every expert's rows fit one pass).  Every wave
// ranks the pairs itself, one per lane, so no wave waits for another: the
// sorted position of a valid pair is the number of valid pairs with a
// smaller id plus those with its id earlier in flat order (stable), and the
// active experts are the first occurrences ranked by id.  Each wave writes
// the same LDS tables (its own later reads then need no barrier).  Returns
// (expert, first sorted position, rows) of active slot `slot`, expert -1
// past the active count.  Block (0, 0) also writes every output of
// moe_nvfp4_sort, the experts split over its waves.
__device__ __forceinline__ int3 fused_sort(const DecArgs &a, SortLds *sl, int slot) {
    const int lane = threadIdx.x & 63, w = moe::wave_id();
    const int P = a.P, E = a.E;
    const int id = lane < P ? a.topk_ids[lane] : -1;
    const bool valid = lane < P && id >= 0 && id < E;
    const unsigned long long vmask = __ballot(valid);
    const unsigned long long same = moe::match_lanes(id, valid, E > 1 ? 32 - __clz(E - 1) : 0);
    const unsigned long long lt = (1ull << lane) - 1ull;
    const bool first = valid && (same & lt) == 0ull;
    const unsigned long long fmask = __ballot(first);
    int less = 0, dless = 0;  // valid pairs / distinct ids below this lane's id
    for (int i = 0; i < P; ++i) {
        const int v = __builtin_amdgcn_readlane(id, i);
        less += ((vmask >> i) & 1ull) && v < id ? 1 : 0;
        dless += ((fmask >> i) & 1ull) && v < id ? 1 : 0;
    }
    const int rows = __popcll(same);
    const int pos = valid ? less + __popcll(same & lt) : -1;
    if (valid) sl->tok[pos] = lane / a.topk;
    const unsigned long long hit = __ballot(first && dless == slot);
    int3 r = make_int3(-1, 0, 0);
    if (hit != 0ull) {
        const int L = __ffsll((long long)hit) - 1;
        r = make_int3(__builtin_amdgcn_readlane(id, L), __builtin_amdgcn_readlane(less, L),
                      __builtin_amdgcn_readlane(rows, L));
    }
    if (blockIdx.x == 0 && blockIdx.y == 0) {
        if (first) {
            sl->active[dless] = id;
            sl->lo[dless] = less;
        }
        const int count = __popcll(fmask), total = __popcll(vmask);
        if (w == 0) {
            if (lane < P) a.sort_pos[lane] = pos;
            if (lane == 0 && total < P) atomicOr(a.err_flag, MOE_NVFP4_FLAG_BAD_EXPERT_ID);
            if (lane == 0) *a.sort_count = count;
        }
        for (int e = moe::kWave * w + lane; e <= E; e += kThreads) {
            // offsets[e]: valid pairs below e = first position of the first
            // active expert at or above e (binary search), else all of them.
            int lo = 0, hi = count;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sl->active[mid] < e) lo = mid + 1;
                else hi = mid;
            }
            a.sort_offsets[e] = lo < count ? sl->lo[lo] : total;
            if (e < E) a.sort_active[e] = e < count ? sl->active[e] : -1;
        }
        for (int p = moe::kWave * w + lane; p < P; p += kThreads) a.sort_tok[p] = p < total ? sl->tok[p] : -1;
    }
    return r;
}

// Block (x, y) of a grid of nx = ceil(units / G) columns: units x, x + nx,
// x + 2 nx, ... (at most G; with the fused sort, units [x G, x G + G)) of
//   y >= extra: the first pass (rows 0 .. pass_rows) of active slot y - extra;
//   y <  extra: further passes number y, y + extra, ... in slot order, so an
//               expert with many routed rows is spread over many blocks of
//               about the same length as the rest.
template <bool GATED, bool SORT>  // SORT: gate+up with the routing sort fused in (fused_sort set)
__global__ __launch_bounds__(kThreads) void k_decode_row(DecArgs a) {
    extern __shared__ uint4 lds4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);
    const int bx = blockIdx.x, y = blockIdx.y;
    if constexpr (!SORT) {
        // The blocks of a row take strided units (block x: x, x + nx, ...),
        // so all of them sweep the expert's weights together.
        const int nx = gridDim.x, nu = (a.units - bx + nx - 1) / nx;
        if (nu <= 0) return;
        if (y >= a.extra) {
            // The nontemporal variant serves the down projection here; large
            // gate+up launches run persistent.
            do_pass<GATED, !GATED>(a, y - a.extra, 0, bx, nu, nx, GATED ? 0 : *a.nactive, lds);
            return;
        }
        int *pre = reinterpret_cast<int *>(lds + kPreOff);
        const int n = *a.nactive;
        pass_prefix(a, n, pre);
        const int total = pre[n];
        for (int g = y; g < total; g += a.extra) {
            const int slot = find_slot(pre, n, g);
            if (g > y) __syncthreads();  // the previous pass's readers of LDS are done
            do_pass<GATED, !GATED>(a, slot, 1 + g - pre[slot], bx, nu, nx, n, lds);
        }
        return;
    }
    const int u_first = bx * a.G;
    const int nu = min(a.G, a.units - u_first);
    if (nu <= 0) return;
    if constexpr (GATED && SORT) {  // extra == 0: one pass per expert
        const int3 r = fused_sort(a, reinterpret_cast<SortLds *>(lds + kPreOff), y);
        if (r.x < 0) return;  // past the active count
        do_pass_rows<GATED, true, false>(a, r.x, r.y, r.y + r.z, 0, u_first, nu, false, lds,
                                         reinterpret_cast<const SortLds *>(lds + kPreOff)->tok);
    }
}

// floor(n / d) for 0 <= n < 2^52 and d > 0, through one fp64 division (its
// quotient is within one of the true one) and an exact integer correction;
// a 64-bit integer division is a long instruction sequence on this hardware.
__device__ __forceinline__ int64_t div_floor(int64_t n, int64_t d) {
    int64_t q = (int64_t)((double)n / (double)d);
    q = q * d > n ? q - 1 : q;
    q = (q + 1) * d <= n ? q + 1 : q;
    return q;
}

// Relative cost of one unit of a pass with r routed rows, for the share
// walk (token groups of 4 share each decoded weight; the weight stream
// itself costs the same).  On the 64-token launch the flatter model below
// measured 3% slower here.
constexpr int kUnitCostMax = 35;  // the larger of unit_cost(16) and unit_cost_one(16)
constexpr int kOnePassShares = 4;  // one pass per block when every pass is worth this many shares
__device__ __forceinline__ int unit_cost(int r) { return 3 + ((r + 3) >> 2); }
// The same for one pass per block: fitted to per-block timestamps of the
// 32-token launch (staging, then about 3.6 + 0.07 r us per unit), where it
// brings the blocks' ends closer together than unit_cost (launch 3%
// shorter).
__device__ __forceinline__ int unit_cost_one(int r) { return 19 + r; }

// An active slot's expert, first sorted position and routed rows, cached in
// LDS while a persistent block finds its share.
struct SlotInfo {
    int e, lo, rows;
};

// Block-wide: every slot's expert and row range (slot(sl) for sl < cap,
// an expert of -1 past the active count), cached in si[sl]; and the
// exclusive prefix sums over the n active slots of the cost of all their
// passes (units x unit_cost per pass in pre, units x unit_cost_one in
// pre1): pre[s] for s < n, pre[n] = total (the same for pre1).  pass_min:
// the unit_cost cost of the cheapest pass.
template <typename SlotFn>
__device__ __forceinline__ void cost_prefix(const DecArgs &a, int n, int *pre, int *pre1, SlotInfo *si,
                                            int &pass_min, SlotFn &&slot) {
    __shared__ int wsum[2][kWaves], wmin[kWaves];
    const int t = threadIdx.x, lane = t & 63, w = moe::wave_id();
    const int pr = a.pass_rows, cap = a.cap;
    int c[4], c1[4], sum = 0, sum1 = 0, cmin = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * t + i;
        const SlotInfo in = sl < cap ? slot(sl) : SlotInfo{-1, 0, 0};
        const int r = in.rows;
        if (sl < cap) si[sl] = in;
        const int full = r / pr, rem = r - full * pr;
        const bool act = sl < n;
        c[i] = act ? a.units * (full * unit_cost(pr) + (rem > 0 ? unit_cost(rem) : 0)) : 0;
        c1[i] = act ? a.units * (full * unit_cost_one(pr) + (rem > 0 ? unit_cost_one(rem) : 0)) : 0;
        sum += c[i];
        sum1 += c1[i];
        if (act) cmin = min(cmin, a.units * unit_cost(rem > 0 ? rem : pr));  // the slot's cheapest pass
    }
    int incl = sum, incl1 = sum1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64), v1 = __shfl_up(incl1, off, 64);
        if (lane >= off) {
            incl += v;
            incl1 += v1;
        }
    }
    const uint32_t wm = moe::wave_min_u32((uint32_t)cmin);
    if (lane == 63) {
        wsum[0][w] = incl;
        wsum[1][w] = incl1;
    }
    if (lane == 0) wmin[w] = (int)wm;
    __syncthreads();
    int base = 0, base1 = 0;
    for (int i = 0; i < w; ++i) {
        base += wsum[0][i];
        base1 += wsum[1][i];
    }
    int run = base + incl - sum, run1 = base1 + incl1 - sum1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * t + i;
        if (sl < n) {
            pre[sl] = run;
            pre1[sl] = run1;
        }
        run += c[i];
        run1 += c1[i];
    }
    if (t == kThreads - 1) {
        pre[n] = run;
        pre1[n] = run1;
    }
    pass_min = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    __syncthreads();
}

// The first unit, in (slot, pass, unit) order, whose cost-weighted start is
// at or after c; s == n when there is none.
struct Cursor {
    int s, p, u;
};
__device__ __forceinline__ Cursor locate(const DecArgs &a, const int *pre, const SlotInfo *si, int n, int c) {
    Cursor k{n, 0, 0};
    if (c >= pre[n]) return k;
    int s = find_slot(pre, n, c);
    int rem = c - pre[s];
    const int pr = a.pass_rows;
    int r = si[s].rows;
    int p = 0;
    for (;;) {
        if (p * pr >= r) {  // past the slot's last pass: first unit of the next slot
            ++s;
            p = 0;
            if (s >= n) break;
            r = si[s].rows;
            rem = 0;
            continue;
        }
        const int w = unit_cost(min(pr, r - p * pr));
        if (rem >= a.units * w) {
            rem -= a.units * w;
            ++p;
            continue;
        }
        const int u = (rem + w - 1) / w;
        if (u >= a.units) {
            ++p;
            rem = 0;
            continue;
        }
        k = Cursor{s, p, u};
        return k;
    }
    return Cursor{n, 0, 0};
}

// Persistent mode (launches with plenty of work).  The work is the list of
// (slot, pass, unit) in order, each unit weighted by unit_cost of its pass;
// block b takes the units whose weighted start lies in the b-th equal share,
// and streams them pass by pass.  Every block is busy for about the same
// time and no block is launched only to find no work.  Set-up reads the
// routing tables once: the slots' experts and row ranges are cached in LDS
// (in the area the activation rows use later) and the share's first 64
// slots move to registers (lane i: slot first + i) before the first pass
// stages over them.
// Fused sort in the persistent launch: the sorted tokens sit at this int
// offset of the pass-prefix area, above its at most kBlockSortPairs + 1
// entries.
constexpr int kSortTokPre = moe::kBlockSortPairs + 4;
static_assert(kSortTokPre + moe::kBlockSortPairs <= kPreLds / 4, "the sorted tokens fit the prefix area");

template <bool GATED, bool SORT>  // SORT: the routing sort runs in every block (P <= 256; block 0 writes it)
__global__ __launch_bounds__(kThreads) void k_decode_row_persist(DecArgs a) {
    extern __shared__ uint4 lds4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);
    int *pre = reinterpret_cast<int *>(lds + kPreOff);
    const int lane = threadIdx.x & 63;
    int pass_min, n;
    SlotInfo *si;
    int *pre1;  // prefix of the one-pass-per-block costs, after the slot cache
    const int *tokl = nullptr;
    if constexpr (SORT) {
        // Set-up area (where the activation rows go later): offsets[E + 1],
        // per-wave histograms [4 E], active list [E], then the slot cache.
        // The sorted tokens go above the pass prefix instead: every pass a
        // block runs reads its rows' tokens there, also after an earlier
        // pass's staging has overwritten the set-up area.
        int *offs = reinterpret_cast<int *>(lds + kHdrLds);
        int *cntw = offs + a.E + 1;
        int *act = cntw + 4 * a.E;
        int *stok = pre + kSortTokPre;
        si = reinterpret_cast<SlotInfo *>(act + a.E);
        pre1 = reinterpret_cast<int *>(si + a.cap);
        const moe::SortOutputs out{a.sort_offsets, a.sort_tok, a.sort_pos, a.sort_active, a.sort_count, a.err_flag};
        n = moe::block_sort_256(a.topk_ids, a.P, a.topk, a.E, offs, cntw, act, stok, out, blockIdx.x == 0);
        tokl = stok;
        cost_prefix(a, n, pre, pre1, si, pass_min, [&](int sl) {
            const int e = sl < n ? act[sl] : -1;
            return e < 0 ? SlotInfo{-1, 0, 0} : SlotInfo{e, offs[e], offs[e + 1] - offs[e]};
        });
    } else {
        si = reinterpret_cast<SlotInfo *>(lds + kHdrLds);
        pre1 = reinterpret_cast<int *>(si + a.cap);
        // The active list is read without waiting for the active count:
        // its entries past the count are -1.
        n = *a.nactive;
        cost_prefix(a, n, pre, pre1, si, pass_min, [&](int sl) {
            const int e = a.active[sl];
            if (e < 0) return SlotInfo{-1, 0, 0};
            const int lo = a.offsets[e];
            return SlotInfo{e, lo, a.offsets[e + 1] - lo};
        });
    }
    const int total = pre[n];
    // Blocks go to the 8 XCDs round-robin; consecutive shares go to one XCD,
    // so the later passes of an expert mostly run where its earlier passes
    // left the weights in L2.
    const int g = gridDim.x;
    const int bx = (g & 7) == 0 ? (int)((blockIdx.x & 7) * (g >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
    const bool nt_ok = a.nt_min_active > 0 && n >= a.nt_min_active;
    if (n > 0 && (int64_t)pass_min * g >= (int64_t)kOnePassShares * total) {
        // Every pass is worth several blocks' shares: block bx takes the pass
        // whose cost range holds its point (bx + 1/2) total / g, and an even
        // part of that pass's units among the blocks whose points fall in
        // it.  Each block then stages once and streams one pass.  (With
        // fewer shares per pass the whole-block rounding unbalances more
        // than a second pass costs: the 64-token launch, about two shares
        // per pass, measured 8% slower this way.)  The points are placed on
        // the unit_cost_one prefix.
        const int total1 = pre1[n];
        const int64_t pt = div_floor((int64_t)(2 * bx + 1) * total1, 2 * (int64_t)g);
        const int sl = find_slot(pre1, n, (int)pt);
        const SlotInfo in = si[sl];
        const int pr = a.pass_rows;
        int64_t ps = pre1[sl];
        int p = 0, pc = 0;
        for (;; ++p) {
            pc = a.units * unit_cost_one(min(pr, in.rows - p * pr));
            if (pt < ps + pc || (p + 1) * pr >= in.rows) break;
            ps += pc;
        }
        // blocks whose points lie in [ps, ps + pc): (2b + 1) total1 in [2 g ps, 2 g (ps + pc))
        auto first_at = [&](int64_t c) -> int64_t {
            const int64_t v = 2 * (int64_t)g * c - total1;
            return v <= 0 ? 0 : div_floor(v + 2 * (int64_t)total1 - 1, 2 * (int64_t)total1);
        };
        const int b_lo = (int)first_at(ps), nb = (int)(first_at(ps + pc) - b_lo);
        const int i = bx - b_lo;
        __syncthreads();  // the set-up's readers of LDS are done
        // Block i of the pass takes units i, i + nb, i + 2 nb, ...  Each pass
        // has blocks in proportion to its cost, so the passes of an expert
        // with several sweep its units at about the same pace, next to each
        // other in bx (one XCD): a pass reading a unit after another mostly
        // finds it in L2, where contiguous ranges of different lengths per
        // pass read each unit at unrelated times.  (Single-pass experts
        // gain too: the 32-token launch measured 48.9 us against 50.2 us
        // with contiguous ranges there.)
        const int nu = i < a.units ? (a.units - i + nb - 1) / nb : 0;
        if (nu > 0)
            do_pass_rows<GATED, SORT, true>(a, in.e, in.lo, in.lo + in.rows, p, i, nu, nt_ok, lds, tokl, nb);
        return;
    }
    const int c0 = (int)div_floor((int64_t)total * bx, g);
    const int c1 = (int)div_floor((int64_t)total * (bx + 1), g);
    Cursor k = locate(a, pre, si, n, c0);
    const Cursor end = locate(a, pre, si, n, c1);
    // The share's first slots move to registers (lane l, entry j: slot
    // s_first + l + 64 j), every slot of the launch when the sort runs here
    // (P <= 256 pairs, so at most 256 slots).
    const int s_first = k.s;
    constexpr int kRegSlots = SORT ? 4 : 1;
    SlotInfo mine[kRegSlots];
#pragma unroll
    for (int j = 0; j < kRegSlots; ++j) {
        const int sl = s_first + lane + 64 * j;
        mine[j] = sl < n ? si[sl] : SlotInfo{-1, 0, 0};
    }
    while (k.s < n && (k.s < end.s || (k.s == end.s && (k.p < end.p || (k.p == end.p && k.u < end.u))))) {
        const bool last_item = k.s == end.s && k.p == end.p;
        const int ub = last_item ? end.u : a.units;
        __syncthreads();  // the set-up's (or the previous pass's) readers of LDS are done
        const int i = k.s - s_first;
        int e = -1, lo = 0, rows = 0;
        if (i < 64 * kRegSlots) {
#pragma unroll
            for (int j = 0; j < kRegSlots; ++j) {
                if (i >> 6 == j) {
                    e = __builtin_amdgcn_readlane(mine[j].e, i & 63);
                    lo = __builtin_amdgcn_readlane(mine[j].lo, i & 63);
                    rows = __builtin_amdgcn_readlane(mine[j].rows, i & 63);
                }
            }
        } else if constexpr (!SORT) {  // a share over more than 64 slots (many experts with few rows)
            e = a.active[k.s];
            lo = a.offsets[e];
            rows = a.offsets[e + 1] - lo;
        }
        do_pass_rows<GATED, SORT, true>(a, e, lo, lo + rows, k.p, k.u, ub - k.u, nt_ok, lds, tokl);
        // next (slot, pass)
        if ((k.p + 1) * a.pass_rows < rows) {
            k = Cursor{k.s, k.p + 1, 0};
        } else {
            k = Cursor{k.s + 1, 0, 0};
        }
    }
}

// Down projection with the top-k blend fused in, for one or a few tokens.
//
// The blend (out[t] = sum over j of w[t, j] * y[pair (t, j)], fp32, ascending
// j, one rounding to bf16) needs every pair of a token at once, so here a
// block takes one token and C = 8 G output columns of the down matrices of
// all of that token's pairs, and the pairs' y values never leave LDS: no y
// tensor, no blend launch, no second trip through memory.  The weights of an
// expert are read once per token routed to it, so this suits decode with few
// tokens (one token: every expert once).
//   * Pairs.  Wave 0 reads the token's routed ids, sorted positions and
//     weights, then the expert tables of the pairs that have an expert
//     ("live": a position and non-NULL weights), and lists the live pairs in
//     ascending j.  Live pair r belongs to wave r mod 4.
//   * Activations.  The h rows of the live pairs (gathered by sorted
//     position) are staged as in the grouped kernel: fp16, one power of two
//     per row.  With one token every row of h is one of its pairs', so the
//     rows are loaded at entry in sorted order, before the pairs are read.
//   * Stream.  Wave w streams units of 8 weight rows, (its p-th live pair,
//     column group g), through the same register ring, lane layout and
//     matrix-core arithmetic as the grouped kernel, so each y value is the
//     one the grouped kernel computes for that row, bit for bit.  Unit
//     results go to an LDS table y[live pair][column].
//   * Blend.  After one barrier, thread n < C sums its column over the pairs
//     in ascending j exactly as the blend kernel does (a pair whose expert is
//     NULL adds w * 0; a pair with no expert adds nothing) and writes bf16.
constexpr int kBlendMaxK = 64;     // pairs per token
constexpr int kBlendMaxCols = 32;  // output columns per block (G <= 4)
struct BlendLds {
    const uint8_t *pa[kBlendMaxK];  // by live index: the pair's expert
    const uint8_t *sa[kBlendMaxK];
    float s2[kBlendMaxK];
    int pos[kBlendMaxK];        // by live index: sorted position (h row)
    uint32_t rmax[kBlendMaxK];  // by live index: staged row maxima
    float w[kBlendMaxK];        // by pair j: routing weight
    int live_of[kBlendMaxK];    // by pair j: live index; -1 NULL expert (y = 0); -2 no expert
    int nlive;
};
constexpr int kBlendTblOff = kWaves * kScaleLds;
constexpr int kBlendYOff = (kBlendTblOff + (int)sizeof(BlendLds) + 15) & ~15;
constexpr int kBlendHdrLds = kBlendYOff + kBlendMaxK * kBlendMaxCols * 4;

__global__ __launch_bounds__(kThreads) void k_decode_down_blend(DecArgs a) {
    extern __shared__ uint4 lds4[];
    uint8_t *lds = reinterpret_cast<uint8_t *>(lds4);
    BlendLds *bl = reinterpret_cast<BlendLds *>(lds + kBlendTblOff);
    float *ypart = reinterpret_cast<float *>(lds + kBlendYOff);
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds + kBlendHdrLds);
    const int t = blockIdx.y, k = a.topk, G = a.G, C = 8 * G;
    const int col0 = blockIdx.x * C;
    const int lane = threadIdx.x & 63, w = moe::wave_id();
    constexpr int D = kDepth;

    // One token: its k routed pairs hold every row of h, so the rows are
    // loaded in sorted order before the pairs are read (they do not wait
    // for the positions); a live pair then uses its position's row.  The
    // threads split the rows as the staging below does: 2^plg threads per
    // row, thread i on row i >> plg and its chunks (8 floats each)
    // i mod 2^plg + 2^plg j.
    constexpr int kPreSB = 4;
    const int cpr = a.K >> 3;
    const int plg = k <= 64 ? (int)threads_per_row_log2(k) : 2;
    const int pm = (int)threadIdx.x >> plg, pj = (int)threadIdx.x & ((1 << plg) - 1);
    const bool pre = gridDim.y == 1 && k <= 64 && ((cpr + (1 << plg) - 1) >> plg) <= kPreSB;
    f32x4_t pf0[kPreSB], pf1[kPreSB];
    if (pre) {
        const float *hsrc = static_cast<const float *>(a.act) + (size_t)(pm < k ? pm : 0) * a.K;
#pragma unroll
        for (int i = 0; i < kPreSB; ++i) {
            const int c = min(pj + (i << plg), cpr - 1);
            pf0[i] = moe::gload<f32x4_t>(hsrc + 8 * c);
            pf1[i] = moe::gload<f32x4_t>(hsrc + 8 * c + 4);
        }
    }

    if (w == 0) {  // the token's pairs: lane j holds pair j
        int pos = -1, id = -1;
        float wj = 0.f;
        if (lane < k) {
            const size_t p = (size_t)t * k + lane;
            id = a.topk_ids[p];
            pos = a.blend_pos[p];
            wj = a.blend_w[p];
        }
        const bool routed = lane < k && pos >= 0 && id >= 0 && id < a.E;
        const uint8_t *pa = nullptr, *sa = nullptr;
        float s2 = 0.f;
        if (routed) {
            pa = a.pa[id];
            sa = a.sa[id];
            s2 = a.s2a[id];
        }
        const bool live = routed && pa != nullptr && sa != nullptr;
        const unsigned long long lm = __ballot(live);
        const int li = __popcll(lm & ((1ull << lane) - 1ull));
        if (live) {
            bl->pa[li] = pa;
            bl->sa[li] = sa;
            bl->s2[li] = s2;
            bl->pos[li] = pos;
        }
        if (lane < k) {
            bl->w[lane] = wj;
            bl->live_of[lane] = live ? li : (routed ? -1 : -2);
        }
        bl->rmax[lane] = 0u;
        if (lane == 0) bl->nlive = __popcll(lm);
    }
    __syncthreads();
    const int nlive = bl->nlive;

    if (nlive > 0) {
        const int K = a.K, ldx = a.ldx;
        const int rowbytes = K >> 1, sbytes = K >> 4;
        const int nseg = (rowbytes + kSegBytes - 1) / kSegBytes;
        const int npw = nlive > w ? (nlive - 1 - w) / kWaves + 1 : 0;  // live pairs w, w + 4, ...
        const int nu = npw * G;                                          // units (pair p, group g)
        const int total = nu * nseg;
        const int n = lane & 15, q = lane >> 4;
        const int rho = n >> 2, c = n & 3;
        const int choff = 64 * q + 16 * c;
        const int s4 = lane >> 4, r8 = (lane >> 1) & 7, hh = lane & 1;
        uint8_t *sc_lds = lds + w * kScaleLds;

        u32x4_t w0[D], w1[D], sv[D / kGroup];
        int ssh[D / kGroup];
        int lu = 0, li = 0, lp = 0, lg = 0;  // next load: unit lu = (pair lp, group lg), segment li
        auto load = [&](int d) {
            if (d % kGroup == 0) {
                // Scale slice of step (lu, li) + s4 for row r8 of the unit (16 bytes, half hh).
                int l = li + s4, u = lu, p = lp, g = lg;
#pragma unroll
                for (int i = 0; i < kGroup - 1; ++i) {
                    const bool wrap = l >= nseg;
                    l = wrap ? l - nseg : l;
                    u = wrap ? u + 1 : u;
                    g = wrap ? g + 1 : g;
                    p = g == G ? p + 1 : p;
                    g = g == G ? 0 : g;
                }
                const bool real = u < nu;
                p = real ? p : npw - 1;
                g = real ? g : G - 1;
                l = real ? l : nseg - 1;
                const int want = 32 * l + 16 * hh;
                const int got = min(want, sbytes - 16);
                ssh[d / kGroup] = (want - got) >> 2;
                const uint8_t *sk = bl->sa[w + kWaves * p];
                sv[d / kGroup] = moe::gload<u32x4_t>(sk + (size_t)(col0 + 8 * g + r8) * sbytes + got);
            }
            const bool real = lu < nu;  // past the end: the last real step again
            const int p = real ? lp : npw - 1, g = real ? lg : G - 1;
            const int off = min(kSegBytes * (real ? li : nseg - 1) + choff, rowbytes - 16);
            const uint8_t *pk = bl->pa[w + kWaves * p] + (size_t)(col0 + 8 * g + rho) * rowbytes + off;
            w0[d] = moe::gload<u32x4_t>(pk);
            w1[d] = moe::gload<u32x4_t>(pk + (size_t)4 * rowbytes);
            if (++li == nseg) {
                li = 0;
                ++lu;
                if (++lg == G) {
                    lg = 0;
                    ++lp;
                }
            }
        };

        auto fill = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            if (nu > 0) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    load(d);
                    __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
                }
            }
        };
        if (pre) {
            // The preloaded rows: maxima, then scaled to fp16 in sorted order.
            fill();
            const bool rin = pm < k;
            uint32_t mx = 0u;
#pragma unroll
            for (int i = 0; i < kPreSB; ++i)
                if (rin && pj + (i << plg) < cpr) mx = max(mx, __float_as_uint(absmax8f(pf0[i], pf1[i])));
            row_group_max(bl->rmax, pm, rin, mx, plg);
            __syncthreads();  // maxima complete
            const float f = exp2i(-row_exp(bl->rmax[rin ? pm : 0]));
#pragma unroll
            for (int i = 0; i < kPreSB; ++i)
                if (rin && pj + (i << plg) < cpr) put_f16x8(xs + pm * ldx + 8 * (pj + (i << plg)), pf0[i], pf1[i], f);
            __syncthreads();
        } else {
            stage<false, true>(a, 0, nlive, nullptr, xs, bl->rmax, fill, bl->pos);
        }

        if (nu > 0) {
            const int cA = n & 3;
            const int sread0 = 32 * rho + 8 * q + 2 * c;
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            int cu = 0, ci = 0, cp = 0, cg = 0;  // stream position being computed
            auto step = [&](const int d, auto refill) {
                if (d % kGroup == 0) {
                    const u32x4_t v = sv[d / kGroup];
                    const int s = ssh[d / kGroup];
                    u32x4_t r;
                    r[0] = s == 0 ? v[0] : (s == 1 ? v[1] : (s == 2 ? v[2] : v[3]));
                    r[1] = s == 0 ? v[1] : (s == 1 ? v[2] : v[3]);
                    r[2] = s == 0 ? v[2] : v[3];
                    r[3] = v[3];
                    *reinterpret_cast<u32x4_t *>(sc_lds + 16 * lane) = r;
                }
                const int rl = w + kWaves * (cu < nu ? cp : npw - 1);  // live row of this unit
                const int xr = pre ? bl->pos[rl] : rl;                 // its staged row
                const int ka = 512 * ci + 128 * q + 32 * cA;
                const int kac = ka < K ? ka : 0;
                f16x8_t a0[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    a0[ks] = *reinterpret_cast<const f16x8_t *>(xs + xr * ldx + kac + 8 * ks);
                const int kq = 512 * ci + 128 * q + 32 * c;
                const bool kin = cu < nu && kq < K;
                const uint8_t *sp = sc_lds + 256 * (d % kGroup) + sread0;
                const uint32_t v0 = *reinterpret_cast<const uint16_t *>(sp);
                const uint32_t v1 = *reinterpret_cast<const uint16_t *>(sp + 128);
                const f16x2_t zero2 = {(_Float16)0.f, (_Float16)0.f};
                const f16x2_t sf0 = kin ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v0, 1.0f, false) : zero2;
                const f16x2_t sf1 = kin ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v1, 1.0f, false) : zero2;
                const f16x2_t sl0 = {sf0.x, sf0.x}, sh0 = {sf0.y, sf0.y};
                const f16x2_t sl1 = {sf1.x, sf1.x}, sh1 = {sf1.y, sf1.y};
                f16x8_t b0[4], b1[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    b0[ks] = decode_b(w0[d][ks], ks < 2 ? sl0 : sh0);
                    b1[ks] = decode_b(w1[d][ks], ks < 2 ? sl1 : sh1);
                }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[ks], b0[ks], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[ks], b1[ks], acc1, 0, 0, 0);
                }
                if (cu < nu && ci == nseg - 1) {  // uniform: this unit is complete
                    // Every A row holds the pair's h row: keep token 0 (q == 0)
                    // of the quad sums.
                    const float oscale = exp2i(row_exp(bl->rmax[xr]));
                    const float s2 = bl->s2[rl];
                    const float g0 = moe::group_sum<4>(pick(acc0, c)) * oscale;
                    const float g1 = moe::group_sum<4>(pick(acc1, c)) * oscale;
                    if (c == 0 && q == 0) {
                        ypart[rl * C + 8 * cg + rho] = g0 * s2;
                        ypart[rl * C + 8 * cg + 4 + rho] = g1 * s2;
                    }
                    acc0 = acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                if (++ci == nseg) {
                    ci = 0;
                    ++cu;
                    if (++cg == G) {
                        cg = 0;
                        ++cp;
                    }
                }
                if constexpr (decltype(refill)::value) {
                    __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
                    load(d);
                    __builtin_amdgcn_sched_barrier(kMoveAcrossLoads);
                }
            };
            int base = 0;
            for (; base + D < total; base += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) step(d, std::true_type{});
            }
#pragma unroll
            for (int d = 0; d < D; ++d) step(d, std::false_type{});
        }
    }
    __syncthreads();  // every live pair's y columns are in LDS
    if ((int)threadIdx.x < C) {
        // Eight pairs at a time: their table entries and y values are read
        // before the fmaf chain (ascending j, as the blend kernel sums), so
        // the LDS reads overlap instead of forming one dependent chain.
        const int col = threadIdx.x;
        float acc = 0.f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            int r[8];
            float wv[8], yv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool in = j0 + u < k;
                r[u] = in ? bl->live_of[j0 + u] : -2;
                wv[u] = in ? bl->w[j0 + u] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) yv[u] = r[u] >= 0 ? ypart[r[u] * C + col] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (r[u] != -2) acc = fmaf(wv[u], yv[u], acc);
        }
        a.blend_out[(size_t)t * a.N + col0 + col] = moe::f32_to_bf16_rne(acc);
    }
}

}  // namespace

// Launch the row-major grouped projection (used by the two C-ABI entry points).
// Shapes: N % 64 == 0, K % 64 == 0 and K >= 256 (checked by the callers).
int moe_launch_sort(const int32_t *topk_ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_tok,
                    int32_t *pair_pos, int32_t *active, int32_t *active_count, uint32_t *err_flag,
                    hipStream_t stream);

namespace {

// Launch shape of the decode kernels for one projection (shared by the
// launcher and the fusion query below).
struct DecConfig {
    int units, G, ldx, pass_rows, extra;
    size_t lds;
    bool persistent;
    bool ok;  // false: an activation row does not fit the LDS budget
};

DecConfig decode_config(bool gated, int N, int K, int P, int E) {
    DecConfig c{};
    const int ucols = gated ? 16 : 32;
    c.units = (N + ucols - 1) / ucols;
    const int cap = E < P ? E : P;
    // Units per block: about 32 ring steps per wave, so a block's start-up
    // (tables, activation staging, first loads) is paid over enough streaming,
    // but at most 6: on short rows (K about 2048) 8 units per block measured
    // 3-8% slower on the down projection than 6 (fewer, longer blocks leave a
    // longer tail), and 4 or fewer paid the start-up too often.  Fewer still
    // when the grid would otherwise not fill two blocks per CU.
    const int nseg = (K / 2 + 255) / 256;
    int G = (32 + nseg - 1) / nseg;
    G = G < 1 ? 1 : (G > 6 ? 6 : G);
    while (G > 1 && (int64_t)cap * ((c.units + G - 1) / G) < 2 * (int64_t)moe_host::cu_count()) --G;
    c.G = G;
    // Staged row stride: 2K bytes padded to 16 mod 256, so the 16 lanes of an
    // A-operand read (4 rows x 4 quarters, 64 bytes apart) hit distinct banks.
    const int pad_bytes = ((16 - (2 * K) % 256) + 256) % 256;
    c.ldx = K + pad_bytes / 2;
    const size_t row_lds = (size_t)c.ldx * 2;
    int pr = (int)(kLdsBudget / row_lds);
    c.ok = pr >= 1;
    if (pr > 4 * kMaxTG) pr = 4 * kMaxTG;
    if (pr > P) pr = P;
    if (pr < 1) pr = 1;
    c.pass_rows = pr;
    c.lds = (size_t)kHdrLds + (size_t)pr * row_lds;
    // Persistent mode for gate+up when the grid would hold many blocks per
    // resident slot and the weighted work count fits an int.  (The down
    // projection measured faster as one block per unit group: with its
    // shorter rows (K = I) a persistent block crosses more pass boundaries,
    // each a fresh activation stage and ring fill, 5% on 64 tokens x 256
    // experts.)
    const int nblk = 2 * moe_host::cu_count();
    const int64_t max_passes = (int64_t)(P - 1) / pr + cap;
    c.persistent = gated && (int64_t)cap * ((c.units + G - 1) / G) > 2 * (int64_t)nblk &&
                   max_passes * c.units * kUnitCostMax < ((int64_t)1 << 31);
    // Further passes number at most sum_e floor((R_e - 1) / pr) <= (P - 1) / pr;
    // the grid's y extent is kept within its limit by striding over them.
    int extra = (P - 1) / pr;
    c.extra = extra > 64 ? 64 : extra;
    return c;
}

// The routing sort runs inside the gate+up launch when every expert's rows
// fit one pass (no further-pass block rows) and the pairs fit a wave, or
// when the launch is persistent and the pairs fit one block's sort.
bool decode_sort_fuses(const DecConfig &c, int P) {
    return c.persistent ? P <= moe::kBlockSortPairs : (c.extra == 0 && P <= kSortPairs);
}

}  // namespace

// Launches that moe_nvfp4_sort_gate_up_silu enqueues for row-major weights (1
// when the sort runs inside the gate+up launch, else 2).
int moe_decode_sort_gate_up_launches(int N, int K, int P, int E) {
    return decode_sort_fuses(decode_config(true, N, K, P, E), P) ? 1 : 2;
}

int moe_launch_decode_row(bool gated, const void *act, const int32_t *sorted_tok, const int32_t *offsets,
                          const int32_t *active, const int32_t *nactive, const moe_nvfp4_experts &A,
                          const moe_nvfp4_experts *B, float *out, int N, int K, int T, int P, int E,
                          hipStream_t stream, const MoeSortFuse *fuse) {
    DecArgs a = {};
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
    a.single_token = gated && T == 1;
    // Nontemporal weight loads once the active experts' weights of this
    // projection exceed the 256 MB Infinity Cache.
    const int64_t expert_bytes = (gated ? 2 : 1) * (int64_t)N * (K / 2 + K / 16);
    a.nt_min_active = (int)(((int64_t)256 << 20) / expert_bytes + 1);
    const DecConfig c = decode_config(gated, N, K, P, E);
    if (!c.ok) return MOE_NVFP4_ELIMIT;
    a.units = c.units;
    a.G = c.G;
    a.ldx = c.ldx;
    a.pass_rows = c.pass_rows;
    const size_t lds = c.lds;
    const int G = c.G;
    const int nblk = 2 * moe_host::cu_count();
    const int cap = E < P ? E : P;
    a.cap = cap;
    if (c.persistent) {
        // The set-up caches a SlotInfo per slot where the activation rows go
        // (with the sort in the launch: after its LDS tables; the sorted
        // tokens go above the pass prefix), then the one-pass cost prefix.
        size_t setup = sizeof(SlotInfo) * (size_t)cap + sizeof(int) * (size_t)(cap + 1);
        const bool sort_here = fuse && decode_sort_fuses(c, P);
        if (sort_here) {
            setup += sizeof(int) * (size_t)(6 * E + 1);
            a.P = P;
            a.topk = fuse->k;
            a.E = E;
            a.topk_ids = fuse->topk_ids;
            a.sort_offsets = fuse->offsets;
            a.sort_tok = fuse->sorted_tok;
            a.sort_pos = fuse->pair_pos;
            a.sort_active = fuse->active;
            a.sort_count = fuse->active_count;
            a.err_flag = fuse->err_flag;
        } else if (fuse) {
            const int rc = moe_launch_sort(fuse->topk_ids, T, fuse->k, E, fuse->offsets, fuse->sorted_tok,
                                           fuse->pair_pos, fuse->active, fuse->active_count, fuse->err_flag,
                                           stream);
            if (rc != MOE_NVFP4_OK) return rc;
        }
        const size_t plds = std::max(lds, (size_t)kHdrLds + setup);
        if (sort_here)
            hipLaunchKernelGGL((k_decode_row_persist<true, true>), dim3(nblk), dim3(kThreads), plds, stream, a);
        else
            hipLaunchKernelGGL((k_decode_row_persist<true, false>), dim3(nblk), dim3(kThreads), plds, stream, a);
        return moe_host::launch_status();
    }
    const int extra = c.extra;
    a.extra = extra;
    if (fuse) {
        if (gated && decode_sort_fuses(c, P)) {
            a.fused_sort = 1;
            a.P = P;
            a.topk = fuse->k;
            a.E = E;
            a.topk_ids = fuse->topk_ids;
            a.sort_offsets = fuse->offsets;
            a.sort_tok = fuse->sorted_tok;
            a.sort_pos = fuse->pair_pos;
            a.sort_active = fuse->active;
            a.sort_count = fuse->active_count;
            a.err_flag = fuse->err_flag;
        } else {
            const int rc = moe_launch_sort(fuse->topk_ids, T, fuse->k, E, fuse->offsets, fuse->sorted_tok,
                                           fuse->pair_pos, fuse->active, fuse->active_count, fuse->err_flag,
                                           stream);
            if (rc != MOE_NVFP4_OK) return rc;
        }
    }
    dim3 grid((unsigned)((a.units + G - 1) / G), (unsigned)(cap + extra));
    if (gated && a.fused_sort)
        hipLaunchKernelGGL((k_decode_row<true, true>), grid, dim3(kThreads), lds, stream, a);
    else if (gated)
        hipLaunchKernelGGL((k_decode_row<true, false>), grid, dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((k_decode_row<false, false>), grid, dim3(kThreads), lds, stream, a);
    return moe_host::launch_status();
}

// Down projection with the blend fused in (moe_nvfp4_down_blend): one block
// per (C output columns, token).  ELIMIT when k > 64, T > 65535, or the
// token's k activation rows do not fit the staging budget.
int moe_launch_down_blend(const float *h, const int32_t *topk_ids, const float *topk_weights,
                          const int32_t *pair_pos, const moe_nvfp4_experts &D, uint16_t *out, int N, int K, int T,
                          int k, int E, hipStream_t stream) {
    if (k > kBlendMaxK || T > 65535) return MOE_NVFP4_ELIMIT;
    DecArgs a = {};
    a.act = h;
    a.pa = D.packed;
    a.sa = D.scale;
    a.s2a = D.scale2;
    a.N = N;
    a.K = K;
    a.topk = k;
    a.E = E;
    a.topk_ids = topk_ids;
    a.blend_w = topk_weights;
    a.blend_pos = pair_pos;
    a.blend_out = out;
    const int pad_bytes = ((16 - (2 * K) % 256) + 256) % 256;
    a.ldx = K + pad_bytes / 2;
    const size_t rows_lds = (size_t)k * (size_t)a.ldx * 2;
    if (rows_lds > (size_t)kLdsBudget) return MOE_NVFP4_ELIMIT;
    // Columns per block: 8 G, G doubled (up to 4) while the grid still holds
    // two blocks per CU, so the h rows staged per block serve more weights.
    int G = 1;
    while (G < 4 && (int64_t)(N / (16 * G)) * T >= 2 * (int64_t)moe_host::cu_count()) G *= 2;
    a.G = G;
    const size_t lds = (size_t)kBlendHdrLds + rows_lds;
    hipLaunchKernelGGL(k_decode_down_blend, dim3((unsigned)(N / (8 * G)), (unsigned)T), dim3(kThreads), lds, stream,
                       a);
    return moe_host::launch_status();
}
