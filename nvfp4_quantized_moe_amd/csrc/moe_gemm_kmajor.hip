// Many-token path: grouped NVFP4 GEMM on the matrix cores, reading the
// K-major transposed twin of each expert weight (packed [K/2, N], scales
// [K/16, N]; transpose.rs, transpose_for_gemm, and prefill_weights.rs,
// prepare_prefill_weights, which builds these twins for the sorted prefill
// path).  Same operation as the decode GEMV: gate+up with the fused SiLU
// product (h fp32 [P, I]) or down (y fp32 [P, H]) over each active expert's
// sorted rows.
//
// gfx950 mapping:
//   * v_mfma_f32_16x16x32_bf16: the activation rows are the A operand, the
//     decoded weights the B operand, fp32 accumulation.  bf16 holds every
//     E2M1 x E4M3 product exactly (at most 6 significant bits) and x as given;
//     h is rounded to bf16 when staged for the down projection.
//   * The weights never pass through LDS.  In the K-major layout one dword
//     at packed row k/2 covers 4 adjacent columns x 2 k, so a lane that loads
//     the dwords of 4 consecutive packed rows holds 8 consecutive k of 4
//     columns: exactly the B operand (8 k of one column) of 4 MFMAs whose
//     columns are interleaved by 4.  Lane (c = lane%16, q = lane/16) owns
//     columns 4c..4c+3 of the wave's 64 and k-octet q of each 32-k step.
//   * Each wave owns 64 weight columns and all rows of the block tile (up to
//     144 rows = 9 MFMA row tiles for gate+up, 128 for down), so every weight
//     element is decoded once per block and reused by every row tile; the 4
//     waves share the activation tile, staged through LDS as bf16 with one
//     barrier per 32-k step.  Gate+up: waves 0/1 hold gate columns, waves 2/3
//     the same up columns; the up accumulators reach the gate waves through
//     LDS in the epilogue.
//   * Gate+up stages x with direct global-to-LDS loads three steps ahead
//     (no registers); down converts fp32 h to bf16 in registers one step
//     ahead.
//   * An expert's rows are split into balanced tiles.  Blocks are dealt to
//     the 8 XCDs in contiguous ranges of (row tile, column tile) units,
//     column tile fastest, so the blocks that share an activation tile run on
//     one XCD together; the ranges are cut from the true unit count, read on
//     the device, so every XCD gets an equal share.
//   * Weight dwords are prefetched kBDist steps ahead in registers; ring
//     refills are unconditional (clamped to the last step) so the compiler
//     keeps them in flight across iterations.  Within a step the next step's
//     weights are decoded between this step's MFMAs.
#include <type_traits>

#include "moe_common.hpp"

namespace {

using moe::gload;
using moe::u32x4_t;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr int kThreads = 256;
constexpr int kBK = 32;                          // k per step
constexpr int kRowBytes = 80;                    // LDS bytes per staged row: 32 bf16 + 16 padding
constexpr int kBDist = 4;                        // weight prefetch distance, in steps
constexpr int kExRows = 48;                      // epilogue exchange: rows per round

// Rows per block tile.  Down stages fp32 h through registers (twice the
// registers of the bf16 x chunks), so its tile is two MFMA row tiles shorter
// to stay within 256 registers at two waves per SIMD.
//
// Gate+up stages x with direct global-to-LDS loads (no registers) into a ring
// of kAStages buffers of unpadded 64-byte rows whose 16-byte octets are
// XOR-swizzled by row (conflict-free operand reads); down converts fp32 h to
// bf16 in registers and stages it into two padded buffers.
template <bool GATED>
struct Tile {
    static constexpr int kMaxRows = GATED ? 144 : 128;
    static constexpr int kMT = kMaxRows / 16;                        // MFMA row tiles
    static constexpr int kRow = GATED ? 64 : kRowBytes;              // LDS bytes per staged row
    static constexpr int kAStages = GATED ? 4 : 2;
    static constexpr int kStage = kMaxRows * kRow;                   // one activation buffer
    static constexpr int kChunks = kMaxRows * 4;                     // 16-byte (8 k) chunks per step
    static constexpr int kSlots = (kChunks + kThreads - 1) / kThreads;
    static constexpr int kDma = kChunks / 64;                        // wave-wide direct loads per step
};
static_assert(Tile<true>::kChunks % 64 == 0, "whole wave-wide direct loads");

// s_waitcnt immediate that waits until at most n vector-memory loads of this
// wave are outstanding (vmcnt in bits 3:0 and 15:14; LDS/scalar and export
// counters left at their maxima, i.e. not waited for).
constexpr int waitcnt_vm(int n) { return (((n >> 4) & 3) << 14) | 0x0F70 | (n & 15); }

// Workgroup barrier without the release fence of __syncthreads: that fence
// would wait for every outstanding load (the direct loads into LDS count as
// outstanding stores), emptying the prefetch ring at every step.  The caller
// waits for the direct loads the other waves need by count; LDS reads and
// writes of this wave are complete once their results were used or their
// counter was waited for, which the compiler does before the MFMAs that use
// them and the asm fences keep memory operations on their side.
__device__ __forceinline__ void block_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Swizzle of the 16-byte octet of staged row r: conflict-free operand reads
// whether the LDS serves 16 lanes x 16 bytes per cycle (64 banks) or 8 lanes
// (32 banks).
__device__ __forceinline__ int octet_swizzle(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
static_assert(kExRows % 16 == 0, "exchange rounds cover whole row tiles");

struct GemmArgs {
    const void *act;              // gate+up: bf16 x [T, K]; down: fp32 h [P, K]
    const int32_t *sorted_tok;
    const int32_t *offsets;
    const int32_t *active;
    const int32_t *nactive;
    const uint8_t *const *pa;
    const uint8_t *const *sa;
    const float *s2a;
    const uint8_t *const *pb;
    const uint8_t *const *sb;
    const float *s2b;
    float *out;
    int N, K;
    int n_ct;      // column tiles
};

// E4M3 block scales of the 4 columns in a scale dword.
struct Scales4 {
    float v[4];
};
__device__ __forceinline__ Scales4 scales4(uint32_t s) {
    return Scales4{{moe::e4m3_f32<0>(s), moe::e4m3_f32<1>(s), moe::e4m3_f32<2>(s), moe::e4m3_f32<3>(s)}};
}

// Decode packed row r (one dword: columns 4c..4c+3, k pair 2r, 2r+1 of the
// lane's octet) into element pair r of the B operands of the 4 interleaved
// column tiles.
__device__ __forceinline__ void decode_row(uint32_t w, const Scales4 &sc, int r, bf16x8_t (&b)[4]) {
    const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0) * sc.v[0];
    const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1) * sc.v[1];
    const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2) * sc.v[2];
    const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3) * sc.v[3];
    const bf16x2_t p0 = __builtin_convertvector(v0, bf16x2_t);
    const bf16x2_t p1 = __builtin_convertvector(v1, bf16x2_t);
    const bf16x2_t p2 = __builtin_convertvector(v2, bf16x2_t);
    const bf16x2_t p3 = __builtin_convertvector(v3, bf16x2_t);
    b[0][2 * r] = p0.x;
    b[0][2 * r + 1] = p0.y;
    b[1][2 * r] = p1.x;
    b[1][2 * r + 1] = p1.y;
    b[2][2 * r] = p2.x;
    b[2][2 * r + 1] = p2.y;
    b[3][2 * r] = p3.x;
    b[3][2 * r + 1] = p3.y;
}

// One element pair u = 4r + j: packed row r, column 4c+j (byte j).  Called
// from fully unrolled loops, where u folds to a constant.
template <int J>
__device__ __forceinline__ bf16x2_t decode_pair(uint32_t w, float sc) {
    return __builtin_convertvector(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J) * sc, bf16x2_t);
}
__device__ __forceinline__ void decode_pair_at(int u, const uint32_t (&w)[4], const Scales4 &sc, bf16x8_t (&b)[4]) {
    const int r = u >> 2, j = u & 3;
    bf16x2_t pr;
    switch (j) {
        case 0: pr = decode_pair<0>(w[r], sc.v[0]); break;
        case 1: pr = decode_pair<1>(w[r], sc.v[1]); break;
        case 2: pr = decode_pair<2>(w[r], sc.v[2]); break;
        default: pr = decode_pair<3>(w[r], sc.v[3]); break;
    }
    b[j][2 * r] = pr.x;
    b[j][2 * r + 1] = pr.y;
}

// All 4 packed rows of a step (8 consecutive k of columns 4c..4c+3).
__device__ __forceinline__ void decode_b(const uint32_t (&w)[4], uint32_t s, bf16x8_t (&b)[4]) {
    const Scales4 sc = scales4(s);
#pragma unroll
    for (int r = 0; r < 4; ++r) decode_row(w[r], sc, r, b);
}

__device__ __forceinline__ u32x4_t f32x8_to_bf16x8(u32x4_t a, u32x4_t b) {
    const f32x2_t v0 = {__uint_as_float(a.x), __uint_as_float(a.y)};
    const f32x2_t v1 = {__uint_as_float(a.z), __uint_as_float(a.w)};
    const f32x2_t v2 = {__uint_as_float(b.x), __uint_as_float(b.y)};
    const f32x2_t v3 = {__uint_as_float(b.z), __uint_as_float(b.w)};
    u32x4_t r;
    r.x = moe::bitcast<uint32_t>(__builtin_convertvector(v0, bf16x2_t));
    r.y = moe::bitcast<uint32_t>(__builtin_convertvector(v1, bf16x2_t));
    r.z = moe::bitcast<uint32_t>(__builtin_convertvector(v2, bf16x2_t));
    r.w = moe::bitcast<uint32_t>(__builtin_convertvector(v3, bf16x2_t));
    return r;
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_kmajor(GemmArgs a) {
    constexpr int kMaxRows = Tile<GATED>::kMaxRows, kMT = Tile<GATED>::kMT, kStage = Tile<GATED>::kStage;
    constexpr int kChunks = Tile<GATED>::kChunks, kSlots = Tile<GATED>::kSlots, kRow = Tile<GATED>::kRow;
    constexpr int kAStages = Tile<GATED>::kAStages;
    constexpr int kLds = GATED && kExRows * 128 * 4 > kAStages * kStage ? kExRows * 128 * 4 : kAStages * kStage;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    auto tiles_of = [](int rows) { return (rows + kMaxRows - 1) / kMaxRows; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::wave_id();

    // ---- which unit: count the row tiles, then cut per-XCD ranges --------
    const int nact = *a.nactive;
    int total = 0;
    for (int base = 0; base < nact; base += 64) {
        const int idx = base + lane;
        int t = 0;
        if (idx < nact) {
            const int ee = a.active[idx];
            t = tiles_of(a.offsets[ee + 1] - a.offsets[ee]);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
        total += t;
    }
    const int units = total * a.n_ct;
    const int per_xcd = (units + 7) >> 3;
    const int local = blockIdx.x >> 3;
    const int unit = (blockIdx.x & 7) * per_xcd + local;
    if (local >= per_xcd || unit >= units) return;  // uniform exit
    const int mt = unit / a.n_ct, ct = unit - mt * a.n_ct;

    int e = -1, lo = 0, m0 = 0, mrows = 0;
    int seen = 0;
    for (int base = 0; base < nact; base += 64) {
        const int idx = base + lane;
        int ee = 0, l = 0, r = 0;
        if (idx < nact) {
            ee = a.active[idx];
            l = a.offsets[ee];
            r = a.offsets[ee + 1] - l;
        }
        const int tiles = tiles_of(r);
        int incl = tiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        const unsigned long long hit = __ballot(idx < nact && mt < seen + incl);
        if (hit) {
            const int f = __ffsll((long long)hit) - 1;
            const int excl = __shfl(incl - tiles, f, 64);
            e = __shfl(ee, f, 64);
            lo = __shfl(l, f, 64);
            const int rows = __shfl(r, f, 64);
            const int nt = __shfl(tiles, f, 64);
            const int t = mt - seen - excl;
            m0 = (int)((long long)t * rows / nt);
            mrows = (int)((long long)(t + 1) * rows / nt) - m0;
            break;
        }
        seen += __shfl(incl, 63, 64);
    }
    e = __builtin_amdgcn_readfirstlane(e);
    if (e < 0) return;  // uniform
    lo = __builtin_amdgcn_readfirstlane(lo);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mrows = __builtin_amdgcn_readfirstlane(mrows);

    const int N = a.N, K = a.K;
    const int c = lane & 15, q = lane >> 4;
    const int n0 = ct * (GATED ? 128 : 256);
    const int n_w = n0 + 64 * (GATED ? (wave & 1) : wave);  // this wave's first weight column
    const bool wact = n_w < N;
    const size_t row0 = (size_t)lo + m0;

    const uint8_t *pA = a.pa[e];
    const uint8_t *pB = GATED ? a.pb[e] : pA;
    if (pA == nullptr || pB == nullptr) {  // absent expert: its rows are zero
        const int cols = GATED ? 128 : 256;
        for (int i = tid; i < mrows * cols; i += kThreads) {
            const int r = i / cols, cc = n0 + (i - r * cols);
            if (cc < N) a.out[(row0 + r) * N + cc] = 0.f;
        }
        return;
    }
    const bool up_wave = GATED && wave >= 2;
    const uint8_t *pk = up_wave ? pB : pA;
    const uint8_t *sk = up_wave ? a.sb[e] : a.sa[e];
    const int n_ld = wact ? n_w : N - 64;  // idle waves (N not a multiple of the tile) read valid columns
    // Per-lane byte offsets (32-bit) from wave-uniform bases, so that loads
    // take the scalar-base + vector-offset form.
    const uint32_t boff = (uint32_t)(4 * q) * N + n_ld + 4 * c;
    const uint32_t soff = (uint32_t)(q >> 1) * N + n_ld + 4 * c;

    const int S = K / kBK;
    const int mt_used = (mrows + 15) >> 4;

    // ---- activation staging: chunk = 8 k of one row ----------------------
    // Byte offsets of each chunk in x (gate+up, gathered by token) or in h
    // (down, sorted order); the host bounds both tensors below 4 GiB.
    const uint8_t *abytes = static_cast<const uint8_t *>(a.act);
    // Gate+up: direct loads.  Wave w issues load slots g = w, w+4, w+8, ...
    // (g < kDma); lane l of slot g writes LDS bytes [16 (64 g + l), +16),
    // i.e. staged row (64 g + l) / 4 and physical octet l % 4, so it fetches
    // the logical octet that the swizzle places there.
    constexpr int kDma = Tile<GATED>::kDma;
    constexpr int kDmaPerWave = (kDma + 3) / 4;
    uint32_t doff[kDmaPerWave];
    // Down: register staging, chunk slots j (thread tid + 256 j).
    uint32_t aoff[kSlots];
    int adst[kSlots];
    if constexpr (GATED) {
#pragma unroll
        for (int t = 0; t < kDmaPerWave; ++t) {
            const int g = wave + 4 * t < kDma ? wave + 4 * t : kDma - 1;
            const int u = 64 * g + lane;
            const int row = u >> 2, oct = (u & 3) ^ octet_swizzle(row);
            const int rr = row < mrows ? row : 0;
            doff[t] = ((uint32_t)a.sorted_tok[row0 + rr] * (uint32_t)K + 8 * oct) * 2u;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const int ch = tid + kThreads * j;
            const int row = ch >> 2, oct = ch & 3;
            const int rr = row < mrows ? row : 0;
            aoff[j] = ((uint32_t)(row0 + rr) * (uint32_t)K + 8 * oct) * 4u;
            adst[j] = row * kRow + 16 * oct;
        }
    }
    // Gate+up: issue step s into ring buffer st (clamped past the last step).
    auto dma_a = [&](int s, int st) {
        const int sc_ = s < S ? s : S - 1;
        const uint8_t *base = abytes + (size_t)sc_ * kBK * 2;
#pragma unroll
        for (int t = 0; t < kDmaPerWave; ++t) {
            if (t < kDmaPerWave - 1 || wave + 4 * t < kDma) {
                const int g = wave + 4 * t;
                __builtin_amdgcn_global_load_lds(
                    (const MOE_GLOBAL void *)(base + doff[t]),
                    (__attribute__((address_space(3))) void *)(lds + st * kStage + 1024 * g), 16, 0, 0);
            }
        }
    };
    // (kChunks need not fill the last slot: slot j is live for tid < kChunks - kThreads*j.)
    u32x4_t ar[kSlots][2];
    auto load_a = [&](int s) {
        const uint8_t *base = abytes + (size_t)s * kBK * 4;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (kThreads * j + kThreads <= kChunks || tid < kChunks - kThreads * j) {
                ar[j][0] = gload<u32x4_t>(base + aoff[j]);
                ar[j][1] = gload<u32x4_t>(base + aoff[j] + 16);
            }
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (kThreads * j + kThreads <= kChunks || tid < kChunks - kThreads * j)
                *reinterpret_cast<u32x4_t *>(lds + buf * kStage + adst[j]) = f32x8_to_bf16x8(ar[j][0], ar[j][1]);
        }
    };

    // ---- weight ring --------------------------------------------------------
    uint32_t bw[kBDist][4];
    uint32_t bs[kBDist];
    auto load_b = [&](int slot_s, uint32_t (&w)[4], uint32_t &sv) {
        const int s = slot_s < S ? slot_s : S - 1;
        const uint8_t *p = pk + (size_t)(16 * s) * N;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = gload<uint32_t>(p + (size_t)r * N + boff);
        sv = gload<uint32_t>(sk + (size_t)(2 * s) * N + soff);
    };

    f32x4_t acc[kMT][4];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // B operands of the current step and of the next one (decoded while the
    // current step's MFMAs run).
    bf16x8_t bop[2][4];
#pragma unroll
    for (int d = 0; d < kBDist; ++d) load_b(d, bw[d], bs[d]);
    decode_b(bw[0], bs[0], bop[0]);
    load_b(kBDist, bw[0], bs[0]);
    if constexpr (GATED) {
        static_assert(kAStages == 4 && kBDist == 4, "the wait counts below assume these depths");
        dma_a(0, 0);
        dma_a(1, 1);
        dma_a(2, 2);
        // Direct loads are waited for by count.  Step 0's landed once at
        // most the newer ones (steps 1 and 2: 2 or 3 loads each) are
        // outstanding; counting 2 per step is exact for waves 1-3 and
        // stricter than needed for wave 0.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        block_barrier();
    } else {
        load_a(0);
        store_a(0);
        __syncthreads();
    }

    // Lane's operand offset in a staged buffer: row c of each 16-row tile, octet q.
    const uint8_t *abase = GATED ? lds + c * kRow + 16 * (q ^ octet_swizzle(c)) : lds + c * kRow + 16 * q;

    // Step s: slot s % kBDist of the ring was decoded into bop[s % 2] during
    // step s - 1; this step decodes step s + 1 and refills its slot with step
    // s + 1 + kBDist.  Every row tile runs (rows past the tile's end compute
    // values that are never stored), so one basic block holds the MFMAs, the
    // pipelined operand reads and the decode, and the scheduler can
    // interleave them.
    auto step = [&](int s, auto slot) {
        constexpr int d = decltype(slot)::value;
        constexpr int p = d & 1;
        constexpr int dn = (d + 1) % kBDist;
        const bool more = s + 1 < S;
        constexpr int st = GATED ? d % kAStages : p;  // buffer read by this step
        if constexpr (GATED)
            dma_a(s + 3, (d + 3) % kAStages);
        else if (more)
            load_a(s + 1);
        const uint8_t *ab = abase + st * kStage;
        const Scales4 scn = scales4(bs[dn]);
        // Hand-ordered: row-tile operands are read two tiles ahead, and one
        // element pair of the next step's decode (4 VALU) follows every other
        // MFMA, so that it issues in the matrix pipe's shadow.  Full
        // scheduling fences keep this order; the empty asm after each decoded
        // pair pins it there (otherwise it is sunk to its use in the next
        // step).
        bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(ab);
        bf16x8_t an = *reinterpret_cast<const bf16x8_t *>(ab + 16 * kRow);
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            const bf16x8_t an2 = *reinterpret_cast<const bf16x8_t *>(ab + (i + 2 < kMT ? i + 2 : kMT - 1) * 16 * kRow);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[p][j], acc[i][j], 0, 0, 0);
                const int m = 4 * i + j;  // MFMA index in the step
                if ((m & 1) == 0 && m / 2 < 16) {
                    decode_pair_at(m / 2, bw[dn], scn, bop[p ^ 1]);
                    asm volatile("" : "+v"(bop[p ^ 1][0]), "+v"(bop[p ^ 1][1]), "+v"(bop[p ^ 1][2]), "+v"(bop[p ^ 1][3]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            av = an;
            an = an2;
        }
        load_b(s + 1 + kBDist, bw[dn], bs[dn]);
        if constexpr (GATED) {
            // Step s + 1's direct loads must have landed before the barrier.
            // Loads issued after them (2 direct loads per step, 5 per
            // refill; the prologue issued steps 0-2 after its refill):
            //   s = 0:  step 2, then step 3 + refill            = 2 + 2 + 5
            //   s = 1:  steps 3, 4 and two refills              = 2 * (2 + 5)
            //   s >= 2: the refill after them, then two steps   = 5 + 2 * (2 + 5)
            if (s == 0)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
            else if (s == 1)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(14));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(19));
            block_barrier();
        } else {
            if (more) store_a(p ^ 1);
            __syncthreads();
        }
    };

    // The step loop is unrolled by the ring depth so that ring slots, B
    // operand parity and activation buffer are compile-time indices.
    static_assert(kBDist == 2 || kBDist == 4, "ring depth");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    int s0 = 0;
    for (; s0 + kBDist <= S; s0 += kBDist) {
        step(s0 + 0, I0{});
        step(s0 + 1, I1{});
        if constexpr (kBDist == 4) {
            step(s0 + 2, I2{});
            step(s0 + 3, I3{});
        }
    }
    if (s0 + 0 < S) step(s0 + 0, I0{});
    if constexpr (kBDist == 4) {
        if (s0 + 1 < S) step(s0 + 1, I1{});
        if (s0 + 2 < S) step(s0 + 2, I2{});
    }

    if constexpr (GATED) {
        // The last steps issued direct loads past the end (clamped repeats
        // that keep the wait counts uniform); drain them before the epilogue
        // reuses the buffers.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        block_barrier();
    }

    // ---- epilogue: acc[i][j][v] = C[row 16i + 4q + v][column n_w + 4c + j] ----
    float *out = a.out;
    if constexpr (!GATED) {
        if (!wact) return;
        const float s2 = a.s2a[e];
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            if (i < mt_used) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * i + 4 * q + v;
                    if (row < mrows) {
                        const float4 o = make_float4(acc[i][0][v] * s2, acc[i][1][v] * s2, acc[i][2][v] * s2,
                                                     acc[i][3][v] * s2);
                        *reinterpret_cast<float4 *>(out + (row0 + row) * N + n_w + 4 * c) = o;
                    }
                }
            }
        }
    } else {
        // Up waves hand u = s2u * acc to the gate waves through LDS, kExRows rows per round.
        const float s2g = a.s2a[e], s2u = a.s2b[e];
        float *ex = reinterpret_cast<float *>(lds);
        const int exc = 64 * (wave & 1) + 4 * c;  // column within the block's 128
#pragma unroll
        for (int i0 = 0; i0 < kMT; i0 += kExRows / 16) {
            if (i0 < mt_used) {
                if (up_wave) {
#pragma unroll
                    for (int i = i0; i < i0 + kExRows / 16 && i < kMT; ++i) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int rl = 16 * (i - i0) + 4 * q + v;
                            *reinterpret_cast<float4 *>(ex + rl * 128 + exc) =
                                make_float4(acc[i][0][v] * s2u, acc[i][1][v] * s2u, acc[i][2][v] * s2u,
                                            acc[i][3][v] * s2u);
                        }
                    }
                }
                __syncthreads();
                if (!up_wave && wact) {
#pragma unroll
                    for (int i = i0; i < i0 + kExRows / 16 && i < kMT; ++i) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int rl = 16 * (i - i0) + 4 * q + v;
                            const int row = 16 * i + 4 * q + v;
                            if (row < mrows) {
                                const float4 u = *reinterpret_cast<const float4 *>(ex + rl * 128 + exc);
                                float4 o;
                                o.x = moe::silu_f32(acc[i][0][v] * s2g) * u.x;
                                o.y = moe::silu_f32(acc[i][1][v] * s2g) * u.y;
                                o.z = moe::silu_f32(acc[i][2][v] * s2g) * u.z;
                                o.w = moe::silu_f32(acc[i][3][v] * s2g) * u.w;
                                *reinterpret_cast<float4 *>(out + (row0 + row) * N + n_w + 4 * c) = o;
                            }
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
}

}  // namespace

int moe_launch_gemm_kmajor(bool gated, const void *act, const int32_t *sorted_tok, const int32_t *offsets,
                           const int32_t *active, const int32_t *nactive, const moe_nvfp4_experts &A,
                           const moe_nvfp4_experts *B, float *out, int N, int K, int P, int E,
                           hipStream_t stream) {
    GemmArgs a;
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
    const int cols = gated ? 128 : 256;
    a.n_ct = (N + cols - 1) / cols;
    // Row tiles: sum over experts of ceil(rows / R) <= ceil(P / R) + min(E, P).
    const int rows = gated ? Tile<true>::kMaxRows : Tile<false>::kMaxRows;
    const int cap = E < P ? E : P;
    const long long mt_bound = (P + rows - 1) / rows + cap;
    const long long units = mt_bound * a.n_ct;
    const long long grid = ((units + 7) / 8) * 8;
    if (grid > 0x7fffffffLL) return MOE_NVFP4_ELIMIT;
    if (gated)
        hipLaunchKernelGGL(k_gemm_kmajor<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(k_gemm_kmajor<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return moe_host::launch_status();
}
