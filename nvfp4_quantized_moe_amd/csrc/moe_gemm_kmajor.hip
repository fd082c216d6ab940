// Many-token path: grouped NVFP4 GEMM on the matrix cores, reading the
// K-major transposed twin of each expert weight (packed [K/2, N], scales
// [K/16, N], or for MXFP4 experts E8M0 scales [K/32, N]; transpose.rs,
// transpose_for_gemm and transpose_for_gemm_gs, and prefill_weights.rs,
// prepare_prefill_weights, which builds these twins for the sorted prefill
// path).  Same operation as the decode GEMV: gate+up with the fused SiLU
// product (h fp32 [P, I]) or down (y fp32 [P, H]) over each active expert's
// sorted rows.
//
// gfx950 mapping:
//   * Matrix cores, fp32 accumulation: the activation rows are the A
//     operand, the decoded weights the B operand.  Gate+up runs
//     v_mfma_f32_16x16x32_bf16: bf16 holds every E2M1 x E4M3 (or E8M0)
//     product exactly and x as given.  Down runs v_mfma_f32_16x16x32_f16
//     with h as fp16 times a power of two per row (11 significant bits).
//   * In the K-major layout one dword at packed row k/2 covers 4 adjacent
//     columns x 2 k, so a lane holding the dwords of 4 consecutive packed rows
//     holds 8 consecutive k of 4 columns: exactly the B operand (8 k of one
//     column) of 4 MFMAs whose columns are interleaved by 4.  Lane
//     (c = lane%16, q = lane/16) owns columns 4c..4c+3 of its wave's 64 and
//     k-octet q of each 32-k step; decoding needs no cross-lane traffic.
//   * Each wave owns 64 weight columns and every row of the block tile, so
//     every weight element is decoded once per block and reused by every row
//     tile; the 4 waves share the activation tile, staged in LDS as bf16 with
//     one barrier per 32-k step.
//   * Gate+up (k_gemm_gate_up, up to 144 rows): waves 0/1 hold 128 gate
//     columns, waves 2/3 the same up columns, and the up accumulators reach
//     the gate waves through LDS for silu(g) * u.  x and the weights move
//     with direct global-to-LDS loads three steps ahead, so no registers hold
//     data in flight; each wave decodes its step's weights from LDS.
//   * Down (k_gemm_down, up to 128 rows, 256 output columns per block):
//     fp32 h is converted to scaled fp16 in registers one step ahead; the weights
//     stream through a register ring four steps deep, and the next step's
//     weights are decoded between this step's MFMAs.
//   * An expert's rows are split into balanced tiles.  Blocks are dealt to
//     the 8 XCDs in contiguous ranges of (row tile, column tile) units,
//     column tile fastest, so the blocks that share an activation tile run on
//     one XCD together; the ranges are cut from the true unit count, read on
//     the device, so every XCD gets an equal share.
#include <type_traits>

#include "moe_common.hpp"

namespace {

using moe::gload;
using moe::u32x4_t;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr int kThreads = 256;
constexpr int kBK = 32;     // k per step
constexpr int kBDist = 4;   // weight prefetch depth, in steps (ring stages)
using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using I2 = std::integral_constant<int, 2>;
using I3 = std::integral_constant<int, 3>;

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
    int ldb;       // row pitch of the K-major twins (packed and scale rows), bytes
    int up_off;    // > 0: concatenated gate||up twin, up columns at this byte offset
};

// ---------------------------------------------------------------------------
// Weight decode.  NVFP4: E2M1 pairs through the f32 converter (scale 1: the
// hardware applies only the scale's exponent), times the E4M3 block scale in
// f32, then rounded to bf16 (exact: at most 6 significant bits).  MXFP4: the
// E8M0 scale is a power of two, i.e. exactly the exponent the converter
// applies, so one instruction turns two E2M1 codes into scaled bf16 (exact
// up to the f32 range: E8M0 codes up to 252).
// ---------------------------------------------------------------------------
struct Scales4 {
    float v[4];
};
// Block scales of the 4 columns in a scale dword: E4M3 codes widened to f32,
// or E8M0 codes placed in the exponent field of an f32 (the converter reads
// that field alone, so code 0 gives 2^-127 and code 255 NaN, as E8M0 defines).
template <bool MX>
__device__ __forceinline__ Scales4 scales4(uint32_t s) {
    if constexpr (MX)
        return Scales4{{__uint_as_float((s & 0xffu) << 23), __uint_as_float(((s >> 8) & 0xffu) << 23),
                        __uint_as_float(((s >> 16) & 0xffu) << 23), __uint_as_float((s >> 24) << 23)}};
    else
        return Scales4{{moe::e4m3_f32<0>(s), moe::e4m3_f32<1>(s), moe::e4m3_f32<2>(s), moe::e4m3_f32<3>(s)}};
}

// One element pair u = 4r + j: packed row r, column 4c+j (byte j).  Called
// from fully unrolled loops, where u folds to a constant.
template <bool MX, int J>
__device__ __forceinline__ bf16x2_t decode_pair(uint32_t w, float sc) {
    if constexpr (MX)
        return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, J);
    else
        return __builtin_convertvector(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J) * sc, bf16x2_t);
}
// All 4 packed rows of a step (8 consecutive k of columns 4c..4c+3) into the
// B operands of the 4 interleaved column tiles.
template <bool MX>
__device__ __forceinline__ void decode_b(const uint32_t (&w)[4], uint32_t s, bf16x8_t (&b)[4]) {
    const Scales4 sc = scales4<MX>(s);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bf16x2_t p0 = decode_pair<MX, 0>(w[r], sc.v[0]);
        const bf16x2_t p1 = decode_pair<MX, 1>(w[r], sc.v[1]);
        const bf16x2_t p2 = decode_pair<MX, 2>(w[r], sc.v[2]);
        const bf16x2_t p3 = decode_pair<MX, 3>(w[r], sc.v[3]);
        b[0][2 * r] = p0.x;
        b[0][2 * r + 1] = p0.y;
        b[1][2 * r] = p1.x;
        b[1][2 * r + 1] = p1.y;
        b[2][2 * r] = p2.x;
        b[2][2 * r + 1] = p2.y;
        b[3][2 * r] = p3.x;
        b[3][2 * r + 1] = p3.y;
    }
}

using moe::waitcnt_vm;
// Workgroup barrier without the release fence of __syncthreads, so no
// outstanding load is drained: callers wait for the direct loads the other
// waves need by count (waitcnt_vm).
__device__ __forceinline__ void block_barrier() { moe::lds_barrier(); }

// Swizzle of the 16-byte octet of staged row r: conflict-free operand reads
// whether the LDS serves 16 lanes x 16 bytes per cycle (64 banks) or 8 lanes
// (32 banks).
__device__ __forceinline__ int octet_swizzle(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// ---------------------------------------------------------------------------
// Work split: the block's (row tile, column tile) unit.
// ---------------------------------------------------------------------------
struct Unit {
    int e, lo, m0, mrows, ct;
};

// Row tiles per expert: ceil(rows / kMaxRows), balanced.  Units are dealt to
// the XCDs in contiguous ranges (blocks go to XCDs round-robin).  Returns
// false, the same on every wave, if the block has no unit.
template <int kMaxRows>
__device__ bool find_unit(const GemmArgs &a, Unit &u) {
    const int lane = threadIdx.x & 63;
    auto tiles_of = [](int rows) { return (rows + kMaxRows - 1) / kMaxRows; };
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
    if (local >= per_xcd || unit >= units) return false;
    const int mt = unit / a.n_ct;
    const int ct = unit - mt * a.n_ct;

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
    u.e = __builtin_amdgcn_readfirstlane(e);
    u.lo = __builtin_amdgcn_readfirstlane(lo);
    u.m0 = __builtin_amdgcn_readfirstlane(m0);
    u.mrows = __builtin_amdgcn_readfirstlane(mrows);
    u.ct = __builtin_amdgcn_readfirstlane(ct);
    return u.e >= 0;
}

// Rows of an absent (NULL) expert are written as zeros.
__device__ void zero_rows(const GemmArgs &a, size_t row0, int mrows, int n0, int cols) {
    for (int i = threadIdx.x; i < mrows * cols; i += kThreads) {
        const int r = i / cols, cc = n0 + (i - r * cols);
        if (cc < a.N) a.out[(row0 + r) * a.N + cc] = 0.f;
    }
}

// ===========================================================================
// Gate+up.
// ===========================================================================
constexpr int kRowsG = 144;                  // rows per block tile
constexpr int kMTG = kRowsG / 16;            // MFMA row tiles
constexpr int kStageG = kRowsG * 64;         // activation buffer: unpadded 64-byte rows, swizzled octets
constexpr int kDmaG = kRowsG * 4 / 64;       // wave-wide direct loads per activation step
constexpr int kDmaPerWaveG = (kDmaG + 3) / 4;
constexpr int kWStage = 4 * 1024 + 4 * 256;  // weight stage: 4 waves x (1 KiB packed), 4 x 256 B scales
constexpr int kExRows = 16;                  // epilogue exchange: rows per round
static_assert(kRowsG * 4 % 64 == 0, "whole wave-wide direct loads");
static_assert(kExRows * 128 * 4 <= kStageG, "exchange fits in one activation buffer");

template <bool MX>  // MXFP4 weights (E8M0 scales per 32 k) instead of NVFP4
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_gate_up(GemmArgs a) {
    // One LDS array per ring stage: alias analysis then tells the compiler's
    // wait insertion which direct loads an LDS read depends on (with one
    // array it would wait for all of them).  Activations sa*, weights sw*:
    // per wave 1 KiB of packed bytes (16 packed rows x 64 columns), then per
    // wave 256 bytes of scales (2 rows x 64 columns, stored twice).
    __shared__ __attribute__((aligned(16))) uint8_t sa0[kStageG], sa1[kStageG], sa2[kStageG], sa3[kStageG];
    __shared__ __attribute__((aligned(16))) uint8_t sw0[kWStage], sw1[kWStage], sw2[kWStage], sw3[kWStage];
    auto abuf = [&](auto st) -> uint8_t * {
        constexpr int v = decltype(st)::value;
        if constexpr (v == 0) return sa0;
        else if constexpr (v == 1) return sa1;
        else if constexpr (v == 2) return sa2;
        else return sa3;
    };
    auto wbuf = [&](auto st) -> uint8_t * {
        constexpr int v = decltype(st)::value;
        if constexpr (v == 0) return sw0;
        else if constexpr (v == 1) return sw1;
        else if constexpr (v == 2) return sw2;
        else return sw3;
    };

    Unit un;
    if (!find_unit<kRowsG>(a, un)) return;  // uniform exit
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::wave_id();
    const int N = a.N, K = a.K;
    const int c = lane & 15, q = lane >> 4;
    const int e = un.e, mrows = un.mrows;
    const int n0 = un.ct * 128;
    const int n_w = n0 + 64 * (wave & 1);  // this wave's first weight column
    const bool wact = n_w < N;
    const size_t row0 = (size_t)un.lo + un.m0;

    // Separate gate and up tables, or one concatenated twin whose up columns
    // start up_off bytes into each packed and scale row.
    // An expert whose packed or scale pointer is NULL is absent.
    const uint8_t *pA = a.pa[e];
    const uint8_t *sA = a.sa[e];
    const uint8_t *pB = a.up_off ? pA : a.pb[e];
    const uint8_t *sB = a.up_off ? sA : a.sb[e];
    if (pA == nullptr || pB == nullptr || sA == nullptr || sB == nullptr) {
        zero_rows(a, row0, mrows, n0, 128);
        return;
    }
    const bool up_wave = wave >= 2;
    const uint8_t *pk = up_wave ? pB + a.up_off : pA;
    const uint8_t *sk = up_wave ? sB + a.up_off : sA;
    const int ldb = a.ldb;
    const int n_ld = wact ? n_w : N - 64;  // idle waves (N not a multiple of 128) read valid columns
    const int S = K / kBK;
    const int mt_used = (mrows + 15) >> 4;

    // ---- activations: direct loads of x rows gathered by token ---------
    // Wave w issues load slots g = w, w+4, w+8 (g < kDmaG); lane l of slot g
    // writes LDS bytes [16 (64 g + l), +16), i.e. staged row (64 g + l) / 4
    // and physical octet l % 4, so it fetches the logical octet that the
    // swizzle places there.  Offsets are 32-bit (x below 4 GiB).
    const uint8_t *xbytes = static_cast<const uint8_t *>(a.act);
    uint32_t doff[kDmaPerWaveG];
#pragma unroll
    for (int t = 0; t < kDmaPerWaveG; ++t) {
        const int g = wave + 4 * t < kDmaG ? wave + 4 * t : kDmaG - 1;
        const int u = 64 * g + lane;
        const int row = u >> 2, oct = (u & 3) ^ octet_swizzle(row);
        const int rr = row < mrows ? row : 0;
        doff[t] = ((uint32_t)a.sorted_tok[row0 + rr] * (uint32_t)K + 8 * oct) * 2u;
    }
    auto dma_a = [&](int s, auto st) {  // step s (clamped past the end) into buffer st
        const int sc_ = s < S ? s : S - 1;
        const uint8_t *base = xbytes + (size_t)sc_ * kBK * 2;
#pragma unroll
        for (int t = 0; t < kDmaPerWaveG; ++t) {
            if (t < kDmaPerWaveG - 1 || wave + 4 * t < kDmaG)
                __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)(base + doff[t]),
                                                 (MOE_LDS void *)(abuf(st) + 1024 * (wave + 4 * t)), 16, 0, 0);
        }
    };

    // ---- weights: direct loads of this wave's 64 columns ----------------
    // Only the loading wave reads them back.  Packed: lane l loads 16 bytes
    // (16 columns) of packed row 16 s + 4 (t & 3) + (t >> 2), t = l >> 2,
    // chunk l & 3; it lands at byte 16 l, so row 4 q + r of the step sits at
    // byte 256 r + 64 q and the dword of columns 4c..4c+3 at + 4c: a lane's
    // four rows are 256 bytes apart and each read of 64 lanes touches 64
    // distinct banks.  Scales: lane l (mod 32) loads the dword of the step's
    // scale row (l >> 4) & 1 (NVFP4: two groups of 16 k; MXFP4: its one
    // group of 32 k, loaded twice), columns 4 (l & 15) .. +3.
    const int bt = lane >> 2;
    const uint32_t bdoff = (uint32_t)(4 * (bt & 3) + (bt >> 2)) * ldb + n_ld + 16 * (lane & 3);
    constexpr int kSRows = MX ? 1 : 2;  // scale rows per 32-k step
    const uint32_t sdoff = (uint32_t)(MX ? 0 : (lane >> 4) & 1) * ldb + n_ld + 4 * (lane & 15);
    auto dma_b = [&](int s, auto st) {
        const int sc_ = s < S ? s : S - 1;
        __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)(pk + (size_t)(16 * sc_) * ldb + bdoff),
                                         (MOE_LDS void *)(wbuf(st) + wave * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)(sk + (size_t)(kSRows * sc_) * ldb + sdoff),
                                         (MOE_LDS void *)(wbuf(st) + 4096 + wave * 256), 4, 0, 0);
    };
    const int brd = wave * 1024 + 64 * q + 4 * c, srd = 4096 + wave * 256 + 4 * (16 * (q >> 1) + c);
    auto read_b = [&](auto st, uint32_t (&w)[4], uint32_t &sv) {
        const uint8_t *b = wbuf(st) + brd;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = *reinterpret_cast<const uint32_t *>(b + 256 * r);
        sv = *reinterpret_cast<const uint32_t *>(wbuf(st) + srd);
    };

    f32x4_t acc[kMTG][4];
#pragma unroll
    for (int i = 0; i < kMTG; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t bop[4];
    uint32_t bw[4], bsv;

    // Every step issues, per wave, 2 activation direct loads (3 on wave 0)
    // and 2 weight loads, three steps ahead.  Before the barrier that ends
    // step s, step s + 1's loads must have landed: issued two steps back, so
    // at most 2 * (2 + 2) = 8 newer loads (stricter than needed on wave 0).
    // Decoding the next step's weights between this step's MFMAs (as the
    // down kernel does) measured slower here: the second set of B operands
    // costs 16 registers this kernel does not have.
    static_assert(kBDist == 4, "four ring stages");
    dma_a(0, I0{});
    dma_b(0, I0{});
    dma_a(1, I1{});
    dma_b(1, I1{});
    dma_a(2, I2{});
    dma_b(2, I2{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
    block_barrier();

    // Lane's operand offset in a staged buffer: row c of each 16-row tile, octet q.
    const int aoffs = c * 64 + 16 * (q ^ octet_swizzle(c));

    // Step s: issue step s + 3, decode this step's weights, run every row
    // tile (rows past the tile's end compute values that are never stored),
    // then wait for step s + 1 and meet at the barrier.
    auto step = [&](int s, auto slot) {
        constexpr int d = decltype(slot)::value;
        using Sn = std::integral_constant<int, (d + 3) % kBDist>;
        dma_a(s + 3, Sn{});
        dma_b(s + 3, Sn{});
        read_b(slot, bw, bsv);
        decode_b<MX>(bw, bsv, bop);
        const uint8_t *ab = abuf(slot) + aoffs;
        // Row-tile operands are read two tiles ahead.
        bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(ab);
        bf16x8_t an = *reinterpret_cast<const bf16x8_t *>(ab + 1024);
#pragma unroll
        for (int i = 0; i < kMTG; ++i) {
            const bf16x8_t an2 = *reinterpret_cast<const bf16x8_t *>(ab + (i + 2 < kMTG ? i + 2 : kMTG - 1) * 1024);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[j], acc[i][j], 0, 0, 0);
            av = an;
            an = an2;
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
        block_barrier();
    };
    int s0 = 0;
    for (; s0 + kBDist <= S; s0 += kBDist) {
        step(s0 + 0, I0{});
        step(s0 + 1, I1{});
        step(s0 + 2, I2{});
        step(s0 + 3, I3{});
    }
    if (s0 + 0 < S) step(s0 + 0, I0{});
    if (s0 + 1 < S) step(s0 + 1, I1{});
    if (s0 + 2 < S) step(s0 + 2, I2{});

    // The last steps issued loads past the end (clamped repeats that keep the
    // wait counts uniform); drain them before the exchange reuses sa0.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_barrier();

    // ---- epilogue: acc[i][j][v] = C[row 16i + 4q + v][column n_w + 4c + j].
    // Up waves hand u = s2u * acc to the gate waves through LDS.
    const float s2g = a.s2a[e], s2u = a.up_off ? s2g : a.s2b[e];
    float *ex = reinterpret_cast<float *>(sa0);
    const int exc = 64 * (wave & 1) + 4 * c;  // column within the block's 128
    constexpr int kExTiles = kExRows / 16;
#pragma unroll
    for (int i0 = 0; i0 < kMTG; i0 += kExTiles) {
        if (i0 < mt_used) {
            if (up_wave) {
#pragma unroll
                for (int i = i0; i < i0 + kExTiles && i < kMTG; ++i) {
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
                for (int i = i0; i < i0 + kExTiles && i < kMTG; ++i) {
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
                            *reinterpret_cast<float4 *>(a.out + (row0 + row) * N + n_w + 4 * c) = o;
                        }
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ===========================================================================
// Down.
//
// h (fp32) enters the matrix cores as fp16 times a power of two per row, the
// weights as fp16: v_mfma_f32_16x16x32_f16 runs at the bf16 rate, and fp16
// keeps 11 significant bits of h where bf16 keeps 8.
//   * Row exponents.  h streams in 32-k steps, so a row's largest magnitude
//     is not known when its first step is staged.  The exponent is set at
//     the row's first nonzero step so that the step's maximum lands in
//     [2^5, 2^6): every staged value then keeps 11 bits down to 2^-20 of
//     that maximum, and a later step may be up to 2^9 times larger before
//     it would reach 2^15.  If one is (the block's flag), the block runs
//     again with each row's exponent taken from its exact maximum, read in
//     a pass over the rows first; its first results are discarded.
//   * Weights.  NVFP4: an E2M1 x E4M3 product is an fp16 number (at most 6
//     significant bits, 2^-10 .. 2688): the fp4 converter, then one fp16
//     multiply.  MXFP4: E8M0 spans more than fp16's range, so each output
//     column is decoded relative to its largest scale code B (read once per
//     block): the converter applies 2^(code + 13 - B), exact for codes down
//     to B - 36 (a smaller one contributes under 2^-33 of the column's
//     largest term and may round away), and the epilogue multiplies by
//     2^(B - 140).  A column holding the NaN code 255 is NaN, as in the
//     plain definition.
// ===========================================================================
constexpr int kRowsD = 128;                // rows per block tile
constexpr int kMTD = kRowsD / 16;
constexpr int kRowD = 80;                  // LDS bytes per staged row: 32 fp16 + 16 padding
constexpr int kStageD = kRowsD * kRowD;
constexpr int kChunksD = kRowsD * 4;       // 16-byte (8 k) chunks per step
constexpr int kSlotsD = kChunksD / kThreads;
constexpr int kExpFirst = 5;               // first nonzero step: its maximum lands in [2^5, 2^6)
constexpr int kExpExact = 14;              // exact pass: the row maximum lands in [2^14, 2^15)
constexpr int kExpLimit = 14;              // a staged maximum must stay below 2^(kExpLimit + 1)
constexpr int kExpUnset = -1000;           // no nonzero value of the row seen yet
constexpr int kMxBias = 127 + 13;          // MXFP4: f32 exponent field of 2^13 (6 * 2^13 < 65504)
static_assert(kChunksD % kThreads == 0, "whole chunk slots");

struct DownLds {
    int efin[kRowsD];  // each row's exponent after the last step
    int redo;          // nonzero: a step exceeded its row's range; run again with exact exponents
};

__device__ __forceinline__ float absmax8(const u32x4_t &a, const u32x4_t &b) {
    const float u = fmaxf(fmaxf(fabsf(__uint_as_float(a.x)), fabsf(__uint_as_float(a.y))),
                          fmaxf(fabsf(__uint_as_float(a.z)), fabsf(__uint_as_float(a.w))));
    const float v = fmaxf(fmaxf(fabsf(__uint_as_float(b.x)), fabsf(__uint_as_float(b.y))),
                          fmaxf(fabsf(__uint_as_float(b.z)), fabsf(__uint_as_float(b.w))));
    return fmaxf(u, v);
}

// Largest magnitude over the quad of lanes holding one row's step (bits of
// a non-negative float); the binade field of a nonzero maximum, subnormals
// counted as the lowest normal binade, or 0 for an all-zero step.
__device__ __forceinline__ int quad_binade(const u32x4_t &a, const u32x4_t &b) {
    uint32_t m = __float_as_uint(absmax8(a, b));
    m = max(m, moe::dpp_u32<moe::kDppXor1>(m));
    m = max(m, moe::dpp_u32<moe::kDppXor2>(m));
    return m == 0u ? 0 : max((int)(m >> 23), 1);
}

// 8 fp32 values times 2^e -> 8 fp16 (round to nearest even).
__device__ __forceinline__ u32x4_t f32x8_to_f16x8(const u32x4_t &a, const u32x4_t &b, int e) {
    auto pk = [e](uint32_t x, uint32_t y) {
        const f32x2_t v = {__builtin_amdgcn_ldexpf(__uint_as_float(x), e), __builtin_amdgcn_ldexpf(__uint_as_float(y), e)};
        return moe::bitcast<uint32_t>(__builtin_convertvector(v, f16x2_t));
    };
    u32x4_t r;
    r.x = pk(a.x, a.y);
    r.y = pk(a.z, a.w);
    r.z = pk(b.x, b.y);
    r.w = pk(b.z, b.w);
    return r;
}

// fp16 scale operands of a step for the lane's 4 columns (bytes of a scale
// dword): NVFP4, the E4M3 value in both halves; MXFP4, the f32 whose
// exponent the converter applies, 2^(code + 13 - B), the field clamped to 1.
struct ScalesH {
    f16x2_t nv[4];
    float mx[4];
};
template <bool MX>
__device__ __forceinline__ ScalesH scales_h(uint32_t s, const int (&cbias)[4]) {
    ScalesH r;
    if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = (int)((s >> (8 * j)) & 0xffu) + cbias[j];
            r.mx[j] = __uint_as_float((uint32_t)(f < 1 ? 1 : f) << 23);
        }
    } else {
        const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
        const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
        r.nv[0] = f16x2_t{lo.x, lo.x};
        r.nv[1] = f16x2_t{lo.y, lo.y};
        r.nv[2] = f16x2_t{hi.x, hi.x};
        r.nv[3] = f16x2_t{hi.y, hi.y};
    }
    return r;
}

template <bool MX, int J>
__device__ __forceinline__ f16x2_t decode_pair_h(uint32_t w, const ScalesH &sc) {
    if constexpr (MX)
        return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.mx[J], J);
    else
        return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, J) * sc.nv[J];
}
// Element pair u = 4r + j (packed row r, column 4c + j) into the B operands.
template <bool MX>
__device__ __forceinline__ void decode_pair_h_at(int u, const uint32_t (&w)[4], const ScalesH &sc,
                                                 f16x8_t (&b)[4]) {
    const int r = u >> 2, j = u & 3;
    f16x2_t pr;
    switch (j) {
        case 0: pr = decode_pair_h<MX, 0>(w[r], sc); break;
        case 1: pr = decode_pair_h<MX, 1>(w[r], sc); break;
        case 2: pr = decode_pair_h<MX, 2>(w[r], sc); break;
        default: pr = decode_pair_h<MX, 3>(w[r], sc); break;
    }
    b[j][2 * r] = pr.x;
    b[j][2 * r + 1] = pr.y;
}
template <bool MX>
__device__ __forceinline__ void decode_b_h(const uint32_t (&w)[4], const ScalesH &sc, f16x8_t (&b)[4]) {
#pragma unroll
    for (int u = 0; u < 16; ++u) decode_pair_h_at<MX>(u, w, sc, b);
}

template <bool MX>  // MXFP4 weights (E8M0 scales per 32 k) instead of NVFP4
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_down(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageD];
    __shared__ __attribute__((aligned(16))) DownLds bk;

    Unit un;
    if (!find_unit<kRowsD>(a, un)) return;  // uniform exit
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = moe::wave_id();
    const int N = a.N, K = a.K;
    const int c = lane & 15, q = lane >> 4;
    const int e = un.e, mrows = un.mrows;
    const int n0 = un.ct * 256;
    const int n_w = n0 + 64 * wave;
    const bool wact = n_w < N;
    const size_t row0 = (size_t)un.lo + un.m0;

    const uint8_t *pk = a.pa[e];
    const uint8_t *sk = a.sa[e];
    if (pk == nullptr || sk == nullptr) {
        zero_rows(a, row0, mrows, n0, 256);
        return;
    }
    const int n_ld = wact ? n_w : N - 64;
    // Per-lane byte offsets (32-bit) from wave-uniform bases.
    const int ldb = a.ldb;
    const uint32_t boff = (uint32_t)(4 * q) * ldb + n_ld + 4 * c;
    // Scale row of k-octet q within a 32-k step: NVFP4 has two (groups of 16), MXFP4 one.
    constexpr int kSRows = MX ? 1 : 2;
    const uint32_t soff = (uint32_t)(MX ? 0 : q >> 1) * ldb + n_ld + 4 * c;
    const int S = K / kBK;
    const int mt_used = (mrows + 15) >> 4;

    if (tid == 0) bk.redo = 0;

    // MXFP4: the largest scale code B of each of the lane's 4 columns (the 4
    // lanes sharing them read every fourth scale row), kept as kMxBias - B.
    int cbias[4] = {0, 0, 0, 0};
    if constexpr (MX) {
        uint32_t m[4] = {0u, 0u, 0u, 0u};
        for (int r = q; r < S; r += 4) {
            const uint32_t d = gload<uint32_t>(sk + (size_t)r * ldb + n_ld + 4 * c);
            m[0] = max(m[0], d & 0xffu);
            m[1] = max(m[1], (d >> 8) & 0xffu);
            m[2] = max(m[2], (d >> 16) & 0xffu);
            m[3] = max(m[3], d >> 24);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[j] = max(m[j], (uint32_t)__shfl_xor((int)m[j], 16, 64));
            m[j] = max(m[j], (uint32_t)__shfl_xor((int)m[j], 32, 64));
            cbias[j] = kMxBias - (int)m[j];
        }
    }

    // ---- activations: fp32 h rows -> fp16 times 2^E(row), register staging
    // one step ahead.  Thread t stages octet t % 4 of rows t / 4 and
    // t / 4 + 64, so a row's 4 octets sit in one quad of lanes, each of which
    // keeps the row's exponent.
    const uint8_t *hbytes = static_cast<const uint8_t *>(a.act);
    const int srow = tid >> 2, soct = tid & 3;
    uint32_t aoff[kSlotsD];
#pragma unroll
    for (int j = 0; j < kSlotsD; ++j) {
        const int row = srow + (kThreads / 4) * j;
        const int rr = row < mrows ? row : 0;
        aoff[j] = ((uint32_t)(row0 + rr) * (uint32_t)K + 8 * soct) * 4u;  // h below 4 GiB
    }
    int ecur[kSlotsD];
    u32x4_t ar[kSlotsD][2];
    auto load_a = [&](int s) __attribute__((always_inline)) {
        const uint8_t *base = hbytes + (size_t)s * kBK * 4;
#pragma unroll
        for (int j = 0; j < kSlotsD; ++j) {
            ar[j][0] = gload<u32x4_t>(base + aoff[j]);
            ar[j][1] = gload<u32x4_t>(base + aoff[j] + 16);
        }
    };
    auto store_a = [&](int buf) __attribute__((always_inline)) {
        bool over = false;
#pragma unroll
        for (int j = 0; j < kSlotsD; ++j) {
            const int fe = quad_binade(ar[j][0], ar[j][1]);
            if (fe != 0 && ecur[j] == kExpUnset) ecur[j] = kExpFirst + 127 - fe;  // the accumulators are still zero
            over |= fe + ecur[j] > 127 + kExpLimit;
            *reinterpret_cast<u32x4_t *>(lds + buf * kStageD + (srow + (kThreads / 4) * j) * kRowD + 16 * soct) =
                f32x8_to_f16x8(ar[j][0], ar[j][1], ecur[j]);
        }
        if (over) bk.redo = 1;
    };

    // ---- weight ring in registers ---------------------------------------
    uint32_t bw[kBDist][4];
    uint32_t bs[kBDist];
    auto load_b = [&](int slot_s, uint32_t (&w)[4], uint32_t &sv) __attribute__((always_inline)) {
        const int s = slot_s < S ? slot_s : S - 1;
        const uint8_t *p = pk + (size_t)(16 * s) * ldb;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = gload<uint32_t>(p + (size_t)r * ldb + boff);
        sv = gload<uint32_t>(sk + (size_t)(kSRows * s) * ldb + soff);
    };

    f32x4_t acc[kMTD][4];
    f16x8_t bop[2][4];  // B operands of the current step and of the next one
    const uint8_t *abase = lds + c * kRowD + 16 * q;

    // Step s: ring slot s % kBDist was decoded into bop[s % 2] during step
    // s - 1; this step decodes step s + 1 and refills its slot with step
    // s + 1 + kBDist (unconditionally, clamped: the compiler then keeps the
    // ring in flight across iterations).  Every row tile runs.
    auto step = [&](int s, auto slot) __attribute__((always_inline)) {
        constexpr int d = decltype(slot)::value;
        constexpr int p = d & 1;
        constexpr int dn = (d + 1) % kBDist;
        const bool more = s + 1 < S;
        if (more) load_a(s + 1);
        const uint8_t *ab = abase + p * kStageD;
        const ScalesH scn = scales_h<MX>(bs[dn], cbias);
        // Hand-ordered: row-tile operands are read two tiles ahead, and one
        // element pair of the next step's decode follows every other MFMA.
        // Full scheduling fences keep this order; the empty asm after each
        // decoded pair pins it there (otherwise it is sunk to its use in the
        // next step).
        f16x8_t av = *reinterpret_cast<const f16x8_t *>(ab);
        f16x8_t an = *reinterpret_cast<const f16x8_t *>(ab + 16 * kRowD);
#pragma unroll
        for (int i = 0; i < kMTD; ++i) {
            const f16x8_t an2 = *reinterpret_cast<const f16x8_t *>(ab + (i + 2 < kMTD ? i + 2 : kMTD - 1) * 16 * kRowD);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bop[p][j], acc[i][j], 0, 0, 0);
                const int m = 4 * i + j;  // MFMA index in the step
                if ((m & 1) == 0 && m / 2 < 16) {
                    decode_pair_h_at<MX>(m / 2, bw[dn], scn, bop[p ^ 1]);
                    asm volatile("" : "+v"(bop[p ^ 1][0]), "+v"(bop[p ^ 1][1]), "+v"(bop[p ^ 1][2]), "+v"(bop[p ^ 1][3]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            av = an;
            an = an2;
        }
        load_b(s + 1 + kBDist, bw[dn], bs[dn]);
        if (more) store_a(p ^ 1);
        __syncthreads();
    };

    // The pipeline: each row's exponent from its first nonzero step (exact =
    // false) or from the rows' exact maxima, read in a pass first (exact =
    // true: used when a later step of some row exceeded its range).
    auto run = [&](bool exact) __attribute__((always_inline)) {
        if (!exact) {
#pragma unroll
            for (int j = 0; j < kSlotsD; ++j) ecur[j] = kExpUnset;
        } else {
            int fmax[kSlotsD];
#pragma unroll
            for (int j = 0; j < kSlotsD; ++j) fmax[j] = 0;
            for (int s = 0; s < S; ++s) {
                load_a(s);
#pragma unroll
                for (int j = 0; j < kSlotsD; ++j) fmax[j] = max(fmax[j], quad_binade(ar[j][0], ar[j][1]));
            }
#pragma unroll
            for (int j = 0; j < kSlotsD; ++j) ecur[j] = fmax[j] == 0 ? kExpUnset : kExpExact + 127 - fmax[j];
        }
#pragma unroll
        for (int i = 0; i < kMTD; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < kBDist; ++d) load_b(d, bw[d], bs[d]);
        load_a(0);
        __syncthreads();  // the redo flag is cleared; earlier readers of the stage buffers are done
        store_a(0);
        decode_b_h<MX>(bw[0], scales_h<MX>(bs[0], cbias), bop[0]);
        load_b(kBDist, bw[0], bs[0]);
        __syncthreads();

        int s0 = 0;
        for (; s0 + kBDist <= S; s0 += kBDist) {
            step(s0 + 0, I0{});
            step(s0 + 1, I1{});
            step(s0 + 2, I2{});
            step(s0 + 3, I3{});
        }
        if (s0 + 0 < S) step(s0 + 0, I0{});
        if (s0 + 1 < S) step(s0 + 1, I1{});
        if (s0 + 2 < S) step(s0 + 2, I2{});
    };
    run(false);
    // The last barrier follows every store_a, so the flag is final.  Exact
    // exponents cannot exceed the range: a second run always completes.
    if (__builtin_amdgcn_readfirstlane(bk.redo) != 0) run(true);

    // ---- epilogue: acc[i][j][v] = C[row 16i + 4q + v][column n_w + 4c + j],
    // scaled by 2^-E(row) (and 2^(B - 140) per MXFP4 column).
    if (soct == 0) {
#pragma unroll
        for (int j = 0; j < kSlotsD; ++j) bk.efin[srow + (kThreads / 4) * j] = ecur[j];
    }
    __syncthreads();
    if (!wact) return;
    const float s2 = a.s2a[e];
#pragma unroll
    for (int i = 0; i < kMTD; ++i) {
        if (i < mt_used) {
            const int4 ev = *reinterpret_cast<const int4 *>(&bk.efin[16 * i + 4 * q]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * i + 4 * q + v;
                if (row < mrows) {
                    const int er = v == 0 ? ev.x : (v == 1 ? ev.y : (v == 2 ? ev.z : ev.w));
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        o[j] = __builtin_amdgcn_ldexpf(acc[i][j][v], -er - cbias[j]) * s2;
                        if constexpr (MX) o[j] = cbias[j] == kMxBias - 255 ? __builtin_nanf("") : o[j];
                    }
                    *reinterpret_cast<float4 *>(a.out + (row0 + row) * N + n_w + 4 * c) =
                        make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

}  // namespace

int moe_launch_gemm_kmajor(bool gated, bool mx, const void *act, const int32_t *sorted_tok,
                           const int32_t *offsets, const int32_t *active, const int32_t *nactive,
                           const moe_nvfp4_experts &A, const moe_nvfp4_experts *B, float *out, int N, int K,
                           int P, int E, int ldb, int up_off, hipStream_t stream) {
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
    a.ldb = ldb;
    a.up_off = up_off;
    const int cols = gated ? 128 : 256;
    a.n_ct = (N + cols - 1) / cols;
    // Row tiles: sum over experts of ceil(rows / R) <= ceil(P / R) + min(E, P).
    const int rows = gated ? kRowsG : kRowsD;
    const int cap = E < P ? E : P;
    const long long mt_bound = (P + rows - 1) / rows + cap;
    const long long units = mt_bound * a.n_ct;
    const long long grid = ((units + 7) / 8) * 8;
    if (grid > 0x7fffffffLL) return MOE_NVFP4_ELIMIT;
    const dim3 g((unsigned)grid), b(kThreads);
    if (gated && mx)
        hipLaunchKernelGGL(k_gemm_gate_up<true>, g, b, 0, stream, a);
    else if (gated)
        hipLaunchKernelGGL(k_gemm_gate_up<false>, g, b, 0, stream, a);
    else if (mx)
        hipLaunchKernelGGL(k_gemm_down<true>, g, b, 0, stream, a);
    else
        hipLaunchKernelGGL(k_gemm_down<false>, g, b, 0, stream, a);
    return moe_host::launch_status();
}
