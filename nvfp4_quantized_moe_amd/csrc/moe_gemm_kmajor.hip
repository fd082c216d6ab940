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
//     160 = 10 MFMA row tiles), so every weight element is decoded once per
//     block and reused by every row tile; the 4 waves share the activation
//     tile, staged through LDS as bf16 (one barrier per 32-k step, two
//     buffers).  Gate+up: waves 0/1 hold gate columns, waves 2/3 the same up
//     columns; the up accumulators reach the gate waves through LDS in the
//     epilogue.
//   * An expert's rows are split into ceil(rows/160) balanced tiles.  Blocks
//     are dealt to the 8 XCDs in contiguous ranges of (row tile, column tile)
//     units, column tile fastest, so the blocks that share an activation tile
//     run on one XCD together; the ranges are cut from the true unit count,
//     read on the device, so every XCD gets an equal share.
//   * Weight dwords are prefetched kBDist steps ahead in registers, ring
//     refills are unconditional (clamped to the last step) so the compiler
//     keeps them in flight across iterations.
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
template <bool GATED>
struct Tile {
    static constexpr int kMaxRows = GATED ? 160 : 128;
    static constexpr int kMT = kMaxRows / 16;                        // MFMA row tiles
    static constexpr int kStage = kMaxRows * kRowBytes;              // one activation buffer
    static constexpr int kChunks = kMaxRows * 4;                     // 16-byte (8 k) chunks per step
    static constexpr int kSlots = (kChunks + kThreads - 1) / kThreads;
};
static_assert(kExRows * 128 * 4 <= 2 * Tile<true>::kStage, "exchange fits in the activation buffers");
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

// Decode 4 packed dwords (rows k/2 .. k/2+3 of columns 4c..4c+3) and their
// 4 E4M3 scales into the B operands of the 4 interleaved column tiles.
__device__ __forceinline__ void decode_b(const uint32_t (&w)[4], uint32_t s, bf16x8_t (&b)[4]) {
    const float sc[4] = {moe::e4m3_f32<0>(s), moe::e4m3_f32<1>(s), moe::e4m3_f32<2>(s), moe::e4m3_f32<3>(s)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[r], 1.0f, 0) * sc[0];
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[r], 1.0f, 1) * sc[1];
        const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[r], 1.0f, 2) * sc[2];
        const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[r], 1.0f, 3) * sc[3];
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
    constexpr int kChunks = Tile<GATED>::kChunks, kSlots = Tile<GATED>::kSlots;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
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
    const uint8_t *bp = pk + (size_t)(4 * q) * N + n_ld + 4 * c;
    const uint8_t *sp = sk + (size_t)(q >> 1) * N + n_ld + 4 * c;

    const int S = K / kBK;
    const int mt_used = (mrows + 15) >> 4;

    // ---- activation staging: chunk = 8 k of one row ----------------------
    const void *asrc[kSlots];
    int adst[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
        const int ch = tid + kThreads * j;
        const int row = ch >> 2, oct = ch & 3;
        const int rr = row < mrows ? row : 0;
        if constexpr (GATED)
            asrc[j] = static_cast<const uint16_t *>(a.act) + (size_t)a.sorted_tok[row0 + rr] * K + 8 * oct;
        else
            asrc[j] = static_cast<const float *>(a.act) + (row0 + rr) * K + 8 * oct;
        adst[j] = row * kRowBytes + 16 * oct;
    }
    // (kChunks need not fill the last slot: slot j is live for tid < kChunks - kThreads*j.)
    u32x4_t ar[kSlots][GATED ? 1 : 2];
    auto load_a = [&](int s) {
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (kThreads * j + kThreads <= kChunks || tid < kChunks - kThreads * j) {
                if constexpr (GATED) {
                    ar[j][0] = gload<u32x4_t>(static_cast<const uint16_t *>(asrc[j]) + kBK * s);
                } else {
                    const float *p = static_cast<const float *>(asrc[j]) + kBK * s;
                    ar[j][0] = gload<u32x4_t>(p);
                    ar[j][1] = gload<u32x4_t>(p + 4);
                }
            }
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (kThreads * j + kThreads <= kChunks || tid < kChunks - kThreads * j) {
                u32x4_t v;
                if constexpr (GATED)
                    v = ar[j][0];
                else
                    v = f32x8_to_bf16x8(ar[j][0], ar[j][1]);
                *reinterpret_cast<u32x4_t *>(lds + buf * kStage + adst[j]) = v;
            }
        }
    };

    // ---- weight ring --------------------------------------------------------
    uint32_t bw[kBDist][4];
    uint32_t bs[kBDist];
    auto load_b = [&](int slot_s, uint32_t (&w)[4], uint32_t &sv) {
        const int s = slot_s < S ? slot_s : S - 1;
        const uint8_t *p = bp + (size_t)(16 * s) * N;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = gload<uint32_t>(p + (size_t)r * N);
        sv = gload<uint32_t>(sp + (size_t)(2 * s) * N);
    };

    f32x4_t acc[kMT][4];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int d = 0; d < kBDist; ++d) load_b(d, bw[d], bs[d]);
    load_a(0);
    store_a(0);
    __syncthreads();

    const uint8_t *abase = lds + c * kRowBytes + 16 * q;

    auto step = [&](int s, auto slot) {
        constexpr int d = decltype(slot)::value;
        const int buf = s & 1;
        const bool more = s + 1 < S;
        if (more) load_a(s + 1);
        bf16x8_t bop[4];
        decode_b(bw[d], bs[d], bop);
        load_b(s + kBDist, bw[d], bs[d]);
        const uint8_t *ab = abase + buf * kStage;
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            if (i < mt_used) {
                const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(ab + i * 16 * kRowBytes);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bop[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) store_a(buf ^ 1);
        __syncthreads();
    };

    int s0 = 0;
    for (; s0 + kBDist <= S; s0 += kBDist) {
        step(s0 + 0, std::integral_constant<int, 0>{});
        step(s0 + 1, std::integral_constant<int, 1>{});
        step(s0 + 2, std::integral_constant<int, 2>{});
        step(s0 + 3, std::integral_constant<int, 3>{});
    }
    static_assert(kBDist == 4, "the step loop is unrolled by the ring depth");
    if (s0 + 0 < S) step(s0 + 0, std::integral_constant<int, 0>{});
    if (s0 + 1 < S) step(s0 + 1, std::integral_constant<int, 1>{});
    if (s0 + 2 < S) step(s0 + 2, std::integral_constant<int, 2>{});

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
