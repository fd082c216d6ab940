// Many-token path: grouped NVFP4 GEMM on the matrix cores, reading the
// K-major transposed twin of each expert weight (packed [K/2, N], scales
// [K/16, N]; transpose.rs, transpose_for_gemm, and prefill_weights.rs,
// prepare_prefill_weights, which builds these twins for the sorted prefill
// path).  Same operation as the decode GEMV: gate+up with the fused SiLU
// product (h fp32 [P, I]) or down (y fp32 [P, H]) over each active expert's
// sorted rows.
//
// gfx950 mapping:
//   * block tile = 64 sorted rows x 512 weight columns (gate+up: 256 gate and
//     the same 256 up columns; down: 512 columns); each of the 4 waves owns
//     64 rows x 128 weight columns = 2 x 4 MFMA 32x32x16 tiles (fp16 in,
//     fp32 accumulate);
//   * one block per (column tile, 64-row tile of an expert); a block finds its
//     expert from the device-side offsets, so the grid is sized from the
//     bound P/64 + min(E, P) on the number of row tiles;
//   * flat tile ids are dealt to the 8 XCDs in contiguous ranges, so the row
//     tiles that share a weight panel run on one XCD at about the same time
//     and the second read of the panel hits that XCD's L2;
//   * K advances 32 at a time: the next step's packed bytes, scales and
//     activation rows are loaded into registers while the matrix cores work
//     on the current step;
//   * weights are decoded once per block into LDS as fp16: E2M1 -> fp16 pairs
//     with the hardware converter, times the E4M3 block scale (exact in fp16:
//     at most 6 significant bits, range 2^-10 .. 2688), written N-major so the
//     MFMA operand is one 16-byte LDS read;
//   * activation rows are converted to fp16 while staged (x is gathered by
//     token id; h is read in sorted order).
#include "moe_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 64;       // rows per block
constexpr int kBK = 32;       // K per step
constexpr int kBCols = 512;   // weight columns per block (both matrices together)
constexpr int kRow = 40;      // halves per LDS row: 32 + 8 padding (conflict-free 16-byte reads)

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
    int mt_bound;   // row tiles per column tile in the grid
    int n_tiles;    // column tiles
};

__device__ __forceinline__ f16x8_t bf16x8_to_f16x8(uint4 v) {
    f16x8_t r;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16);
        const float hi = __uint_as_float(w[i] & 0xffff0000u);
        r[2 * i] = (_Float16)lo;
        r[2 * i + 1] = (_Float16)hi;
    }
    return r;
}

__device__ __forceinline__ f16x8_t f32x8_to_f16x8(float4 a, float4 b) {
    f16x8_t r;
    r[0] = (_Float16)a.x;
    r[1] = (_Float16)a.y;
    r[2] = (_Float16)a.z;
    r[3] = (_Float16)a.w;
    r[4] = (_Float16)b.x;
    r[5] = (_Float16)b.y;
    r[6] = (_Float16)b.z;
    r[7] = (_Float16)b.w;
    return r;
}

template <int B>
__device__ __forceinline__ f16x8_t decode_col(const uint32_t (&w)[8], int half, _Float16 s) {
    // Column B of rows 4*half .. 4*half+3 (k2 rows) -> 8 consecutive k, scaled.
    f16x8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2_t v = moe::e2m1x2_f16<B>(w[4 * half + i]) * s;
        r[2 * i] = v.x;
        r[2 * i + 1] = v.y;
    }
    return r;
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_gemm_kmajor(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 As[kBM * kRow];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[kBCols * kRow];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Flat tile id, dealt to XCDs in contiguous ranges (gridDim.x is a multiple of 8).
    const int per_xcd = gridDim.x >> 3;
    const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (tile >= a.n_tiles * a.mt_bound) return;
    const int ntile = tile / a.mt_bound, mt = tile - ntile * a.mt_bound;

    // Which expert owns row tile mt (prefix over ceil(rows_e / 64), active order).
    const int nact = *a.nactive;
    int e = -1, lo = 0, rows = 0, m0 = 0;
    int seen = 0;
    for (int base = 0; base < nact; base += 64) {
        const int idx = base + lane;
        int ee = 0, l = 0, h = 0;
        if (idx < nact) {
            ee = a.active[idx];
            l = a.offsets[ee];
            h = a.offsets[ee + 1];
        }
        const int tiles = (h - l + kBM - 1) / kBM;
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
            rows = __shfl(h - l, f, 64);
            m0 = (mt - seen - excl) * kBM;
            break;
        }
        seen += __shfl(incl, 63, 64);
    }
    if (e < 0) return;  // past the last row tile: uniform exit

    const int N = a.N, K = a.K;
    const int n0 = ntile * (GATED ? kBCols / 2 : kBCols);
    const int mrows = min(kBM, rows - m0);

    const uint8_t *pA = a.pa[e];
    const uint8_t *pB = GATED ? a.pb[e] : pA;
    const int wcols = GATED ? 64 : 128;  // output columns per wave
    const int wc0 = n0 + wave * wcols;
    if (pA == nullptr || pB == nullptr) {  // absent expert: zero rows
        for (int i = lane; i < mrows * wcols; i += 64) {
            const int r = i / wcols, c = wc0 + (i - r * wcols);
            if (c < N) a.out[(size_t)(lo + m0 + r) * N + c] = 0.f;
        }
        return;
    }
    const uint8_t *sA = a.sa[e];
    const uint8_t *sB = GATED ? a.sb[e] : sA;

    // ---- per-thread load assignment -------------------------------------
    // weights: 4 columns x 8 k2-rows (one 16-k scale group) per thread
    const int cb = tid & 127, g = tid >> 7;
    const bool upper = GATED && cb >= 64;
    const int bcol = GATED ? n0 + (cb & 63) * 4 : n0 + cb * 4;  // weight column in its matrix
    const bool bvalid = bcol < N;
    const uint8_t *bp = (upper ? pB : pA) + bcol;
    const uint8_t *bs = (upper ? sB : sA) + bcol;
    // activations: row am, 8 consecutive k at 8*apart
    const int am = tid >> 2, apart = tid & 3;
    const bool avalid = am < mrows;
    const void *arow = nullptr;
    if (avalid) {
        if constexpr (GATED)
            arow = static_cast<const uint16_t *>(a.act) + (size_t)a.sorted_tok[lo + m0 + am] * K + 8 * apart;
        else
            arow = static_cast<const float *>(a.act) + (size_t)(lo + m0 + am) * K + 8 * apart;
    }

    uint32_t wr[8];
    uint32_t sr = 0;
    uint4 ar0 = make_uint4(0, 0, 0, 0), ar1 = make_uint4(0, 0, 0, 0);
    auto load_step = [&](int k0) {
        if (bvalid) {
            const size_t r0 = (size_t)(k0 / 2 + 8 * g);
#pragma unroll
            for (int r = 0; r < 8; ++r) wr[r] = *reinterpret_cast<const uint32_t *>(bp + (r0 + r) * N);
            sr = *reinterpret_cast<const uint32_t *>(bs + (size_t)(k0 / 16 + g) * N);
        }
        if (avalid) {
            if constexpr (GATED) {
                ar0 = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(arow) + k0);
            } else {
                const float *p = static_cast<const float *>(arow) + k0;
                ar0 = *reinterpret_cast<const uint4 *>(p);
                ar1 = *reinterpret_cast<const uint4 *>(p + 4);
            }
        }
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Column offsets (in the 512-wide LDS panel) of this wave's 4 B sub-tiles.
    int bsub[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bsub[j] = GATED ? ((j >> 1) * 256 + wave * 64 + (j & 1) * 32) : (wave * 128 + j * 32);

    load_step(0);
    for (int k0 = 0; k0 < K; k0 += kBK) {
        __syncthreads();  // previous step's LDS reads are done
        {
            f16x8_t av;
            if (!avalid) {
#pragma unroll
                for (int i = 0; i < 8; ++i) av[i] = (_Float16)0.f;
            } else if constexpr (GATED) {
                av = bf16x8_to_f16x8(ar0);
            } else {
                av = f32x8_to_f16x8(moe::bitcast<float4>(ar0), moe::bitcast<float4>(ar1));
            }
            *reinterpret_cast<f16x8_t *>(&As[am * kRow + 8 * apart]) = av;
        }
        {
            _Float16 s[4];
            if (bvalid) {
                s[0] = (_Float16)moe::e4m3_f32<0>(sr);
                s[1] = (_Float16)moe::e4m3_f32<1>(sr);
                s[2] = (_Float16)moe::e4m3_f32<2>(sr);
                s[3] = (_Float16)moe::e4m3_f32<3>(sr);
            } else {
                s[0] = s[1] = s[2] = s[3] = (_Float16)0.f;
#pragma unroll
                for (int r = 0; r < 8; ++r) wr[r] = 0u;
            }
            _Float16 *bdst = &Bs[(cb * 4) * kRow + 16 * g];
            *reinterpret_cast<f16x8_t *>(bdst + 0 * kRow) = decode_col<0>(wr, 0, s[0]);
            *reinterpret_cast<f16x8_t *>(bdst + 0 * kRow + 8) = decode_col<0>(wr, 1, s[0]);
            *reinterpret_cast<f16x8_t *>(bdst + 1 * kRow) = decode_col<1>(wr, 0, s[1]);
            *reinterpret_cast<f16x8_t *>(bdst + 1 * kRow + 8) = decode_col<1>(wr, 1, s[1]);
            *reinterpret_cast<f16x8_t *>(bdst + 2 * kRow) = decode_col<2>(wr, 0, s[2]);
            *reinterpret_cast<f16x8_t *>(bdst + 2 * kRow + 8) = decode_col<2>(wr, 1, s[2]);
            *reinterpret_cast<f16x8_t *>(bdst + 3 * kRow) = decode_col<3>(wr, 0, s[3]);
            *reinterpret_cast<f16x8_t *>(bdst + 3 * kRow + 8) = decode_col<3>(wr, 1, s[3]);
        }
        __syncthreads();
        if (k0 + kBK < K) load_step(k0 + kBK);

#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            const int kk = ks + 8 * (lane >> 5);
            f16x8_t av[2], bv[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const f16x8_t *>(&As[(32 * i + (lane & 31)) * kRow + kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[j] = *reinterpret_cast<const f16x8_t *>(&Bs[(bsub[j] + (lane & 31)) * kRow + kk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue: C[row, col] of a 32x32 tile sits in lane (col + 32*((row/4)&1)),
    // register 4*(row/8) + row%4.
    const int ccol = lane & 31, rhalf = (lane >> 5) * 4;
    if constexpr (GATED) {
        const float s2g = a.s2a[e], s2u = a.s2b[e];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = n0 + wave * 64 + j * 32 + ccol;
                if (col >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + rhalf + (r & 3);
                    if (row < mrows) {
                        const float gv = acc[i][j][r] * s2g, uv = acc[i][j + 2][r] * s2u;
                        a.out[(size_t)(lo + m0 + row) * N + col] = moe::silu_f32(gv) * uv;
                    }
                }
            }
    } else {
        const float s2 = a.s2a[e];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wave * 128 + j * 32 + ccol;
                if (col >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + rhalf + (r & 3);
                    if (row < mrows) a.out[(size_t)(lo + m0 + row) * N + col] = acc[i][j][r] * s2;
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
    const int cap = E < P ? E : P;
    a.mt_bound = (P + kBM - 1) / kBM + cap;
    const int cols = gated ? kBCols / 2 : kBCols;
    a.n_tiles = (N + cols - 1) / cols;
    const long long tiles = (long long)a.mt_bound * a.n_tiles;
    const long long grid = ((tiles + 7) / 8) * 8;
    if (grid > 0x7fffffffLL) return MOE_NVFP4_ELIMIT;
    if (gated)
        hipLaunchKernelGGL(k_gemm_kmajor<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(k_gemm_kmajor<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return moe_host::launch_status();
}
