// Byte-matrix transpose dst[c * pitch + r] = src[r * cols + c] (pitch = rows
// for the plain transpose).
//
// transpose.rs, transpose_for_gemm_gs: the load-time twin of an NVFP4 weight
// is the byte transpose of its packed [N, K/2] and scale [N, K/16] tensors
// (nibble pairs stay together); transpose_concat_for_gemm_padded writes
// several such transposes side by side into one twin whose rows are `pitch`
// bytes apart.  HBM-bound copy: a 64x64-byte tile moves
// through LDS so both the read of src rows and the write of dst rows are
// 16-byte coalesced; ragged or unaligned edges fall back to byte accesses.
#include "moe_common.hpp"

namespace {

constexpr int kTile = 64;
constexpr int kTileStride = kTile + 4;  // padded LDS row (bytes)
constexpr int kTransposeThreads = 256;

__global__ __launch_bounds__(kTransposeThreads) void k_transpose_u8(const uint8_t *__restrict__ src,
                                                                   uint8_t *__restrict__ dst, int rows,
                                                                   int cols, int tiles_c, int64_t pitch) {
    __shared__ uint32_t tile_w[kTile * kTileStride / 4];
    uint8_t *tile = reinterpret_cast<uint8_t *>(tile_w);

    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int r0 = tr * kTile, c0 = tc * kTile;
    const int tid = threadIdx.x;
    const int a = tid >> 2;        // tile row (load) / tile column (store)
    const int seg = (tid & 3) * 16;  // 16-byte segment inside the tile line

    // Load: src row r0 + a, columns c0 + seg .. +16.
    {
        const int r = r0 + a, c = c0 + seg;
        uint8_t *t = tile + a * kTileStride + seg;
        if (r < rows) {
            const uint8_t *s = src + (size_t)r * cols + c;
            if (c + 16 <= cols && ((reinterpret_cast<uintptr_t>(s) & 15) == 0)) {
                const uint4 v = *reinterpret_cast<const uint4 *>(s);
                uint32_t *tw = reinterpret_cast<uint32_t *>(t);
                tw[0] = v.x;
                tw[1] = v.y;
                tw[2] = v.z;
                tw[3] = v.w;
            } else {
                for (int i = 0; i < 16; ++i) t[i] = (c + i < cols) ? s[i] : 0;
            }
        }
    }
    __syncthreads();
    // Store: dst row c0 + a (= src column), columns r0 + seg .. +16 (= src rows).
    {
        const int c = c0 + a, r = r0 + seg;
        if (c < cols && r < rows) {
            uint32_t wv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) v |= (uint32_t)tile[(seg + q * 4 + b) * kTileStride + a] << (8 * b);
                wv[q] = v;
            }
            uint8_t *d = dst + (size_t)c * (size_t)pitch + r;
            if (r + 16 <= rows && ((reinterpret_cast<uintptr_t>(d) & 15) == 0)) {
                *reinterpret_cast<uint4 *>(d) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            } else {
                for (int i = 0; i < 16 && r + i < rows; ++i) d[i] = (uint8_t)(wv[i >> 2] >> (8 * (i & 3)));
            }
        }
    }
}

int launch_transpose(const uint8_t *src, uint8_t *dst, int32_t rows, int32_t cols, int64_t pitch, void *stream) {
    if (!src || !dst) return MOE_NVFP4_ENULL;
    if (rows < 1 || cols < 1 || pitch < rows) return MOE_NVFP4_ESHAPE;
    if ((int64_t)rows * cols > (int64_t(1) << 40) || pitch * cols > (int64_t(1) << 40)) return MOE_NVFP4_ELIMIT;
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    if (tiles_r * tiles_c > 0x7fffffffLL) return MOE_NVFP4_ELIMIT;
    hipLaunchKernelGGL(k_transpose_u8, dim3((unsigned)(tiles_r * tiles_c)), dim3(kTransposeThreads), 0,
                       (hipStream_t)stream, src, dst, rows, cols, (int)tiles_c, pitch);
    return moe_host::launch_status();
}

}  // namespace

extern "C" int transpose_u8(const uint8_t *src, uint8_t *dst, int32_t rows, int32_t cols, void *stream) {
    return launch_transpose(src, dst, rows, cols, rows, stream);
}

extern "C" int transpose_u8_pitched(const uint8_t *src, uint8_t *dst, int32_t rows, int32_t cols,
                                    int64_t dst_pitch, void *stream) {
    return launch_transpose(src, dst, rows, cols, dst_pitch, stream);
}
