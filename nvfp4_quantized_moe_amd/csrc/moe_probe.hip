// Streaming-read ceiling: the HBM read bandwidth a plain kernel reaches on
// this part, measured beside the projection kernels (the weight streams of
// the decode path are bounded by it, not by the 8 TB/s of the data sheet).
// Each block reads one contiguous share of the buffer; every load
// instruction covers 1 KiB (64 lanes x 16 bytes) and each lane keeps 8 in
// flight.  The loaded words are folded with XOR into a value stored only if
// it equals a constant, so the loads cannot be dropped.
#include "moe_common.hpp"

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint8_t *src, int64_t n16, uint32_t *sink) {
    const int64_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per_block;
    const int64_t hi = lo + per_block < n16 ? lo + per_block : n16;
    moe::u32x4_t acc = {0u, 0u, 0u, 0u};
    int64_t i = lo + threadIdx.x;
    for (; i + (kReadUnroll - 1) * kReadThreads < hi; i += kReadUnroll * kReadThreads) {
        moe::u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = moe::gload<moe::u32x4_t>(src + 16 * (i + u * kReadThreads));
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    for (; i < hi; i += kReadThreads) acc ^= moe::gload<moe::u32x4_t>(src + 16 * i);
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

extern "C" int moe_nvfp4_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink) return MOE_NVFP4_ENULL;
    if (bytes < 16 || bytes % 16 != 0) return MOE_NVFP4_ESHAPE;
    const int blocks = 8 * moe_host::cu_count();
    hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(kReadThreads), 0, (hipStream_t)stream,
                       static_cast<const uint8_t *>(src), bytes / 16, sink);
    return moe_host::launch_status();
}
