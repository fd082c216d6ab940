// C-ABI entry points of the two projection steps: host-side argument checks,
// then one launch on the caller's stream.  The weight layout picks the
// kernel: row-major -> decode kernel (few rows per expert), K-major (NVFP4 or
// MXFP4) -> grouped MFMA GEMM (many rows per expert), mirroring the pages'
// split between the row-major decode kernels (nvfp4_moe_grouped.rs) and the
// transposed twins built for the sorted prefill path (prefill_weights.rs).
#include "moe_common.hpp"

int moe_launch_decode_row(bool gated, const void *act, const int32_t *sorted_tok, const int32_t *offsets,
                          const int32_t *active, const int32_t *nactive, const moe_nvfp4_experts &A,
                          const moe_nvfp4_experts *B, float *out, int N, int K, int T, int P, int E,
                          hipStream_t stream, const MoeSortFuse *fuse);
int moe_decode_sort_gate_up_launches(int N, int K, int P, int E);
int moe_launch_down_blend(const float *h, const int32_t *topk_ids, const float *topk_weights,
                          const int32_t *pair_pos, const moe_nvfp4_experts &D, uint16_t *out, int N, int K, int T,
                          int k, int E, hipStream_t stream);
int moe_launch_sort(const int32_t *topk_ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_tok,
                    int32_t *pair_pos, int32_t *active, int32_t *active_count, uint32_t *err_flag,
                    hipStream_t stream);
int moe_launch_gemm_kmajor(bool gated, bool mx, const void *act, const int32_t *sorted_tok,
                           const int32_t *offsets, const int32_t *active, const int32_t *nactive,
                           const moe_nvfp4_experts &A, const moe_nvfp4_experts *B, float *out, int N, int K,
                           int P, int E, int ldb, int up_off, hipStream_t stream);

namespace {

int check_common(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I, int32_t layout) {
    if (T < 1 || k < 1 || E < 1 || k > E || H < 1 || I < 1) return MOE_NVFP4_ESHAPE;
    if (E > MOE_NVFP4_MAX_EXPERTS || (int64_t)T * k > MOE_NVFP4_MAX_PAIRS) return MOE_NVFP4_ELIMIT;
    if (H > MOE_NVFP4_MAX_WIDTH || I > MOE_NVFP4_MAX_WIDTH) return MOE_NVFP4_ELIMIT;
    if (layout != MOE_NVFP4_ROW_MAJOR && layout != MOE_NVFP4_K_MAJOR && layout != MOE_NVFP4_K_MAJOR_MXFP4)
        return MOE_NVFP4_ELAYOUT;
    if (H % 64 != 0 || I % 64 != 0) return MOE_NVFP4_ESHAPE;
    if (layout == MOE_NVFP4_ROW_MAJOR && (H < 256 || I < 256)) return MOE_NVFP4_ESHAPE;
    return MOE_NVFP4_OK;
}

}  // namespace

extern "C" int moe_nvfp4_gate_up_silu(const uint16_t *x, int32_t T, int32_t k, int32_t E, int32_t H,
                                      int32_t I, moe_nvfp4_experts gate, moe_nvfp4_experts up,
                                      const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                                      const int32_t *active_experts, const int32_t *active_count, float *h,
                                      void *stream) {
    if (!x || !expert_offsets || !sorted_token_ids || !active_experts || !active_count || !h)
        return MOE_NVFP4_ENULL;
    if (moe_host::experts_null(gate) || moe_host::experts_null(up)) return MOE_NVFP4_ENULL;
    if (gate.layout != up.layout) return MOE_NVFP4_ELAYOUT;
    const int rc = check_common(T, k, E, H, I, gate.layout);
    if (rc != MOE_NVFP4_OK) return rc;
    const int P = T * k;
    if (gate.layout == MOE_NVFP4_ROW_MAJOR)
        return moe_launch_decode_row(true, x, sorted_token_ids, expert_offsets, active_experts, active_count,
                                     gate, &up, h, I, H, T, P, E, (hipStream_t)stream, nullptr);
    if ((uint64_t)T * H * 2 > 0xffffffffull) return MOE_NVFP4_ELIMIT;  // 32-bit activation offsets
    return moe_launch_gemm_kmajor(true, gate.layout == MOE_NVFP4_K_MAJOR_MXFP4, x, sorted_token_ids,
                                  expert_offsets, active_experts, active_count, gate, &up, h, I, H, P, E, I, 0,
                                  (hipStream_t)stream);
}

extern "C" int moe_nvfp4_sort_gate_up_silu(const int32_t *topk_ids, const uint16_t *x, int32_t T, int32_t k,
                                           int32_t E, int32_t H, int32_t I, moe_nvfp4_experts gate,
                                           moe_nvfp4_experts up, int32_t *expert_offsets,
                                           int32_t *sorted_token_ids, int32_t *pair_pos, int32_t *active_experts,
                                           int32_t *active_count, uint32_t *err_flag, float *h, void *stream) {
    if (!topk_ids || !x || !expert_offsets || !sorted_token_ids || !pair_pos || !active_experts ||
        !active_count || !err_flag || !h)
        return MOE_NVFP4_ENULL;
    if (moe_host::experts_null(gate) || moe_host::experts_null(up)) return MOE_NVFP4_ENULL;
    if (gate.layout != up.layout) return MOE_NVFP4_ELAYOUT;
    const int rc = check_common(T, k, E, H, I, gate.layout);
    if (rc != MOE_NVFP4_OK) return rc;
    const int P = T * k;
    const hipStream_t st = (hipStream_t)stream;
    if (gate.layout == MOE_NVFP4_ROW_MAJOR) {
        const MoeSortFuse fuse{topk_ids, k, expert_offsets, sorted_token_ids, pair_pos, active_experts,
                               active_count, err_flag};
        return moe_launch_decode_row(true, x, sorted_token_ids, expert_offsets, active_experts, active_count, gate,
                                     &up, h, I, H, T, P, E, st, &fuse);
    }
    if ((uint64_t)T * H * 2 > 0xffffffffull) return MOE_NVFP4_ELIMIT;  // 32-bit activation offsets
    const int src = moe_launch_sort(topk_ids, T, k, E, expert_offsets, sorted_token_ids, pair_pos, active_experts,
                                    active_count, err_flag, st);
    if (src != MOE_NVFP4_OK) return src;
    return moe_launch_gemm_kmajor(true, gate.layout == MOE_NVFP4_K_MAJOR_MXFP4, x, sorted_token_ids,
                                  expert_offsets, active_experts, active_count, gate, &up, h, I, H, P, E, I, 0, st);
}

extern "C" int moe_nvfp4_sort_gate_up_launches(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                                               int32_t layout) {
    const int rc = check_common(T, k, E, H, I, layout);
    if (rc != MOE_NVFP4_OK) return rc;
    if (layout != MOE_NVFP4_ROW_MAJOR) return 2;
    return moe_decode_sort_gate_up_launches(I, H, T * k, E);
}

extern "C" int moe_nvfp4_gate_up_silu_concat(const uint16_t *x, int32_t T, int32_t k, int32_t E, int32_t H,
                                             int32_t I, moe_nvfp4_experts gate_up, int32_t pitch,
                                             const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                                             const int32_t *active_experts, const int32_t *active_count,
                                             float *h, void *stream) {
    if (!x || !expert_offsets || !sorted_token_ids || !active_experts || !active_count || !h)
        return MOE_NVFP4_ENULL;
    if (moe_host::experts_null(gate_up)) return MOE_NVFP4_ENULL;
    const int rc = check_common(T, k, E, H, I, gate_up.layout);
    if (rc != MOE_NVFP4_OK) return rc;
    if (gate_up.layout == MOE_NVFP4_ROW_MAJOR) return MOE_NVFP4_ELAYOUT;
    if ((int64_t)pitch < 2 * (int64_t)I || pitch % 16 != 0) return MOE_NVFP4_ESHAPE;
    if ((uint64_t)T * H * 2 > 0xffffffffull) return MOE_NVFP4_ELIMIT;  // 32-bit activation offsets
    return moe_launch_gemm_kmajor(true, gate_up.layout == MOE_NVFP4_K_MAJOR_MXFP4, x, sorted_token_ids,
                                  expert_offsets, active_experts, active_count, gate_up, nullptr, h, I, H,
                                  T * k, E, pitch, I, (hipStream_t)stream);
}

extern "C" int moe_nvfp4_down(const float *h, int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                              moe_nvfp4_experts down, const int32_t *expert_offsets,
                              const int32_t *active_experts, const int32_t *active_count, float *y,
                              void *stream) {
    if (!h || !expert_offsets || !active_experts || !active_count || !y) return MOE_NVFP4_ENULL;
    if (moe_host::experts_null(down)) return MOE_NVFP4_ENULL;
    const int rc = check_common(T, k, E, H, I, down.layout);
    if (rc != MOE_NVFP4_OK) return rc;
    const int P = T * k;
    if (down.layout == MOE_NVFP4_ROW_MAJOR)
        return moe_launch_decode_row(false, h, nullptr, expert_offsets, active_experts, active_count, down,
                                     nullptr, y, H, I, T, P, E, (hipStream_t)stream, nullptr);
    if ((uint64_t)P * I * 4 > 0xffffffffull) return MOE_NVFP4_ELIMIT;  // 32-bit activation offsets
    return moe_launch_gemm_kmajor(false, down.layout == MOE_NVFP4_K_MAJOR_MXFP4, h, nullptr, expert_offsets,
                                  active_experts, active_count, down, nullptr, y, H, I, P, E, H, 0,
                                  (hipStream_t)stream);
}

extern "C" int moe_nvfp4_down_blend(const float *h, int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                                    moe_nvfp4_experts down, const int32_t *topk_ids, const float *topk_weights,
                                    const int32_t *pair_pos, uint16_t *out, void *stream) {
    if (!h || !topk_ids || !topk_weights || !pair_pos || !out) return MOE_NVFP4_ENULL;
    if (moe_host::experts_null(down)) return MOE_NVFP4_ENULL;
    const int rc = check_common(T, k, E, H, I, down.layout);
    if (rc != MOE_NVFP4_OK) return rc;
    if (down.layout != MOE_NVFP4_ROW_MAJOR) return MOE_NVFP4_ELAYOUT;
    return moe_launch_down_blend(h, topk_ids, topk_weights, pair_pos, down, out, H, I, T, k, E,
                                 (hipStream_t)stream);
}
