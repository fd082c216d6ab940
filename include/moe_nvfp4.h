/*
 * moe_nvfp4.h — C ABI of the grouped NVFP4 mixture-of-experts expert
 * projection for AMD Instinct MI355X (gfx950).
 *
 * The path has four calls per MoE layer, issued in this order on one stream:
 *
 *   moe_nvfp4_sort          group the routed (token, expert) pairs by expert
 *   moe_nvfp4_gate_up_silu  h = silu(x Wg^T) * (x Wu^T) per routed pair
 *   moe_nvfp4_down          y = h Wd^T per routed pair
 *   moe_nvfp4_blend         out[t] = sum_j w[t, j] * y[pair of (t, j)]
 *
 * plus a load-time byte transpose, transpose_u8, that builds the K-major
 * transposed twin of a weight for the many-token path.  Also declared here:
 *
 *   moe_nvfp4_route                 the router ahead of the path (softmax,
 *                                   top-k, weights renormalised over the k)
 *   moe_nvfp4_sort_gate_up_silu     sort + gate+up, one launch at few pairs
 *   moe_nvfp4_sort_gate_up_launches host-only: is that one launch or two
 *   moe_nvfp4_down_blend            down + blend in one launch (few tokens)
 *   transpose_u8_pitched,           a concatenated gate||up K-major twin with
 *   moe_nvfp4_gate_up_silu_concat   a padded row pitch, and gate+up over it
 *
 * and the layout MOE_NVFP4_K_MAJOR_MXFP4 (MXFP4 experts: E8M0 scales per 32).
 *
 * Sources of the operations (the reference pages are Rust source pages of a
 * model runtime; each is cited by its file name and the item on it):
 *   - NVFP4 layout: quant_shard.rs, layout comment above shard_quantized_nvfp4
 *     (packed [N, K/2] u8 E2M1 nibbles, [N, K/group] u8 E4M3 scales, one f32
 *     per-tensor scale_2); nvfp4_moe_grouped.rs, module doc (group 16).
 *   - Sort, gate+up+SiLU, down, blend: nvfp4_moe_grouped.rs, module doc and
 *     the docs of moe_expert_gate_up_act_nvfp4_grouped and
 *     moe_expert_down_act_nvfp4_grouped; the per-expert pointer tables are
 *     that page's Nvfp4ExpertTables.
 *   - Transposed twin: transpose.rs, transpose_for_gemm / transpose_for_gemm_gs
 *     (packed [N, K/2] -> [K/2, N], scales [N, K/16] -> [K/16, N]).
 *   - NULL experts contribute nothing: expert.rs, ExpertWeight::null.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *     caller owns every buffer.  The library allocates nothing, frees nothing,
 *     keeps no state between calls and never synchronizes: each call only
 *     enqueues work on `stream` (a hipStream_t; NULL = the default stream).
 *   - Outputs never alias inputs.
 *   - Return value: MOE_NVFP4_OK (0) on success; a negative MOE_NVFP4_E*
 *     code when the host-side argument check fails, in which case NOTHING
 *     was launched; a positive hipError_t if a launch itself failed.
 *   - Shapes: T tokens, k experts per token (top-k), P = T * k routed pairs,
 *     E experts, H hidden width, I expert intermediate width.  Matrices are
 *     row-major and dense (row stride = row length), except the
 *     concatenated twin, whose row pitch is an argument.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_NVFP4_ABI_VERSION 7

/* Weight layouts of a projection [N, K] (N outputs, K inputs). */
#define MOE_NVFP4_ROW_MAJOR     0 /* packed [N, K/2], E4M3 scales [N, K/16]  (decode GEMV path)     */
#define MOE_NVFP4_K_MAJOR       1 /* packed [K/2, N], E4M3 scales [K/16, N]  (many-token MFMA path) */
#define MOE_NVFP4_K_MAJOR_MXFP4 2 /* packed [K/2, N], E8M0 scales [K/32, N]  (many-token MFMA path) */

/* Host-side argument errors (nothing is launched). */
#define MOE_NVFP4_OK          0
#define MOE_NVFP4_ENULL      -1 /* a required pointer is NULL                          */
#define MOE_NVFP4_ESHAPE     -2 /* a size is out of range or not admitted (see call)    */
#define MOE_NVFP4_ELAYOUT    -3 /* unknown layout, or gate/up layouts differ            */
#define MOE_NVFP4_ELIMIT     -4 /* a size exceeds a documented maximum of the call      */

/* Device error flag bits (moe_nvfp4_sort's err_flag). */
#define MOE_NVFP4_FLAG_BAD_EXPERT_ID 1u

/*
 * One NVFP4 projection across the experts (the pages' Nvfp4ExpertTables):
 * device arrays of E device pointers and E floats.
 *   packed[e]  E2M1 nibbles, two per byte, low nibble = even k.
 *              ROW_MAJOR: [N, K/2]; K_MAJOR, K_MAJOR_MXFP4: [K/2, N].
 *   scale[e]   E4M3 (OCP "FN": bias 7, max 448, NaN = S.1111.111) block
 *              scales, one per 16 consecutive k.  ROW_MAJOR: [N, K/16];
 *              K_MAJOR: [K/16, N].
 *              K_MAJOR_MXFP4: E8M0 block scales (OCP MX: value
 *              2^(code - 127)), one per 32 consecutive k, [K/32, N]
 *              (transpose.rs, transpose_for_gemm: native-MXFP4 experts use
 *              a scale group of 32).
 *   scale2[e]  the per-tensor f32 scale_2 (1.0 for plain MXFP4).
 * Weight element (n, k) = e2m1(nibble) * e4m3(scale of group k/16) * scale_2,
 * or, for K_MAJOR_MXFP4, e2m1(nibble) * e8m0(scale of group k/32) * scale_2.
 * packed[e] == NULL or scale[e] == NULL marks an absent expert (not owned
 * under expert parallelism): its rows of h and y are written as 0, so it
 * contributes 0.  The tables must hold at least E entries (the calls read
 * entry e for every routed id e < E).
 * Scale codes must not be NaN (E4M3 0x7F, 0xFF; E8M0 0xFF): results are
 * then unspecified.  E8M0 codes above 252 can take a weight past the f32
 * range (it then decodes to infinity).
 */
typedef struct {
    const uint8_t *const *packed;
    const uint8_t *const *scale;
    const float *scale2;
    int32_t layout; /* MOE_NVFP4_ROW_MAJOR, MOE_NVFP4_K_MAJOR or MOE_NVFP4_K_MAJOR_MXFP4 */
} moe_nvfp4_experts;

/* Maximum sizes admitted by the calls below. */
#define MOE_NVFP4_MAX_EXPERTS 1024
#define MOE_NVFP4_MAX_PAIRS   (1 << 22)
#define MOE_NVFP4_MAX_WIDTH   (1 << 16) /* H and I */

/*
 * moe_nvfp4_sort — group the P = T*k routed pairs by expert
 * (nvfp4_moe_grouped.rs, module doc: rows grouped by expert, active experts
 * listed, intermediates laid out by sorted position).
 *
 *   topk_ids          in  int32 [T, k]  expert of pair f = t*k + j.
 *   expert_offsets    out int32 [E+1]   exclusive prefix sum of the per-expert
 *                                       pair counts; rows of expert e are the
 *                                       sorted positions [off[e], off[e+1]).
 *   sorted_token_ids  out int32 [P]     token t of the pair at each sorted
 *                                       position; -1 past the last valid pair.
 *   pair_pos          out int32 [P]     sorted position of flat pair f; -1 for
 *                                       a pair with an invalid expert id.
 *   active_experts    out int32 [E]     experts with at least one pair, in
 *                                       ascending id order; -1 past the count.
 *   active_count      out int32 [1]     number of active experts.
 *   err_flag          in/out uint32 [1] zeroed by the caller; OR-ed with
 *                                       MOE_NVFP4_FLAG_BAD_EXPERT_ID if any id
 *                                       lies outside [0, E).  Such a pair joins
 *                                       no expert and contributes 0.
 * Order within an expert is by flat pair index (stable), so every output is
 * unique and deterministic.  Errors: ENULL; ESHAPE if T < 1, k < 1, E < 1 or
 * k > E; ELIMIT if E > MOE_NVFP4_MAX_EXPERTS or P > MOE_NVFP4_MAX_PAIRS.
 */
int moe_nvfp4_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                   int32_t *expert_offsets, int32_t *sorted_token_ids, int32_t *pair_pos,
                   int32_t *active_experts, int32_t *active_count, uint32_t *err_flag,
                   void *stream);

/*
 * moe_nvfp4_gate_up_silu — fused gate+up projection and SiLU product
 * (nvfp4_moe_grouped.rs, doc of moe_expert_gate_up_act_nvfp4_grouped).
 * For every active expert e and every sorted position p of e, with token
 * t = sorted_token_ids[p] and n < I:
 *     g = sum_k x[t, k] * Wg_e[n, k],   u = sum_k x[t, k] * Wu_e[n, k],
 *     h[p, n] = g / (1 + exp(-g)) * u        (fp32 accumulation and output)
 *
 *   x                 in  bf16 [T, H]
 *   gate, up          NVFP4 tables, N = I, K = H, both in the same layout.
 *                     ROW_MAJOR runs the decode GEMV (few tokens per expert);
 *                     K_MAJOR and K_MAJOR_MXFP4 run the grouped MFMA GEMM
 *                     (many tokens).
 *   expert_offsets, sorted_token_ids, active_experts, active_count:
 *                     moe_nvfp4_sort's outputs (read on the device only).
 *   h                 out fp32 [P, I]; rows of positions that belong to no
 *                     active expert are left untouched.
 * Admission: H % 64 == 0 and I % 64 == 0 (both layouts), H >= 256 and
 * I >= 256 (ROW_MAJOR); ROW_MAJOR also K <= 36736 (K = H here, I for the
 * down projection: the decode kernel stages whole activation rows in its
 * shared memory), ELIMIT above; packed, scale and activation buffers 16-byte
 * aligned; K_MAJOR(_MXFP4): the activation tensor (x here, h for the down
 * projection) below 4 GiB.  The K-major path feeds the matrix cores with
 * bf16 operands (x as given, the decoded weights exactly), so it admits the
 * whole bf16 range.
 * Errors: ENULL, ESHAPE, ELAYOUT (unknown layout, or gate and up differ),
 * ELIMIT (E, P or width above the maxima, or a K-major activation tensor of
 * 4 GiB or more).
 */
int moe_nvfp4_gate_up_silu(const uint16_t *x, int32_t T, int32_t k, int32_t E, int32_t H,
                           int32_t I, moe_nvfp4_experts gate, moe_nvfp4_experts up,
                           const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                           const int32_t *active_experts, const int32_t *active_count,
                           float *h, void *stream);

/*
 * moe_nvfp4_sort_gate_up_silu — moe_nvfp4_sort followed by
 * moe_nvfp4_gate_up_silu (the first two steps of nvfp4_moe_grouped.rs,
 * module doc), enqueued as ONE launch when the weights are ROW_MAJOR, the
 * P = T*k pairs number at most 64 and every expert's rows fit one staging
 * pass of the decode kernel (the few-token decode case, where a launch costs
 * more than the sort's work); otherwise as the two launches.  Every output
 * (the sort's five, err_flag, h) is defined exactly as by the two calls and
 * is complete when the work enqueued on `stream` is; err_flag is zeroed by
 * the caller as for moe_nvfp4_sort.  Arguments, admission and errors are the
 * union of the two calls'.
 */
int moe_nvfp4_sort_gate_up_silu(const int32_t *topk_ids, const uint16_t *x, int32_t T, int32_t k,
                                int32_t E, int32_t H, int32_t I, moe_nvfp4_experts gate,
                                moe_nvfp4_experts up, int32_t *expert_offsets,
                                int32_t *sorted_token_ids, int32_t *pair_pos,
                                int32_t *active_experts, int32_t *active_count, uint32_t *err_flag,
                                float *h, void *stream);

/*
 * moe_nvfp4_sort_gate_up_launches — how many launches
 * moe_nvfp4_sort_gate_up_silu enqueues for these sizes and layout on the
 * current device: 1 (the sort runs inside the gate+up launch) or 2.  Host
 * only; no device work.  Errors as moe_nvfp4_gate_up_silu's size and layout
 * checks.
 */
int moe_nvfp4_sort_gate_up_launches(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                                    int32_t layout);

/*
 * moe_nvfp4_gate_up_silu_concat — moe_nvfp4_gate_up_silu over a
 * concatenated gate||up K-major twin (transpose.rs,
 * transpose_concat_for_gemm_padded: gate and up, which share K = H, are
 * transposed side by side into one twin with a padded row pitch, so one GEMM
 * reads both; the result carries the first part's scale_2, and the caller
 * ensures both parts share it).  Computes exactly what
 * moe_nvfp4_gate_up_silu computes with
 *     Wg_e = columns [0, I) and Wu_e = columns [I, 2I) of the twin.
 *
 *   gate_up   one table: packed[e] [K/2, pitch] and scale[e] [K/g, pitch]
 *             (g = 16, or 32 for K_MAJOR_MXFP4) with rows `pitch` bytes
 *             apart; columns 2I .. pitch are padding (never read);
 *             scale2[e] serves both halves.  Layout K_MAJOR or
 *             K_MAJOR_MXFP4.
 *   pitch     row pitch of the twin in bytes: pitch >= 2I, pitch % 16 == 0.
 * Other arguments, admission and errors as moe_nvfp4_gate_up_silu; ESHAPE
 * also for a bad pitch, ELAYOUT for a row-major table.
 */
int moe_nvfp4_gate_up_silu_concat(const uint16_t *x, int32_t T, int32_t k, int32_t E, int32_t H,
                                  int32_t I, moe_nvfp4_experts gate_up, int32_t pitch,
                                  const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                                  const int32_t *active_experts, const int32_t *active_count,
                                  float *h, void *stream);

/*
 * moe_nvfp4_down — down projection over the SiLU product
 * (nvfp4_moe_grouped.rs, doc of moe_expert_down_act_nvfp4_grouped: k is the
 * intermediate width, rows of the activation and output are sorted
 * positions).  For every active expert e, position p of e and n < H:
 *     y[p, n] = sum_i h[p, i] * Wd_e[n, i]          (fp32 accumulation)
 *
 *   h      in  fp32 [P, I]   (the kernels round it to 16-bit floats for
 *                             the products; accumulation stays fp32)
 *   down   NVFP4 (or, K-major only, MXFP4) table, N = H, K = I.
 *   y      out fp32 [P, H]; rows of positions outside every active expert are
 *          left untouched.
 * Admission and errors as moe_nvfp4_gate_up_silu.
 */
int moe_nvfp4_down(const float *h, int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                   moe_nvfp4_experts down, const int32_t *expert_offsets,
                   const int32_t *active_experts, const int32_t *active_count, float *y,
                   void *stream);

/*
 * moe_nvfp4_blend — weighted sum of each token's top-k outputs
 * (nvfp4_moe_grouped.rs, module doc: the weighted-sum blend).
 *     out[t, n] = bf16_rne( sum_{j=0..k-1} topk_weights[t, j] * y[pair_pos[t*k+j], n] )
 * summed in fp32 in ascending j; a pair with pair_pos < 0 adds nothing.
 *
 *   y             in  fp32 [P, H]
 *   topk_weights  in  fp32 [T, k]
 *   pair_pos      in  int32 [T*k]  (moe_nvfp4_sort's output)
 *   out           out bf16 [T, H]
 * Errors: ENULL; ESHAPE if T < 1, k < 1 or H < 1; ELIMIT if P or H exceed
 * the maxima.
 */
int moe_nvfp4_blend(const float *y, const float *topk_weights, const int32_t *pair_pos,
                    int32_t T, int32_t k, int32_t H, uint16_t *out, void *stream);

/*
 * moe_nvfp4_down_blend — moe_nvfp4_down followed by moe_nvfp4_blend, in one
 * launch and without the y tensor (nvfp4_moe_grouped.rs, module doc: the
 * down projection of every routed pair, then the weighted sum of each
 * token's rows):
 *     out[t, n] = bf16_rne( sum_{j=0..k-1} topk_weights[t, j] * y_j[n] ),
 *     y_j[n]    = sum_i h[p, i] * Wd_e[n, i],  p = pair_pos[t*k+j], e = topk_ids[t*k+j],
 * summed in fp32 in ascending j; a pair with pair_pos < 0 adds nothing and a
 * pair whose expert is NULL adds w * 0.  Each y value is the one
 * moe_nvfp4_down computes, so out equals moe_nvfp4_down then
 * moe_nvfp4_blend bit for bit while no expert holds more than 4 routed pairs
 * (so for one token unless an id repeats more than 4 times; beyond that the
 * two differ only in the order of the fp32 sums inside a dot product).  One
 * block serves
 * one token for all of its pairs, so an expert's weights are read once per
 * token routed to it: meant for decode with one or a few tokens.
 *
 *   h             in  fp32 [P, I] (moe_nvfp4_gate_up_silu's output)
 *   down          NVFP4 table, ROW_MAJOR only; N = H, K = I.
 *   topk_ids      in  int32 [T, k] (the ids given to moe_nvfp4_sort)
 *   topk_weights  in  fp32 [T, k]
 *   pair_pos      in  int32 [T*k]  (moe_nvfp4_sort's output)
 *   out           out bf16 [T, H]
 * Admission: as moe_nvfp4_down for ROW_MAJOR, plus k <= 64, T <= 65535 and
 * the token's k activation rows staged in shared memory:
 * k * (2 I + pad) <= 73728 bytes (pad < 256), ELIMIT above.
 * Errors: ENULL, ESHAPE, ELAYOUT (any layout but ROW_MAJOR), ELIMIT.
 */
int moe_nvfp4_down_blend(const float *h, int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                         moe_nvfp4_experts down, const int32_t *topk_ids, const float *topk_weights,
                         const int32_t *pair_pos, uint16_t *out, void *stream);

/*
 * transpose_u8 — out-of-place byte-matrix transpose
 * (transpose.rs, transpose_for_gemm_gs and its host loop):
 *     dst[c * rows + r] = src[r * cols + c]     for r < rows, c < cols.
 * Applied to a packed weight with rows = N, cols = K/2 and to its scales
 * with rows = N, cols = K/16 (MXFP4: K/32), it builds the K-major twin.  src is left
 * unchanged; src and dst must not overlap.
 * Errors: ENULL; ESHAPE if rows < 1 or cols < 1; ELIMIT if rows * cols
 * exceeds 2^40 bytes.
 */
int transpose_u8(const uint8_t *src, uint8_t *dst, int32_t rows, int32_t cols, void *stream);

/*
 * transpose_u8_pitched — transpose_u8 into a column window of a wider matrix
 * (transpose.rs, transpose_concat_for_gemm_padded and the shared
 * implementation behind the concatenating builders, whose host loop writes
 * part p at column offset n_off of rows `stride` bytes apart):
 *     dst[c * dst_pitch + r] = src[r * cols + c]   for r < rows, c < cols.
 * Bytes of dst outside those positions are not touched, so the caller zeroes
 * pad columns and places each part by offsetting dst.
 * Errors: ENULL; ESHAPE if rows < 1, cols < 1 or dst_pitch < rows; ELIMIT if
 * rows * cols or dst_pitch * cols exceeds 2^40 bytes.
 */
int transpose_u8_pitched(const uint8_t *src, uint8_t *dst, int32_t rows, int32_t cols,
                         int64_t dst_pitch, void *stream);

/*
 * moe_nvfp4_route — router ahead of the path: softmax over each token's
 * expert logits, the k largest kept, weights renormalised over them.  The
 * pages show only the router's logit GEMM (prefill_weights.rs, doc of
 * dense_gemm_prefill: the gate GEMM); the outputs are the topk_ids and
 * topk_weights that moe_nvfp4_sort and moe_nvfp4_blend take.
 *
 *   logits        in  f32 [T, E]
 *   topk_ids      out int32 [T, k]  the k largest logits of row t in
 *                                   descending order; equal logits by lower
 *                                   expert id; -0.0 equals +0.0; NaN below
 *                                   every number.
 *   topk_weights  out f32 [T, k]    exp(l_j - l_max) / sum_i exp(l_i - l_max)
 *                                   over the k selected (equal to the softmax
 *                                   over all E renormalised over them); NaN
 *                                   where a selected logit is NaN or infinite.
 * Errors: ENULL; ESHAPE if T < 1, E < 1, k < 1 or k > E; ELIMIT if
 * E > MOE_NVFP4_MAX_EXPERTS, k > 64 or T * k > MOE_NVFP4_MAX_PAIRS.
 */
int moe_nvfp4_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                    float *topk_weights, void *stream);

/* ABI version of the loaded library (MOE_NVFP4_ABI_VERSION). */
int moe_nvfp4_abi_version(void);

/* ------------------------------------------------------------------------
 * Measurement support (not a step of the path).
 * ------------------------------------------------------------------------
 * moe_nvfp4_stream_read: read `bytes` of device memory at `src` once, in
 * contiguous 1 KiB wave loads (8 per lane in flight), and discard the data:
 * the streaming-read ceiling of this part, against which the decode path's
 * weight bandwidth is read (a kernel that only streams reads, no arithmetic).
 * `sink` is a device u32 that is written only in a case that does not occur
 * for ordinary data (it keeps the loads from being removed).
 * Errors: ENULL; ESHAPE if bytes < 16 or bytes % 16 != 0.
 */
int moe_nvfp4_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
