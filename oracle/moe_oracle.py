"""fp64 CPU oracle for the grouped NVFP4 MoE expert projection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP kernels; the only thing both sides consume in common
is the seeded input bytes from ``synth``.

What it computes is the plain definition of a top-k routed SwiGLU
mixture-of-experts over NVFP4-dequantised weights, in float64, step by step:

  1. NVFP4 decode (quant_shard.rs page, the layout comment above
     ``shard_quantized_nvfp4``; nvfp4_moe_grouped.rs page, module doc, which
     names the three parts: E2M1 codes, one E4M3 scale per 16 values and one
     f32 scale per tensor; expert.rs page, ``QuantWeight::Nvfp4`` doc): W[n, k] = e2m1(nibble) *
     e4m3(scale[n, k // 16]) * scale_2.  The transposed twin
     (transpose.rs page, ``transpose_for_gemm``) stores the same bytes at
     [k // 2, n] and [k // 16, n].
  2. Routing sort (nvfp4_moe_grouped.rs page, module doc: rows grouped by
     expert, active experts listed, intermediates laid out by sorted
     position).
  3. Gate+up with the SiLU product (nvfp4_moe_grouped.rs page, doc of
     ``moe_expert_gate_up_act_nvfp4_grouped``).
  4. Down projection over the SiLU product (same page, doc of
     ``moe_expert_down_act_nvfp4_grouped``).
  5. Weighted top-k blend (same page, module doc: the weighted-sum blend).

MXFP4 experts (transpose.rs page, doc of ``transpose_for_gemm``: experts in
native MXFP4 use a scale group of 32; doc of ``transpose_for_gemm_gs``: the
scale tensor is [N, K / group]): the same E2M1 codes with one E8M0 scale per
32 values, W[n, k] = e2m1(nibble) * e8m0(scale[n, k // 32]) * scale_2.

Readings where the pages are silent (each listed in the design notes):
  * E2M1 is the OCP FP4 format (1 sign, 2 exponent bits with bias 1,
    1 mantissa bit; code 0b?001 is the subnormal 0.5).
  * E4M3 is the OCP "FN" variant: bias 7, subnormals, no infinities, NaN
    only at S.1111.111, largest finite 448 (prefill_weights.rs page, the
    shared-expert copies, gives 448 as the E4M3 saturation point).
  * The low nibble of a packed byte holds the even k.
  * E8M0 (the MXFP4 scale) is the OCP MX scale format: the byte is a biased
    exponent, value 2^(code - 127), code 255 is NaN; no sign, no mantissa.
  * The sort is stable by flat pair index t*k + j; active experts ascend.
  * Pairs whose expert id lies outside [0, E) belong to no expert: they
    raise the error flag, get position -1 and contribute zero.
  * A NULL expert (absent pointers; expert.rs page, ``ExpertWeight::null``)
    contributes exactly zero: its rows of h and y are 0.
  * gate and up are not rounded to bf16 before the SiLU; SiLU(z) = z / (1 + e^-z).
  * Everything is carried in float64; inputs (bf16 x, f32 routing weights,
    f32 scale_2) are widened exactly.
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np


# --------------------------------------------------------------------------
# Decode tables (closed forms of the two minifloat formats)
# --------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


def e4m3fn_value(code: int) -> float:
    """Value of an 8-bit E4M3 (FN) code: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 7
    if exp == 0xF and man == 7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e8m0_value(code: int) -> float:
    """Value of an 8-bit E8M0 scale code: 2^(code - 127); code 255 is NaN."""
    if code == 255:
        return math.nan
    return math.ldexp(1.0, code - 127)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3FN = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

# Scale format of each weight format: (values per scale, scale code table).
FORMATS = {"nvfp4": (16, E4M3FN), "mxfp4": (32, E8M0)}


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# NVFP4 dequantisation
# --------------------------------------------------------------------------
def dequant(packed: np.ndarray, scale: np.ndarray, scale2, n: int, k: int, kmajor: bool = False,
            fmt: str = "nvfp4") -> np.ndarray:
    """Dequantise one projection to float64 [n, k].

    NVFP4 (group g = 16, E4M3 scales) or MXFP4 (g = 32, E8M0 scales).
    Row-major: packed [n, k/2], scale [n, k/g].  K-major twin: packed
    [k/2, n], scale [k/g, n].  Element (n, k) reads nibble (k & 1) of byte
    (n, k >> 1) and scale byte (n, k // g).  Exact in float64 (NVFP4: at
    most 2 + 4 + 24 significant bits; MXFP4: the scale is a power of two).
    """
    g, table = FORMATS[fmt]
    if kmajor:
        assert packed.shape == (k // 2, n) and scale.shape == (k // g, n)
        pb = packed.T
        sb = scale.T
    else:
        assert packed.shape == (n, k // 2) and scale.shape == (n, k // g)
        pb = packed
        sb = scale
    kk = np.arange(k)
    byte = pb[:, kk >> 1].astype(np.uint8)
    code = (byte >> (4 * (kk & 1)).astype(np.uint8)) & 0xF
    s = table[sb[:, kk // g]]
    return E2M1[code] * s * float(np.float32(scale2))


# --------------------------------------------------------------------------
# Load-time byte transpose (transpose.rs page, host loop of transpose_for_gemm_gs)
# --------------------------------------------------------------------------
def transpose_u8(src: np.ndarray) -> np.ndarray:
    """dst[c, r] = src[r, c] for a byte matrix [rows, cols] -> [cols, rows]."""
    assert src.dtype == np.uint8 and src.ndim == 2
    return np.ascontiguousarray(src.T)


def transpose_concat(parts, stride: int) -> np.ndarray:
    """Concatenated transposed twin (transpose.rs page, doc of
    ``transpose_concat_for_gemm_padded`` and the implementation behind the
    concatenating builders): byte matrices [n_p, cols] sharing cols are
    transposed side by side, part p at columns [off_p, off_p + n_p) of a
    [cols, stride] matrix, off_p the sum of the earlier n; the pad columns
    sum(n) .. stride are zero."""
    cols = parts[0].shape[1]
    out = np.zeros((cols, stride), dtype=np.uint8)
    off = 0
    for p in parts:
        assert p.dtype == np.uint8 and p.shape[1] == cols
        out[:, off: off + p.shape[0]] = p.T
        off += p.shape[0]
    assert off <= stride
    return out


# --------------------------------------------------------------------------
# Router (ahead of the path: softmax over the expert logits, top k kept,
# weights renormalised over them).  The pages show only the router's logit
# GEMM (prefill_weights.rs page, doc of dense_gemm_prefill: the gate GEMM);
# the selection and weights follow the routing the workloads are defined by.
# --------------------------------------------------------------------------
def route_topk(logits: np.ndarray, k: int):
    """Top-k routing of each row of f32 logits [T, E].

    ids: the k largest logits of the row in descending order, equal logits by
    lower expert id, NaN below every number (-0.0 equals +0.0).
    weights (float64): softmax renormalised over the selected experts,
    p_j / sum_i p_i with p = softmax(row); the full denominator cancels, so
    w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the selected i.
    """
    assert logits.dtype == np.float32 and logits.ndim == 2
    T, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = logits[t].astype(np.float64)
        key = np.where(np.isnan(row), -np.inf, row)          # NaN ranks lowest...
        nan_last = np.isnan(row).astype(np.int64)             # ...even below -inf
        order = np.lexsort((np.arange(E), nan_last, -key))[:k]
        ids[t] = order
        sel = row[order]
        z = np.exp(sel - sel[0])
        w[t] = z / z.sum()
    return ids, w


# --------------------------------------------------------------------------
# Routing sort
# --------------------------------------------------------------------------
def sort_routes(topk_ids: np.ndarray, E: int) -> dict:
    """Group the T*k routed pairs by expert.

    Returns int32 arrays: expert_offsets [E+1] (exclusive prefix of the
    per-expert counts), sorted_token_ids [P] (token of the pair at each
    sorted position, -1 past the last valid pair), pair_pos [P] (sorted
    position of flat pair f, -1 for an invalid id), active_experts [E]
    (experts with at least one pair, ascending, -1 past active_count),
    active_count, and err (1 if any id lies outside [0, E)).
    """
    T, k = topk_ids.shape
    P = T * k
    flat = topk_ids.reshape(-1).astype(np.int64)
    f = np.arange(P)
    valid = (flat >= 0) & (flat < E)
    fv = f[valid]
    order = fv[np.lexsort((fv, flat[valid]))]          # by (expert, flat index)
    counts = np.bincount(flat[valid], minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_tok = np.full(P, -1, dtype=np.int64)
    sorted_tok[: order.size] = order // k
    pair_pos = np.full(P, -1, dtype=np.int64)
    pair_pos[order] = np.arange(order.size)
    active = np.nonzero(counts)[0]
    active_experts = np.full(E, -1, dtype=np.int64)
    active_experts[: active.size] = active
    return {
        "expert_offsets": offsets.astype(np.int32),
        "sorted_token_ids": sorted_tok.astype(np.int32),
        "pair_pos": pair_pos.astype(np.int32),
        "active_experts": active_experts.astype(np.int32),
        "active_count": int(active.size),
        "err": int(not bool(valid.all())),
    }


# --------------------------------------------------------------------------
# The three arithmetic steps
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gate_up_silu_rows(x_rows: np.ndarray, Wg: np.ndarray, Wu: np.ndarray) -> np.ndarray:
    """h = silu(x Wg^T) * (x Wu^T) for float64 rows x [R, H], weights [I, H]."""
    return silu(x_rows @ Wg.T) * (x_rows @ Wu.T)


def down_rows(h_rows: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """y = h Wd^T for float64 rows h [R, I], weight [H, I]."""
    return h_rows @ Wd.T


def blend(y: np.ndarray, topk_weights: np.ndarray, pair_pos: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[pair_pos[t*k + j]], j ascending; invalid pairs add 0."""
    T, k = topk_weights.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    w = topk_weights.astype(np.float64)
    for t in range(T):
        for j in range(k):
            p = int(pair_pos[t * k + j])
            if p >= 0:
                out[t] += w[t, j] * y[p]
    return out


# Weight provider: (expert, projection) -> (packed, scale, scale2) or None for a NULL expert.
WeightFn = Callable[[int, int], Optional[tuple]]


def expert_weights(weights: WeightFn, e: int, H: int, I: int, kmajor: bool, fmt: str = "nvfp4"):
    """Dequantised (Wg [I,H], Wu [I,H], Wd [H,I]) of expert e, or None if it is NULL."""
    parts = [weights(e, p) for p in (0, 1, 2)]
    if any(p is None for p in parts):
        return None
    dims = ((I, H), (I, H), (H, I))
    return tuple(dequant(pk, sc, s2, n, kk, kmajor, fmt) for (pk, sc, s2), (n, kk) in zip(parts, dims))


def moe_layer(x_bits: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
              weights: WeightFn, E: int, H: int, I: int, kmajor: bool = False, fmt: str = "nvfp4") -> dict:
    """The whole path: sort, gate+up+SiLU, down, blend.  Returns the sort
    outputs plus float64 h [P, I], y [P, H] and out [T, H]."""
    T, k = topk_ids.shape
    P = T * k
    x = bf16_bits_to_f64(x_bits)
    srt = sort_routes(topk_ids, E)
    h = np.zeros((P, I), dtype=np.float64)
    y = np.zeros((P, H), dtype=np.float64)
    offs = srt["expert_offsets"]
    for e in srt["active_experts"][: srt["active_count"]]:
        lo, hi = int(offs[e]), int(offs[e + 1])
        W = expert_weights(weights, int(e), H, I, kmajor, fmt)
        if W is None:
            continue
        Wg, Wu, Wd = W
        rows = x[srt["sorted_token_ids"][lo:hi]]
        h[lo:hi] = gate_up_silu_rows(rows, Wg, Wu)
        y[lo:hi] = down_rows(h[lo:hi], Wd)
    out = blend(y, topk_weights, srt["pair_pos"])
    return dict(srt, h=h, y=y, out=out)
