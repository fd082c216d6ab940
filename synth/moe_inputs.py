"""Seeded input generators (no projection arithmetic here).

Every array is drawn from numpy's PCG64 under
``SeedSequence([2026, cfg_id, tag, a, b])`` so that any single expert
projection can be regenerated on its own:

    tag 1  activations x                (a = batch, b = 0)
    tag 2  router logits                (a = batch, b = 0)
    tag 3  Zipf rank permutation        (a = b = 0)
    tag 4  packed E2M1 bytes            (a = expert, b = projection)
    tag 5  E4M3 block-scale codes       (a = expert, b = projection)
    tag 6  E8M0 block-scale codes       (a = expert, b = projection; MXFP4)

Projection ids: 0 = gate, 1 = up, 2 = down.  Gate and up are ``[N=I, K=H]``,
down is ``[N=H, K=I]``; all are generated row-major (packed ``[N, K/2]``,
scales ``[N, K/16]``), as the NVFP4 layout on the pages defines them
(quant_shard.rs page, layout comment above ``shard_quantized_nvfp4``).

Value distributions (one per input, stated by the workload definitions):
  * packed bytes uniform over 0..255, so both nibbles are uniform over the
    16 E2M1 codes; the low nibble holds the even k;
  * block scales: a real ``u ~ U[2^-4, 2^2]`` encoded to the nearest E4M3
    (FN variant) code by torch's float8_e4m3fn cast, ties to even;
  * per-tensor scale_2 = float32(1 / (448 * 6)) for every projection;
  * MXFP4 weights (the many-token shape with native-MXFP4 experts): the
    same packed bytes; block scales drawn as for NVFP4 (a real
    ``u ~ U[2^-4, 2^2]``) times 2^-11 (the magnitude NVFP4's scale_2 of
    1/2688 ~ 2^-11.4 gives), rounded to the nearest power of two in log2
    (E8M0 holds powers of two only): codes 112..118, most of them 116..118;
    scale_2 = 1 (MXFP4 has no per-tensor scale);
  * x: standard normal float32, rounded to bf16 (nearest-even) by torch;
  * router: standard-normal logits (plus, for the skewed workload, a Zipf
    bias ``-s * ln(rank)`` over a seeded rank permutation of the experts),
    top-k by descending logit with ties to the lower expert id, weights =
    softmax probabilities of the chosen experts renormalised to sum 1,
    stored as float32.  Routing is an input to the projection, not part
    of it.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2
SCALE2_F32 = np.float32(1.0 / (448.0 * 6.0))
SCALE2_MX_F32 = np.float32(1.0)
_SEED_ROOT = 2026


@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    T: int          # tokens
    H: int          # hidden width (gate/up K, down N)
    I: int          # expert intermediate width (gate/up N, down K)
    E: int          # experts
    k: int          # experts per token (top-k)
    routing: str    # "uniform" | "zipf"
    kmajor: bool    # weights consumed in the transposed [K/2, N] layout
    zipf_s: float = 1.1

    @property
    def P(self) -> int:
        return self.T * self.k


CONFIGS = {
    1: MoeShape("tiny_t4_h256_i512_e4_top2", 4, 256, 512, 4, 2, "uniform", False),
    2: MoeShape("decode_t1_h2048_i768_e128_top8", 1, 2048, 768, 128, 8, "uniform", False),
    3: MoeShape("decode_t32_h2688_i1856_e128_top6_zipf1.1", 32, 2688, 1856, 128, 6, "zipf", False),
    4: MoeShape("decode_t64_h7168_i2048_e256_top8", 64, 7168, 2048, 256, 8, "uniform", False),
    5: MoeShape("prefill_t2048_h4096_i1536_e64_top4_kmajor", 2048, 4096, 1536, 64, 4, "uniform", True),
}


def config(cfg_id: int) -> MoeShape:
    return CONFIGS[cfg_id]


def _rng(cfg_id: int, tag: int, a: int = 0, b: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_ROOT, cfg_id, tag, a, b])))


def proj_dims(shape: MoeShape, proj: int) -> tuple[int, int]:
    """(N, K) of a projection: gate/up map H -> I, down maps I -> H."""
    if proj in (PROJ_GATE, PROJ_UP):
        return shape.I, shape.H
    if proj == PROJ_DOWN:
        return shape.H, shape.I
    raise ValueError(proj)


def expert_bytes(shape: MoeShape, group: int = 16) -> int:
    """Weight bytes of one expert: packed K/2 + scale K/group bytes per row
    (group 16 for NVFP4, 32 for MXFP4), 3 projections."""
    tot = 0
    for proj in (PROJ_GATE, PROJ_UP, PROJ_DOWN):
        n, k = proj_dims(shape, proj)
        tot += n * (k // 2) + n * (k // group)
    return tot


def gen_x(cfg_id: int, shape: MoeShape | None = None, batch: int = 0) -> np.ndarray:
    """Activations as bf16 bit patterns, uint16 [T, H]; ``batch`` selects an
    independent draw of the same workload."""
    shape = shape or config(cfg_id)
    f = _rng(cfg_id, 1, batch).standard_normal((shape.T, shape.H), dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def gen_logits(cfg_id: int, shape: MoeShape | None = None, batch: int = 0) -> np.ndarray:
    """Router logits float32 [T, E]: the draw behind ``gen_routing`` (with
    the Zipf bias where the workload has one), rounded to f32."""
    shape = shape or config(cfg_id)
    logits = _rng(cfg_id, 2, batch).standard_normal((shape.T, shape.E))
    if shape.routing == "zipf":
        rank = 1 + _rng(cfg_id, 3).permutation(shape.E)
        logits = logits - shape.zipf_s * np.log(rank.astype(np.float64))[None, :]
    elif shape.routing != "uniform":
        raise ValueError(shape.routing)
    return logits.astype(np.float32)


def gen_routing(cfg_id: int, shape: MoeShape | None = None, batch: int = 0):
    """Router output: (topk_ids int32 [T, k], topk_weights float32 [T, k]);
    ``batch`` selects an independent draw (the Zipf rank order is shared)."""
    shape = shape or config(cfg_id)
    logits = _rng(cfg_id, 2, batch).standard_normal((shape.T, shape.E))
    if shape.routing == "zipf":
        rank = 1 + _rng(cfg_id, 3).permutation(shape.E)
        logits = logits - shape.zipf_s * np.log(rank.astype(np.float64))[None, :]
    elif shape.routing != "uniform":
        raise ValueError(shape.routing)
    ids = np.empty((shape.T, shape.k), dtype=np.int32)
    w = np.empty((shape.T, shape.k), dtype=np.float32)
    eidx = np.arange(shape.E)
    for t in range(shape.T):
        order = np.lexsort((eidx, -logits[t]))[: shape.k]
        z = logits[t] - logits[t].max()
        p = np.exp(z) / np.exp(z).sum()
        ids[t] = order
        w[t] = (p[order] / p[order].sum()).astype(np.float32)
    return ids, w


def gen_expert(cfg_id: int, e: int, proj: int, shape: MoeShape | None = None):
    """One row-major NVFP4 projection: (packed uint8 [N, K/2], scale uint8 [N, K/16])."""
    shape = shape or config(cfg_id)
    n, k = proj_dims(shape, proj)
    packed = _rng(cfg_id, 4, e, proj).integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    u = _rng(cfg_id, 5, e, proj).uniform(2.0 ** -4, 4.0, size=(n, k // 16)).astype(np.float32)
    scale = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return packed, scale


def gen_expert_mx(cfg_id: int, e: int, proj: int, shape: MoeShape | None = None):
    """One row-major MXFP4 projection: (packed uint8 [N, K/2], E8M0 scale codes uint8 [N, K/32])."""
    shape = shape or config(cfg_id)
    n, k = proj_dims(shape, proj)
    packed = _rng(cfg_id, 4, e, proj).integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    u = _rng(cfg_id, 6, e, proj).uniform(2.0 ** -4, 4.0, size=(n, k // 32))
    scale = (127 - 11 + np.floor(np.log2(u) + 0.5)).astype(np.uint8)
    return packed, scale
