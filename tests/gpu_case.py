"""Device-side test cases built from the seeded generators.

A ``Case`` uploads one workload's inputs (x, routing, the experts' NVFP4 or
MXFP4 weights) to the GPU, builds the pointer tables, and runs the four C-ABI
calls through ``MoeLayer``.  The oracle side regenerates any expert's bytes
from the same seeds on the CPU (``weight_fn``), so only what a check needs is
ever dequantised.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import nvfp4_quantized_moe_amd as moe
import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Case:
    def __init__(self, cfg_id: int, shape: synth.MoeShape | None = None, nulls=(), kmajor: bool | None = None,
                 ids: np.ndarray | None = None, weights: np.ndarray | None = None, all_experts: bool = False,
                 fmt: str = "nvfp4", gen=None, concat: bool = False):
        self.cfg_id = cfg_id
        self.shape = shape or synth.config(cfg_id)
        s = self.shape
        self.kmajor = s.kmajor if kmajor is None else kmajor
        # Weight format: NVFP4 (E4M3 per 16) or MXFP4 (E8M0 per 32, K-major only).
        self.fmt = fmt
        mx = fmt == "mxfp4"
        assert not mx or self.kmajor
        self.gen = gen or (synth.gen_expert_mx if mx else synth.gen_expert)
        group = 32 if mx else 16
        self.x_bits = synth.gen_x(cfg_id, s)
        gids, gw = synth.gen_routing(cfg_id, s)
        self.ids = gids if ids is None else ids.astype(np.int32)
        self.w = gw if weights is None else weights.astype(np.float32)
        self.nulls = set(nulls)
        flat = self.ids.reshape(-1)
        self.active = sorted({int(e) for e in flat if 0 <= e < s.E})
        need = range(s.E) if all_experts else self.active
        self.dev = {}
        for e in need:
            if e in self.nulls:
                continue
            for proj in (0, 1, 2):
                n, k = synth.proj_dims(s, proj)
                pk, sc = self.gen(cfg_id, e, proj, s)
                pk_d = torch.from_numpy(pk).cuda()
                sc_d = torch.from_numpy(sc).cuda()
                if self.kmajor:
                    pk_d, sc_d = moe.transpose_for_gemm(pk_d, sc_d, n, k, group)
                self.dev[(e, proj)] = (pk_d, sc_d)
        s2 = synth.SCALE2_MX_F32 if mx else synth.SCALE2_F32
        self.scale2 = {p: np.float32(s2) for p in (0, 1, 2)}
        self.tables = [self._table(p, self.layout) for p in (0, 1, 2)]
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        self.ids_d = torch.from_numpy(self.ids).cuda()
        self.w_d = torch.from_numpy(self.w).cuda()
        # Optional concatenated gate||up twin per expert (K-major only), built
        # from the row-major bytes with the pitched transpose.
        self.concat = concat
        self.pitch = 0
        gate_up = None
        if concat:
            assert self.kmajor
            rows = []
            for e in range(s.E):
                if (e, 0) not in self.dev:
                    rows.append(None)
                    continue
                parts = []
                for proj in (0, 1):
                    pk, sc = self.gen(cfg_id, e, proj, s)
                    parts.append((torch.from_numpy(pk).cuda(), torch.from_numpy(sc).cuda(), s.I))
                pt, st, self.pitch = moe.transpose_concat_for_gemm(parts, s.H, group, align=16)
                self.dev[(e, "gate_up")] = (pt, st)
                rows.append((pt, st, self.scale2[0]))
            gate_up = moe.ExpertTables(rows, self.layout)
        self.layer = moe.MoeLayer(s.T, s.k, s.E, s.H, s.I, *self.tables, gate_up=gate_up, pitch=self.pitch)

    def _table(self, proj, layout):
        rows = []
        for e in range(self.shape.E):
            t = self.dev.get((e, proj))
            rows.append(None if t is None else (t[0], t[1], self.scale2[proj]))
        return moe.ExpertTables(rows, layout)

    @property
    def layout(self) -> int:
        if self.fmt == "mxfp4":
            return moe.K_MAJOR_MXFP4
        return moe.K_MAJOR if self.kmajor else moe.ROW_MAJOR

    def set_scale2(self, proj: int, value: float):
        self.scale2[proj] = np.float32(value)
        self.tables[proj] = self._table(proj, self.layout)
        self.layer.gate, self.layer.up, self.layer.down = self.tables

    # oracle-side weights (row-major numpy, regenerated from the seeds)
    def weight_fn(self):
        s = self.shape

        def fn(e, proj):
            if e in self.nulls:
                return None
            pk, sc = self.gen(self.cfg_id, e, proj, s)
            return pk, sc, self.scale2[proj]

        return fn

    def run(self, fuse_blend: bool = False):
        """One forward; by default down and blend as two calls, so y is there
        to check."""
        self.layer.err_flag.zero_()
        out = self.layer.forward(self.x, self.ids_d, self.w_d, fuse_blend=fuse_blend)
        torch.cuda.synchronize()
        return out

    def sort_outputs(self) -> dict:
        L = self.layer
        n = int(L.active_count.item())
        return {
            "expert_offsets": L.expert_offsets.cpu().numpy(),
            "sorted_token_ids": L.sorted_token_ids.cpu().numpy(),
            "pair_pos": L.pair_pos.cpu().numpy(),
            "active_experts": L.active_experts.cpu().numpy(),
            "active_count": n,
            "err": int(L.err_flag.item()),
        }
