"""Benchmark of the grouped NVFP4 MoE expert projection on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload N] [--eager] [--format nvfp4|mxfp4]
                    [--gate-up separate|concat]

A step is one MoE layer forward through the whole path — routing sort,
gate+up+SiLU, down, blend — over one batch of synthetic input (at one
token the sort runs inside the gate+up launch and the blend inside the down
launch).  Every input is resident in HBM before timing starts.  Consecutive
steps run different layers' expert weights (separate HBM copies, as
successive layers of a model would), so the weights a step reads were last
touched far more than the 256 MB Infinity Cache ago: the measured bandwidth
is HBM bandwidth.

With no --workload the line covers both halves of the metric: the 1-token
decode workload (the top-level fields) and the 32-token decode workload
(the ``decode_batch_32`` block, same fields).  --workload N measures that
workload alone.

The K timed steps are captured into one HIP graph.  It is replayed once
untimed (the first replay of a graph also uploads it).  Then, queued back
to back behind a one-wave spin kernel of about a millisecond (which covers
the host's submission of everything after it): a 1 GiB buffer read once
through the streaming-read kernel to evict the caches, the W warm-up steps
again (other weight copies than the timed ones), one read of every routing
batch's inputs (x, expert ids, weights, as the router and the previous
layer would just have written them), the start event, the timed replay and
the end event (``--eager`` launches the steps one by one instead).  The
eviction reads rather than writes: a rewritten buffer left the Infinity
Cache full of dirty lines, whose write-back slowed the first dozen steps
after it (a 20-step replay of the 1-token step measured 20.0 us per step
against 17.1 us over 2000 steps; with the read and the warm-up replay,
18.0 us).  ``--warm-cache`` (context only, labelled in config.cache) keeps
one weight copy and skips the eviction.  Reported on one JSON line, per
workload:
  value       expert-weight bytes of the active experts per step / step time (GB/s)
  tokens_per_s, pct_of_hbm_peak
  dtype       the arithmetic: f16 (decode: fp16 matrix-core operands, fp32
              accumulation) or bf16/f16 (many-token: bf16 gate+up, fp16 down)
  roofline    the dominant kernel (gate+up+SiLU, with the routing sort fused
              in where the step runs it that way: one token): its
              algorithmic bytes per launch / its mean launch duration, timed
              with HIP events on the stream it runs on, against 8 TB/s (the
              many-token K-major workload: its flops per launch against the
              2.5 PFLOP/s fp16/bf16 matrix-core peak); traffic = HBM bytes per
              launch from the committed counter summary in profiles/ while
              the kernel sources are unchanged since it was taken, else null
  projection_launches  the down launch the step runs (HIP events, as for
              roofline) and the expert-weight bytes over the gate+up and down
              launch times alone (sort, blend and launch gaps excluded)
  router      launch time of moe_nvfp4_route on the workload's logits (the
              router ahead of the path; not part of the step)
  cpu_baseline the fp64 oracle on the host cores for a bounded sample of the
              same workload, in the same unit
  cpu_oracle_1thread (top level) the oracle with BLAS held to one thread on
              one forward of each of the tiny, 1-token and 32-token workloads
  --format mxfp4 runs the many-token workload with MXFP4 experts (E8M0
  scales per 32 k) instead of NVFP4; --gate-up concat runs its gate+up over
  one concatenated gate||up twin per expert; the workload name says so.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix-core peak
METRIC = "expert-weight HBM GB/s (% of peak) + MoE-layer tokens/s, decode batch 1/32"
SPIN_CYCLES = 2_500_000  # a one-wave spin of about 1 ms ahead of each timed region


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=None,
                    help="workload id 1..5 (default: 2, the 1-token decode, with 3, the 32-token decode, as a block)")
    ap.add_argument("--layers", type=int, default=0, help="weight copies cycled over (0 = auto)")
    ap.add_argument("--batches", type=int, default=8, help="distinct routing batches cycled over")
    ap.add_argument("--eager", action="store_true", help="launch step by step instead of one graph")
    ap.add_argument("--format", choices=["nvfp4", "mxfp4"], default="nvfp4",
                    help="expert weight format (mxfp4: K-major workloads only)")
    ap.add_argument("--gate-up", choices=["separate", "concat"], default="separate",
                    help="gate and up as two K-major twins, or one concatenated twin (K-major workloads only)")
    ap.add_argument("--warm-cache", action="store_true",
                    help="context only, labelled as such: one weight copy and no cache eviction, so the step "
                         "reads its weights from wherever the caches hold them")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--measure", choices=["stream", "transpose"], default=None,
                    help="instead of the step: the streaming-read ceiling over a 4 GiB buffer "
                         "(moe_nvfp4_stream_read), or transpose_u8 over the many-token workload's weights")
    ap.add_argument("--profile-pass", choices=["gate_up", "down", "down_blend", "copy"], default=None,
                    help="for counter runs under rocprofv3: launch only gate+up+SiLU (after one sort), or "
                         "only the down projection, or only the down projection with the blend fused in "
                         "(each after one sort and gate+up), --steps times, or a plain 1 GiB device copy "
                         "--steps times, then exit")
    return ap.parse_args()


KERNEL_SOURCES = ("nvfp4_quantized_moe_amd/csrc/moe_decode_row.hip",
                  "nvfp4_quantized_moe_amd/csrc/moe_gemm_kmajor.hip",
                  "nvfp4_quantized_moe_amd/csrc/moe_common.hpp")


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    an edit to a comment does not invalidate the counters."""
    import hashlib
    import re

    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate+up launch from the committed counter summary of this
    workload (profiles/traffic_<workload>.txt), or None when there is none or
    the kernel sources changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def active_weight_bytes(shape, ids, group: int = 16) -> int:
    import synth

    act = np.unique(ids[(ids >= 0) & (ids < shape.E)])
    return int(act.size) * synth.expert_bytes(shape, group)


def gate_up_bytes(shape, ids, group: int = 16) -> int:
    """Algorithmic bytes of one gate+up launch: the active experts' gate and up
    weights (packed + scales), x read once, h written once, 4-byte scale_2s."""
    act = np.unique(ids[(ids >= 0) & (ids < shape.E)]).size
    w = act * 2 * (shape.I * shape.H // 2 + shape.I * shape.H // group + 4)
    return int(w + shape.T * shape.H * 2 + shape.P * shape.I * 4)


def cpu_baseline(shape, cfg_id, seconds, fmt="nvfp4"):
    """Time the fp64 oracle on a bounded sample: whole layer forwards of the
    same workload (tokens sampled down for the many-token workload)."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info

        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = int(max(blas)) if blas else 1
    except Exception:  # pragma: no cover
        cores = 1
    T = shape.T if shape.T <= 64 else 64
    sub = synth.MoeShape(shape.name + "_cpu", T, shape.H, shape.I, shape.E, shape.k, shape.routing, False,
                         shape.zipf_s)

    mx = fmt == "mxfp4"
    group = 32 if mx else 16

    def wf(e, proj):
        if mx:
            pk, sc = synth.gen_expert_mx(cfg_id, e, proj, shape)
            return pk, sc, synth.SCALE2_MX_F32
        pk, sc = synth.gen_expert(cfg_id, e, proj, shape)
        return pk, sc, synth.SCALE2_F32

    done_tokens, done_bytes, t_used, runs = 0, 0, 0.0, 0
    b = 0
    while t_used < seconds and runs < 50:
        x = synth.gen_x(cfg_id, shape, batch=b)[:T]
        ids, w = synth.gen_routing(cfg_id, shape, batch=b)
        ids, w = ids[:T], w[:T]
        # weight bytes are generated outside the timed region; decode + compute inside
        cache = {}
        for e in np.unique(ids):
            for p in (0, 1, 2):
                cache[(int(e), p)] = wf(int(e), p)
        t0 = time.perf_counter()
        oracle.moe_layer(x, ids, w, lambda e, p: cache[(e, p)], sub.E, sub.H, sub.I, fmt=fmt)
        t_used += time.perf_counter() - t0
        done_tokens += T
        done_bytes += active_weight_bytes(sub, ids, group)
        runs += 1
        b += 1
    return {
        "value": round(done_bytes / t_used / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(done_tokens / t_used, 3),
        "cores": cores,
        "kind": "oracle",
        "sample": f"{runs} fp64 oracle layer forwards of {T} token(s) each (dequant + sort + gate/up + down + blend, "
                  f"weights generated outside the timing), {t_used:.1f} s of CPU time; numpy elementwise work on "
                  f"1 thread, BLAS on up to {cores}",
    }


def cpu_oracle_1thread():
    """The oracle with BLAS held to one thread (numpy's elementwise work is
    single-threaded anyway): one layer forward of each of the tiny, 1-token
    and 32-token decode workloads, weights generated outside the timing."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits

    res = {}
    with threadpool_limits(limits=1):
        for cfg_id in (1, 2, 3):
            shape = synth.config(cfg_id)
            x = synth.gen_x(cfg_id, shape)
            ids, w = synth.gen_routing(cfg_id, shape)
            cache = {(int(e), p): (*synth.gen_expert(cfg_id, int(e), p, shape), synth.SCALE2_F32)
                     for e in np.unique(ids) for p in (0, 1, 2)}
            t0 = time.perf_counter()
            oracle.moe_layer(x, ids, w, lambda e, p: cache[(e, p)], shape.E, shape.H, shape.I)
            dt = time.perf_counter() - t0
            res[shape.name] = {"seconds_per_forward": round(dt, 3),
                               "value": round(active_weight_bytes(shape, ids) / dt / 1e9, 4), "unit": "GB/s",
                               "tokens_per_s": round(shape.T / dt, 3), "cores": 1}
    return res


def flush_caches(dev, scratch=[]):
    """Read a 1 GiB device buffer once with the library's streaming-read
    kernel (more than the 256 MB Infinity Cache and the L2s together), so the
    next step finds nothing of its weights cached and no dirty line to write
    back."""
    import torch

    import nvfp4_quantized_moe_amd as moe

    if not scratch:
        scratch.append(torch.ones(1 << 30, dtype=torch.uint8, device=dev))
        scratch.append(torch.zeros(1, dtype=torch.int32, device=dev))
    moe.moe_nvfp4_stream_read(scratch[0], scratch[1])


def touch_inputs(tensors, sink=[]):
    """Read every routing batch's activations, expert ids and weights once
    (the streaming-read kernel), as the router and the previous layer would
    have just written them: after the eviction only the expert weights of
    the timed steps should come from HBM."""
    import torch

    import nvfp4_quantized_moe_amd as moe

    for t in tensors:
        if not sink:
            sink.append(torch.zeros(1, dtype=torch.int32, device=t.device))
        nbytes = t.numel() * t.element_size()
        if nbytes >= 16 and nbytes % 16 == 0:
            moe.moe_nvfp4_stream_read(t.view(-1), sink[0])


def measure(args, cfg_id, K, W):
    """One workload: build its inputs and weight copies, time K steps, and
    return its fields of the JSON line."""
    import torch

    import nvfp4_quantized_moe_amd as moe
    import synth

    dev = torch.device("cuda:0")
    shape = synth.config(cfg_id)
    mx = args.format == "mxfp4"
    if mx and not shape.kmajor:
        sys.exit("bench.py: --format mxfp4 runs on the K-major (many-token) workload only")
    group = 32 if mx else 16
    scale2 = synth.SCALE2_MX_F32 if mx else synth.SCALE2_F32
    gen = synth.gen_expert_mx if mx else synth.gen_expert
    concat = args.gate_up == "concat"
    if concat and not shape.kmajor:
        sys.exit("bench.py: --gate-up concat runs on the K-major (many-token) workload only")
    if mx:
        shape = dataclasses.replace(shape, name=shape.name + "_mxfp4")
        layout = moe.K_MAJOR_MXFP4
    else:
        layout = moe.K_MAJOR if shape.kmajor else moe.ROW_MAJOR
    if concat:
        shape = dataclasses.replace(shape, name=shape.name + "_concat")

    # ---- inputs: R routing batches, L layers of expert weights -----------
    R = max(1, args.batches)
    xs, idss, ws = [], [], []
    for b in range(R):
        xs.append(torch.from_numpy(synth.gen_x(cfg_id, shape, batch=b).view(np.int16)).to(dev).view(torch.bfloat16))
        ids, w = synth.gen_routing(cfg_id, shape, batch=b)
        idss.append(ids)
        ws.append(w)
    ids_d = [torch.from_numpy(i).to(dev) for i in idss]
    w_d = [torch.from_numpy(w).to(dev) for w in ws]
    step_bytes = [active_weight_bytes(shape, i, group) for i in idss]
    all_bytes = shape.E * synth.expert_bytes(shape, group)
    if args.warm_cache:
        L = 1
    elif args.layers > 0:
        L = args.layers
    else:
        L = max(1, math.ceil(2.0e9 / min(step_bytes)))
        L = min(L, 64, max(1, int(48e9 // all_bytes)))
    base = {}
    for e in range(shape.E):
        for p in (0, 1, 2):
            n, k = synth.proj_dims(shape, p)
            pk, sc = gen(cfg_id, e, p, shape)
            pk_d, sc_d = torch.from_numpy(pk).to(dev), torch.from_numpy(sc).to(dev)
            if shape.kmajor:
                pk_d, sc_d = moe.transpose_for_gemm(pk_d, sc_d, n, k, group)
            base[(e, p)] = (pk_d, sc_d)
    pitch = 0
    if concat:
        for e in range(shape.E):
            parts = [(torch.from_numpy(pk).to(dev), torch.from_numpy(sc).to(dev), shape.I)
                     for pk, sc in (gen(cfg_id, e, p, shape) for p in (0, 1))]
            pt, st, pitch = moe.transpose_concat_for_gemm(parts, shape.H, group, align=16)
            base[(e, "gu")] = (pt, st)
    layers = []
    for li in range(L):
        wts = base if li == 0 else {key: (a.clone(), b.clone()) for key, (a, b) in base.items()}
        tabs = [moe.ExpertTables([(wts[(e, p)][0], wts[(e, p)][1], scale2) for e in range(shape.E)],
                                 layout, device=dev) for p in (0, 1, 2)]
        gu = None
        if concat:
            gu = moe.ExpertTables([(wts[(e, "gu")][0], wts[(e, "gu")][1], scale2) for e in range(shape.E)],
                                  layout, device=dev)
        layers.append((wts, tabs, gu))
    bufs = moe.MoeLayer(shape.T, shape.k, shape.E, shape.H, shape.I, *layers[0][1], device=dev,
                        gate_up=layers[0][2], pitch=pitch)

    # The gate+up launch the step runs: at few tokens the sort is fused into
    # it (one kernel), which is then the launch timed and profiled.
    fused_sort = (not concat) and moe.moe_nvfp4_sort_gate_up_launches(shape.T, shape.k, shape.E, shape.H, shape.I,
                                                                      layout) == 1

    def gate_up_launch(li, s):
        tabs, gu = layers[li % L][1], layers[li % L][2]
        if fused_sort:
            moe.moe_nvfp4_sort_gate_up_silu(ids_d[0], xs[0], shape.E, shape.H, shape.I, tabs[0], tabs[1],
                                            bufs.expert_offsets, bufs.sorted_token_ids, bufs.pair_pos,
                                            bufs.active_experts, bufs.active_count, bufs.err_flag, bufs.h, s)
        elif gu is not None:
            moe.moe_nvfp4_gate_up_silu_concat(xs[0], shape.k, shape.E, shape.H, shape.I, gu, pitch,
                                              bufs.expert_offsets, bufs.sorted_token_ids, bufs.active_experts,
                                              bufs.active_count, bufs.h, s)
        else:
            moe.moe_nvfp4_gate_up_silu(xs[0], shape.k, shape.E, shape.H, shape.I, tabs[0], tabs[1],
                                       bufs.expert_offsets, bufs.sorted_token_ids, bufs.active_experts,
                                       bufs.active_count, bufs.h, s)

    def sort_launch(s):
        moe.moe_nvfp4_sort(ids_d[0], shape.E, bufs.expert_offsets, bufs.sorted_token_ids, bufs.pair_pos,
                           bufs.active_experts, bufs.active_count, bufs.err_flag, s)

    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    if args.profile_pass == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                dst.copy_(src)
        torch.cuda.synchronize()
        return None
    if args.profile_pass in ("gate_up", "down", "down_blend"):
        with torch.cuda.stream(stream):
            sort_launch(stream)
            if args.profile_pass != "gate_up":
                gate_up_launch(0, stream)
            for i in range(args.steps):
                dn = layers[i % L][1][2]
                if args.profile_pass == "gate_up":
                    gate_up_launch(i, stream)
                elif args.profile_pass == "down":
                    moe.moe_nvfp4_down(bufs.h, shape.T, shape.k, shape.E, shape.H, shape.I, dn,
                                       bufs.expert_offsets, bufs.active_experts, bufs.active_count, bufs.y, stream)
                else:
                    moe.moe_nvfp4_down_blend(bufs.h, ids_d[0], w_d[0], bufs.pair_pos, shape.E, shape.H, shape.I, dn,
                                             bufs.out, stream)
        torch.cuda.synchronize()
        return None

    def step(i, s):
        bufs.gate, bufs.up, bufs.down = layers[i % L][1]
        bufs.gate_up = layers[i % L][2]
        b = i % R
        bufs.forward(xs[b], ids_d[b], w_d[b], stream=s)

    def run_steps(first, n, s):
        for i in range(first, first + n):
            step(i, s)

    with torch.cuda.stream(stream):
        run_steps(0, min(W, 3), stream)  # plain warm launch before any capture
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if args.eager:
        if not args.warm_cache:
            flush_caches(dev)
        with torch.cuda.stream(stream):
            run_steps(0, W, stream)
        touch_inputs(xs + ids_d + w_d)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(SPIN_CYCLES)
            t_start.record(stream)
            run_steps(W, K, stream)
            t_end.record(stream)
        torch.cuda.synchronize()
    else:
        # Warm-up steps run as their own graph; the timed graph is replayed
        # once untimed (its first replay uploads it), the caches are flushed,
        # the warm-up graph runs again, and the timed graph's next replay is
        # timed.
        g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream):
            run_steps(0, max(W, 1), stream)
        with torch.cuda.graph(g_main, stream=stream):
            run_steps(W, K, stream)
        torch.cuda.synchronize()
        g_warm.replay()
        g_main.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            # The GPU spins for about a millisecond while the host submits
            # the eviction, the warm-up replay, the input reads and the timed
            # graph, so these run back to back and the timed region holds
            # the K steps, not the submission latency of the replay.
            torch.cuda._sleep(SPIN_CYCLES)
            if not args.warm_cache:
                flush_caches(dev)
            g_warm.replay()
            touch_inputs(xs + ids_d + w_d)
            t_start.record(stream)
            g_main.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    bytes_timed = sum(step_bytes[i % R] for i in range(W, W + K))
    value = bytes_timed / (total_ms / 1e3) / 1e9
    tokens_per_s = shape.T * K / (total_ms / 1e3)

    # ---- dominant kernel: gate+up+SiLU launch duration.  HIP events on the
    # stream it runs on bracket Kr back-to-back launches (one routing batch,
    # the weight copies cycled as in the timed steps); the mean per launch
    # includes the short gap between consecutive launches.
    Kr = min(max(K, 50), 200)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        sort_launch(stream)
        for rep in range(2):  # the first pass warms the launch path
            e0.record(stream)
            for i in range(Kr):
                gate_up_launch(i, stream)
            e1.record(stream)
    torch.cuda.synchronize()
    gu_ms = e0.elapsed_time(e1) / Kr
    gu_bytes = float(gate_up_bytes(shape, idss[0], group)) + (shape.P * 4 if fused_sort else 0)
    traffic = measured_traffic(shape.name)
    if shape.kmajor:
        # Many-token path: a dense contraction on the matrix cores.
        flops = 4.0 * shape.P * shape.I * shape.H  # gate and up, 2 flops per MAC
        roof = {"bound": "mfma", "achieved": round(flops / (gu_ms / 1e3) / 1e12, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        roof["frac"] = round(roof["achieved"] / MFMA_F16_PEAK_TFLOPS, 4)
        roof["algorithmic_flops_per_launch"] = round(flops)
    else:
        achieved = gu_bytes / (gu_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    kname = "moe_nvfp4_sort_gate_up_silu (sort fused in)" if fused_sort else "moe_nvfp4_gate_up_silu"
    roof.update({"traffic": traffic, "kernel": kname, "launch_us": round(gu_ms * 1e3, 3),
                 "algorithmic_bytes_per_launch": round(gu_bytes)})

    # ---- the down launch the step runs (with the blend fused in at one
    # token with row-major weights), timed the same way after one gate+up.
    fused_blend = shape.T == 1 and not shape.kmajor
    with torch.cuda.stream(stream):
        gate_up_launch(0, stream)
        for rep in range(2):
            e0.record(stream)
            for i in range(Kr):
                dn = layers[i % L][1][2]
                if fused_blend:
                    moe.moe_nvfp4_down_blend(bufs.h, ids_d[0], w_d[0], bufs.pair_pos, shape.E, shape.H, shape.I, dn,
                                             bufs.out, stream)
                else:
                    moe.moe_nvfp4_down(bufs.h, shape.T, shape.k, shape.E, shape.H, shape.I, dn, bufs.expert_offsets,
                                       bufs.active_experts, bufs.active_count, bufs.y, stream)
            e1.record(stream)
    torch.cuda.synchronize()
    dn_ms = e0.elapsed_time(e1) / Kr
    # Expert-weight bytes over the two projection launches alone (sort,
    # blend and launch gaps excluded), beside value's whole-step rate.
    kernels = {"down_kernel": "moe_nvfp4_down_blend (blend fused in)" if fused_blend else "moe_nvfp4_down",
               "down_launch_us": round(dn_ms * 1e3, 3),
               "weight_GBps_over_gate_up_and_down_launches": round(step_bytes[0] / ((gu_ms + dn_ms) / 1e3) / 1e9, 1)}

    # ---- the router ahead of the path (softmax, top-k, renormalise), timed
    # on its own over the workload's logits; it is not part of the step.
    logits_d = torch.from_numpy(synth.gen_logits(cfg_id, shape)).to(dev)
    r_ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device=dev)
    r_w = torch.empty((shape.T, shape.k), dtype=torch.float32, device=dev)
    Kq = 100
    with torch.cuda.stream(stream):
        for rep in range(2):
            e0.record(stream)
            for i in range(Kq):
                moe.moe_nvfp4_route(logits_d, shape.k, r_ids, r_w, stream)
            e1.record(stream)
    torch.cuda.synchronize()
    router = {"kernel": "moe_nvfp4_route", "launch_us": round(e0.elapsed_time(e1) / Kq * 1e3, 3),
              "in_step": False}

    block = {
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 6),
        "dtype": "bf16/f16" if shape.kmajor else "f16",
        "accumulate": "f32",
        "config": {
            "workload": shape.name,
            "tokens": shape.T, "hidden": shape.H, "expert_inter": shape.I, "experts": shape.E, "top_k": shape.k,
            "routing": shape.routing, "weight_layout": "k_major" if shape.kmajor else "row_major",
            "weight_format": args.format, "gate_up_twin": args.gate_up if shape.kmajor else "row_major",
            "weight_copies_cycled": L, "routing_batches_cycled": R,
            "launch": "eager" if args.eager else "hip_graph",
            "cache": "warm (one weight copy, no eviction)" if args.warm_cache else "cold (weights from HBM)",
        },
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "active_weight_bytes_per_step": round(bytes_timed / K),
        "roofline": roof,
        "projection_launches": kernels,
        "router": router,
        "cpu_baseline": None,
    }
    del layers, base, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        block["cpu_baseline"] = cpu_baseline(shape, cfg_id, args.cpu_seconds, args.format)
    return block


def measure_aux(args):
    """--measure: the streaming-read ceiling, or the load-time transpose's
    throughput on the many-token workload's 192 weights (64 experts x gate,
    up, down: packed and scale tensors), as GB/s of bytes read + written."""
    import torch

    import nvfp4_quantized_moe_amd as moe
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.measure == "stream":
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        buf.fill_(7)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        reps = 20
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(3):
                moe.moe_nvfp4_stream_read(buf, sink, stream)
            e0.record(stream)
            for _ in range(reps):
                moe.moe_nvfp4_stream_read(buf, sink, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return {"measure": "stream_read", "bytes_per_launch": nbytes, "launch_us": round(ms * 1e3, 2),
                "GBps": round(nbytes / (ms / 1e3) / 1e9, 1), "pct_of_8TBps": round(nbytes / (ms / 1e3) / 8e12 * 100, 1),
                "launches": reps}
    cfg = 5
    shape = synth.config(cfg)
    jobs = []
    for e in range(shape.E):
        for p in (0, 1, 2):
            n, k = synth.proj_dims(shape, p)
            pk, sc = synth.gen_expert(cfg, e, p, shape)
            for src, rows, cols in ((pk, n, k // 2), (sc, n, k // 16)):
                s_d = torch.from_numpy(src).to(dev)
                jobs.append((s_d, torch.empty((cols, rows), dtype=torch.uint8, device=dev), rows, cols))
    moved = 2 * sum(r * c for _, _, r, c in jobs)
    reps = 5
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for s_d, d_d, r, c in jobs:
            moe.transpose_u8(s_d, d_d, r, c, stream)
        e0.record(stream)
        for _ in range(reps):
            for s_d, d_d, r, c in jobs:
                moe.transpose_u8(s_d, d_d, r, c, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"measure": "transpose_u8", "workload": shape.name, "launches_per_pass": len(jobs),
            "bytes_read_plus_written_per_pass": moved, "pass_us": round(ms * 1e3, 1),
            "GBps": round(moved / (ms / 1e3) / 1e9, 1), "pct_of_8TBps": round(moved / (ms / 1e3) / 8e12 * 100, 1)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the path runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_quantized_moe_amd as moe

    if not torch.cuda.is_available():
        sys.exit("bench.py: no GPU")
    moe.lib()  # fail loudly when the HIP library is missing
    if args.measure:
        print(json.dumps(measure_aux(args)), flush=True)
        return
    K, W = args.steps, args.warmup
    first = args.workload if args.workload is not None else 2
    main_block = measure(args, first, K, W)
    if main_block is None:  # a profiling pass
        return
    line = {"metric": METRIC, "value": main_block.pop("value"), "unit": main_block.pop("unit"), "n_gpus": 1,
            "steps": K, "warmup": W, "ms_per_step": main_block.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": main_block.pop("dtype"), "data": "synthetic"}
    line.update(main_block)
    if args.workload is None:
        line["decode_batch_32"] = measure(args, 3, K, W)
        if not args.no_cpu_baseline:
            line["cpu_oracle_1thread"] = cpu_oracle_1thread()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
