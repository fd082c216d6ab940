"""GPU parity: every kernel of the path against the fp64 oracle, through the C ABI.

Integer outputs (sort, transpose) must match bit for bit; floating outputs
must pass both the official and the strict rule of ``tests/parity.py``.
Sizes: every workload is compared element by element at its full size; the
largest decode workload (64 tokens, E=256, 5.5 GB of weights) runs in the
same launch configuration the benchmark uses, its oracle spread over a
thread pool one expert per task.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import nvfp4_quantized_moe_amd as moe
import oracle
import synth
from tests import parity
from tests.gpu_case import Case, say

pytestmark = pytest.mark.gpu


def _h2f(t):
    return t.detach().float().cpu().numpy().astype(np.float64)  # may hold untouched rows


def _check_sort(case, ref):
    got = case.sort_outputs()
    for key in ("expert_offsets", "sorted_token_ids", "pair_pos", "active_experts"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["active_count"] == ref["active_count"]
    assert got["err"] == ref["err"]


def _full_check(case, tag):
    s = case.shape
    case.run()
    ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), s.E, s.H, s.I, kmajor=False,
                           fmt=case.fmt)
    _check_sort(case, ref)
    n = int(ref["expert_offsets"][-1])
    eh = parity.assert_parity(_h2f(case.layer.h)[:n], ref["h"][:n], f"{tag} h")
    ey = parity.assert_parity(_h2f(case.layer.y)[:n], ref["y"][:n], f"{tag} y")
    eo = parity.assert_parity(_h2f(case.layer.out), ref["out"], f"{tag} out")
    say(tag, "h", eh, "y", ey, "out", eo)
    return ref


# ---------------------------------------------------------------- transpose_u8
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (64, 64), (70, 130), (1536, 2048), (1536, 256),
                                       (4096, 768), (4096, 96), (1856, 116), (33, 4000)])
def test_transpose_u8_bit_exact(rows, cols):
    say("transpose_u8", rows, cols)
    rng = np.random.default_rng(rows * 7919 + cols)
    a = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    src = torch.from_numpy(a).cuda()
    dst = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    moe.transpose_u8(src, dst, rows, cols)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), oracle.transpose_u8(a))
    assert np.array_equal(src.cpu().numpy(), a)   # input untouched


# ---------------------------------------------------------------- sort
def _run_sort(ids, E):
    T, k = ids.shape
    d = torch.from_numpy(ids.astype(np.int32)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = [torch.full((E + 1,), 7, **i32), torch.full((T * k,), 7, **i32), torch.full((T * k,), 7, **i32),
            torch.full((E,), 7, **i32), torch.full((1,), 7, **i32), torch.zeros(1, **i32)]
    moe.moe_nvfp4_sort(d, E, *outs)
    torch.cuda.synchronize()
    o = [t.cpu().numpy() for t in outs]
    return {"expert_offsets": o[0], "sorted_token_ids": o[1], "pair_pos": o[2], "active_experts": o[3],
            "active_count": int(o[4][0]), "err": int(o[5][0])}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_sort_configs_bit_exact(cfg):
    say("sort cfg", cfg)
    s = synth.config(cfg)
    ids, _ = synth.gen_routing(cfg)
    got, ref = _run_sort(ids, s.E), oracle.sort_routes(ids, s.E)
    for key in ("expert_offsets", "sorted_token_ids", "pair_pos", "active_experts", "active_count", "err"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("T,k,E,mode", [(1, 1, 1, "rand"), (3, 4, 5, "dup"), (9, 3, 7, "invalid"),
                                         (16384, 8, 256, "rand"), (2048, 4, 1024, "rand"), (512, 1, 1024, "skew"),
                                         (100, 8, 8, "all_same"), (1000, 3, 50, "rand"),
                                         (5000, 7, 300, "invalid"), (1 << 19, 8, 1024, "rand"),
                                         (65, 1, 7, "rand"), (16, 8, 40, "dup"), (32, 6, 128, "invalid"),
                                         (85, 3, 3, "invalid"), (51, 5, 1024, "rand"), (64, 4, 9, "all_same"),
                                         (257, 1, 33, "rand")])
def test_sort_edge_cases_bit_exact(T, k, E, mode):
    """Includes the maximum sizes: 2^22 pairs (MOE_NVFP4_MAX_PAIRS) over 1024
    experts (MOE_NVFP4_MAX_EXPERTS), and pair counts on both sides of the
    single-block kernel's 64-pairs-per-wave boundaries (65 .. 257)."""
    say("sort edge", T, k, E, mode)
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if mode == "dup":
        ids[1, :] = 3
    elif mode == "invalid":
        ids[0, 1] = E
        ids[5, 0] = -7
        ids[8, 2] = 1 << 30
    elif mode == "skew":
        ids[:, 0] = np.minimum(rng.zipf(1.5, T) - 1, E - 1)
    elif mode == "all_same":
        ids[:] = 5
    got, ref = _run_sort(ids, E), oracle.sort_routes(ids, E)
    for key in ("expert_offsets", "sorted_token_ids", "pair_pos", "active_experts", "active_count", "err"):
        assert np.array_equal(got[key], ref[key]), key


# ---------------------------------------------------------------- whole layer
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_layer_decode_configs(cfg):
    say("layer cfg", cfg)
    _full_check(Case(cfg), f"cfg{cfg}")


def test_layer_prefill_kmajor_full():
    say("layer cfg 5 (K-major, 2048 tokens)")
    _full_check(Case(5), "cfg5")


def test_layer_decode64_full_size():
    """64 tokens, H=7168, I=2048, E=256, top-8: the full layer on the GPU in
    the launch configuration the benchmark uses (about 220 active experts,
    5.5 GB of weights: persistent gate+up, nontemporal weight loads for the
    experts read by one pass) against the oracle on every routed pair's h and
    y row and every token's output row.  The oracle's per-expert work (its
    own dequantisation, gate+up and down functions, as in moe_layer) runs on
    a thread pool, one independent expert per task."""
    say("layer cfg 4 full size, whole layer")
    case = Case(4)
    s = case.shape
    case.run()
    ref_sort = oracle.sort_routes(case.ids, s.E)
    _check_sort(case, ref_sort)
    x = oracle.bf16_bits_to_f64(case.x_bits)
    wf = case.weight_fn()
    offs, tok = ref_sort["expert_offsets"], ref_sort["sorted_token_ids"]
    active = [int(e) for e in ref_sort["active_experts"][: ref_sort["active_count"]]]
    h_ref, y_ref = np.zeros((s.P, s.I)), np.zeros((s.P, s.H))

    def one(e):
        lo, hi = int(offs[e]), int(offs[e + 1])
        Wg, Wu, Wd = oracle.expert_weights(wf, e, s.H, s.I, False)
        hh = oracle.gate_up_silu_rows(x[tok[lo:hi]], Wg, Wu)
        return lo, hi, hh, oracle.down_rows(hh, Wd)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for lo, hi, hh, yy in ex.map(one, active):
            h_ref[lo:hi], y_ref[lo:hi] = hh, yy
    out_ref = oracle.blend(y_ref, case.w, ref_sort["pair_pos"])
    rows = np.diff(offs)
    say("cfg4: active experts", len(active), "rows per expert max", int(rows.max()),
        "experts with one row", int((rows == 1).sum()))
    eh = parity.assert_parity(_h2f(case.layer.h), h_ref, "cfg4 h")
    ey = parity.assert_parity(_h2f(case.layer.y), y_ref, "cfg4 y")
    eo = parity.assert_parity(_h2f(case.layer.out), out_ref, "cfg4 out")
    say("cfg4 h", eh, "y", ey, "out", eo)


# ---------------------------------------------------------------- per-kernel, oracle inputs
@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_down_and_blend_from_oracle_inputs(cfg):
    """down fed with the oracle's h (as f32) and blend fed with the oracle's y."""
    say("down/blend with oracle inputs, cfg", cfg)
    case = Case(cfg)
    s = case.shape
    case.run()  # produces the sort outputs the kernels index with
    ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), s.E, s.H, s.I)
    n = int(ref["expert_offsets"][-1])
    h32 = ref["h"].astype(np.float32)
    L = case.layer
    L.h.copy_(torch.from_numpy(h32).cuda())
    moe.moe_nvfp4_down(L.h, s.T, s.k, s.E, s.H, s.I, L.down, L.expert_offsets, L.active_experts,
                       L.active_count, L.y)
    torch.cuda.synchronize()
    wf = case.weight_fn()
    y_ref = np.zeros((s.P, s.H))
    offs = ref["expert_offsets"]
    for e in ref["active_experts"][: ref["active_count"]]:
        lo, hi = offs[e], offs[e + 1]
        y_ref[lo:hi] = oracle.down_rows(h32[lo:hi].astype(np.float64), oracle.expert_weights(wf, int(e), s.H, s.I, False)[2])
    parity.assert_parity(_h2f(L.y)[:n], y_ref[:n], f"cfg{cfg} down")
    y32 = ref["y"].astype(np.float32)
    L.y.copy_(torch.from_numpy(y32).cuda())
    moe.moe_nvfp4_blend(L.y, case.w_d, L.pair_pos, L.out)
    torch.cuda.synchronize()
    o_ref = oracle.blend(y32.astype(np.float64), case.w, ref["pair_pos"])
    parity.assert_parity(_h2f(L.out), o_ref, f"cfg{cfg} blend")


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("T,H,I,E,k", [(5, 576, 448, 3, 2), (40, 320, 384, 1, 1), (13, 640, 256, 6, 3),
                                        (1, 256, 256, 2, 2), (130, 256, 320, 4, 2), (37, 1216, 704, 5, 3)])
def test_ragged_shapes(T, H, I, E, k, kmajor):
    say("ragged", T, H, I, E, k, "kmajor" if kmajor else "row")
    shape = synth.MoeShape(f"ragged_{T}_{H}_{I}_{E}_{k}", T, H, I, E, k, "uniform", kmajor)
    _full_check(Case(11, shape), f"ragged {T},{H},{I},{E},{k},{kmajor}")


@pytest.mark.parametrize("kmajor", [False, True])
def test_null_expert_contributes_zero(kmajor):
    say("null expert", kmajor)
    shape = synth.MoeShape("null", 6, 256, 320, 4, 2, "uniform", kmajor)
    ids, _ = synth.gen_routing(12, shape)
    e_null = int(ids[0, 0])
    case = Case(12, shape, nulls=(e_null,))
    ref = _full_check(case, f"null {kmajor}")
    lo, hi = ref["expert_offsets"][e_null], ref["expert_offsets"][e_null + 1]
    assert not _h2f(case.layer.h)[lo:hi].any() and not _h2f(case.layer.y)[lo:hi].any()


def test_null_experts_in_the_32_token_launches():
    """The 32-token workload (persistent gate+up with the sort inside, one
    pass per block over strided unit shares; down as one block per strided
    unit group) with two NULL experts: the busiest one, whose rows take
    several passes, and one with a single routed row.  Their h and y rows
    are zero (written for every strided unit), and the whole layer matches
    the oracle, in which a NULL expert contributes nothing."""
    say("null experts at 32 tokens")
    shape = synth.config(3)
    ids, _ = synth.gen_routing(3, shape)
    cnt = np.bincount(ids.reshape(-1), minlength=shape.E)
    e_busy = int(np.argmax(cnt))
    e_one = int(np.nonzero(cnt == 1)[0][0])
    say("busy expert", e_busy, "rows", int(cnt[e_busy]), "one-row expert", e_one)
    case = Case(3, nulls=(e_busy, e_one))
    ref = _full_check(case, "null experts t32")
    h, y = _h2f(case.layer.h), _h2f(case.layer.y)
    for e in (e_busy, e_one):
        lo, hi = ref["expert_offsets"][e], ref["expert_offsets"][e + 1]
        assert hi > lo and not h[lo:hi].any() and not y[lo:hi].any(), e


def test_invalid_ids_flagged_and_skipped():
    say("invalid ids")
    shape = synth.MoeShape("bad", 8, 256, 512, 4, 2, "uniform", False)
    ids, w = synth.gen_routing(13, shape)
    ids[1, 1] = 9
    ids[6, 0] = -1
    case = Case(13, shape, ids=ids, weights=w)
    ref = _full_check(case, "invalid ids")
    assert ref["err"] == 1 and case.sort_outputs()["err"] == moe.FLAG_BAD_EXPERT_ID


@pytest.mark.parametrize("cfg", [2, 5])
def test_deterministic_and_power_of_two_scaling(cfg):
    say("determinism / scale_2 x4, cfg", cfg)
    case = Case(cfg)
    a = case.run().clone()
    ya = case.layer.y.clone()
    b = case.run().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    case.set_scale2(2, float(synth.SCALE2_F32) * 4)
    case.run()
    n = int(case.layer.expert_offsets[-1].item())
    assert torch.equal(case.layer.y[:n], ya[:n] * 4)


def test_many_rows_one_expert_passes():
    """One expert takes every token: one pass, several passes on their own
    block rows, and (T=1100) more further passes than block rows for them."""
    say("many rows one expert")
    for T in (1, 2, 3, 7, 8, 9, 23, 40, 1100):
        shape = synth.MoeShape(f"one_{T}", T, 512, 256, 2, 1, "uniform", False)
        ids = np.zeros((T, 1), dtype=np.int32)
        _full_check(Case(14, shape, ids=ids, weights=np.ones((T, 1), np.float32)), f"one expert T={T}")


def test_kmajor_matches_rowmajor_on_same_weights():
    say("K-major vs row-major")
    shape = synth.MoeShape("both", 48, 512, 384, 8, 2, "uniform", False)
    a = Case(15, shape, kmajor=False)
    b = Case(15, shape, kmajor=True)
    oa, ob = _h2f(a.run()), _h2f(b.run())
    ref = oracle.moe_layer(a.x_bits, a.ids, a.w, a.weight_fn(), shape.E, shape.H, shape.I)
    parity.assert_parity(oa, ref["out"], "row-major")
    parity.assert_parity(ob, ref["out"], "K-major")


@pytest.mark.parametrize("kmajor,T,E", [(False, 6, 4), (True, 6, 4), (False, 40, 2)])
def test_activation_range(kmajor, T, E):
    """Token rows scaled by 2^40, 2^-40 and 2^60 (beyond fp16's range either
    way): the decode path stages each row with its own power-of-two factor and
    the many-token path computes in bf16, so every row of h, y and out follows
    the oracle at its own magnitude (scale-invariant rules, row by row).
    40 tokens over 2 experts puts the decode passes on the token-dense path."""
    say("activation range", "kmajor" if kmajor else "row-major", T, E)
    shape = synth.MoeShape("range", T, 512, 384, E, 2, "uniform", kmajor)
    case = Case(16, shape)
    bits = case.x_bits.astype(np.uint32)
    shift = {1: 40, 2: -40, 4: 60}  # h of the 2^60 row is near 2^108, inside fp32
    for t, sh in shift.items():
        nz = (bits[t] & 0x7f80) != 0  # leave zeros and subnormals alone
        e = ((bits[t] >> 7) & 0xff).astype(np.int64) + sh
        assert ((e[nz] > 0) & (e[nz] < 255)).all()
        bits[t] = np.where(nz, (bits[t] & 0x807f) | (e.astype(np.uint32) << 7), bits[t])
    case.x_bits = bits.astype(np.uint16)
    case.x = torch.from_numpy(case.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    case.run()
    ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), shape.E, shape.H, shape.I)
    _check_sort(case, ref)
    h, y, out = _h2f(case.layer.h), _h2f(case.layer.y), _h2f(case.layer.out)
    for p in range(shape.P):
        parity.assert_parity_relative(h[p], ref["h"][p], f"h row {p}")
        parity.assert_parity_relative(y[p], ref["y"][p], f"y row {p}")
    for t in range(shape.T):
        parity.assert_parity_relative(out[t], ref["out"][t], f"out row {t}")


@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("routing", ["uniform", "zipf"])
def test_many_experts_and_passes(routing, kmajor):
    """64 experts, 800 routed rows: several units per block, and with
    Zipf-skewed routing experts whose rows take several passes on extra
    block rows (row-major) or several row tiles (K-major)."""
    say("many experts and passes", routing, "kmajor" if kmajor else "row-major")
    shape = synth.MoeShape(f"wide_{routing}", 200, 768, 1024, 64, 4, routing, kmajor)
    _full_check(Case(17, shape), f"wide {routing} {kmajor}")


def test_layer_many_sparse_experts():
    """256 routed pairs over about 225 of 1024 experts, H = 2048: the
    persistent gate+up (sort inside) walks shares that cross expert
    boundaries, and the down projection's grid holds about 225 live expert
    rows; the whole layer against the oracle."""
    say("layer over many sparse experts")
    shape = synth.MoeShape("sparse_e1024", 32, 2048, 512, 1024, 8, "uniform", False)
    _full_check(Case(28, shape), "many sparse experts")


def test_kmajor_few_experts_many_rows():
    """4 experts, 700 tokens, top-2: about 350 rows per expert, so every
    expert is split into several balanced row tiles in both projections."""
    say("K-major, few experts with many rows")
    shape = synth.MoeShape("tall", 700, 512, 640, 4, 2, "uniform", True)
    _full_check(Case(18, shape), "tall kmajor")


# ---------------------------------------------------------------- router (next step F1)
def _route_gpu(logits, k):
    T, E = logits.shape
    d = torch.from_numpy(logits).cuda()
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    moe.moe_nvfp4_route(d, k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check_route(logits, k, tag):
    ids, w = _route_gpu(logits, k)
    rids, rw = oracle.route_topk(logits, k)
    assert np.array_equal(ids, rids), tag          # integer decisions from the same f32 comparisons
    np.testing.assert_allclose(w.astype(np.float64), rw, rtol=1e-5, atol=1e-7, equal_nan=True, err_msg=tag)
    say(tag, "max |dw|", float(np.nanmax(np.abs(w - rw))) if w.size else 0.0)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_router_configs(cfg):
    say("router cfg", cfg)
    s = synth.config(cfg)
    _check_route(synth.gen_logits(cfg), s.k, f"router cfg{cfg}")


@pytest.mark.parametrize("T,E,k,mode", [(1, 1, 1, "rand"), (9, 7, 7, "rand"), (5, 1024, 64, "rand"),
                                         (33, 37, 5, "ties"), (6, 16, 4, "nan"), (200, 256, 8, "coarse")])
def test_router_edge_cases(T, E, k, mode):
    say("router edge", T, E, k, mode)
    rng = np.random.default_rng(T * 13 + E * 7 + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if mode == "ties":
        lg[:, ::3] = lg[:, :1]                     # many exact ties per row
        lg[0, :] = 0.0
        lg[0, 1::2] = -0.0
    elif mode == "nan":
        lg[0, 2] = np.nan
        lg[1, :] = np.nan                           # all NaN: ids 0..k-1, weights NaN
        lg[2, :3] = np.nan
    elif mode == "coarse":
        lg = np.round(lg * 4).astype(np.float32)    # few distinct values: ties everywhere
    _check_route(lg, k, f"router {T},{E},{k},{mode}")


def test_router_feeds_the_layer():
    """Device router -> sort -> gate+up -> down -> blend equals the oracle
    layer on the oracle's routing of the same logits (tiny workload)."""
    say("router feeds the layer")
    case = Case(1)
    s = case.shape
    logits = synth.gen_logits(1)
    ids_d = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    moe.moe_nvfp4_route(torch.from_numpy(logits).cuda(), s.k, ids_d, w_d)
    out = case.layer.forward(case.x, ids_d, w_d)
    torch.cuda.synchronize()
    rids, rw = oracle.route_topk(logits, s.k)
    ref = oracle.moe_layer(case.x_bits, rids, rw.astype(np.float32), case.weight_fn(), s.E, s.H, s.I)
    parity.assert_parity(_h2f(out), ref["out"], "routed layer")


# ---------------------------------------------------------------- shared expert (next step F2)
@pytest.mark.parametrize("kmajor", [False, True])
def test_shared_expert_in_the_same_launches(kmajor):
    """Every token also routes to a shared expert (table slot E, weight 1):
    the four launches compute it with the routed experts; the output matches
    the oracle layer on the same extended routing."""
    say("shared expert", "kmajor" if kmajor else "row-major")
    base = synth.config(3)
    ids, w = synth.gen_routing(3, base)
    ids_d, w_d = moe.with_shared_expert(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), base.E)
    aug_ids, aug_w = ids_d.cpu().numpy(), w_d.cpu().numpy()
    assert np.array_equal(aug_ids[:, :-1], ids) and np.all(aug_ids[:, -1] == base.E)
    assert np.array_equal(aug_w[:, :-1], w) and np.all(aug_w[:, -1] == 1.0)
    shape = synth.MoeShape("shared3", base.T, base.H, base.I, base.E + 1, base.k + 1, "zipf", kmajor)
    _full_check(Case(3, shape, ids=aug_ids, weights=aug_w), f"shared {kmajor}")


# ---------------------------------------------------------------- MXFP4 experts (next step F3)
def test_layer_prefill_kmajor_mxfp4_full():
    """The many-token workload (2048 tokens, H=4096, I=1536, E=64, top-4) with
    MXFP4 experts: K-major twins with one E8M0 scale per 32 k."""
    say("layer cfg 5 shape, MXFP4 experts")
    _full_check(Case(5, fmt="mxfp4"), "cfg5 mxfp4")


@pytest.mark.parametrize("T,H,I,E,k", [(5, 576, 448, 3, 2), (130, 256, 320, 4, 2), (37, 1216, 704, 5, 3),
                                        (300, 128, 64, 2, 2)])
def test_ragged_shapes_mxfp4(T, H, I, E, k):
    say("ragged mxfp4", T, H, I, E, k)
    shape = synth.MoeShape(f"ragged_mx_{T}_{H}_{I}_{E}_{k}", T, H, I, E, k, "uniform", True)
    _full_check(Case(21, shape, fmt="mxfp4"), f"ragged mxfp4 {T},{H},{I},{E},{k}")


def test_mxfp4_null_expert_and_scale_range():
    """E8M0 codes over 2^-60 .. 2^20 (gate, up) and 2^-30 .. 2^10 (down), one
    NULL expert.  Here the output columns, not the rows, differ by orders of
    magnitude (each weight row has its own scale codes), so the strict rule
    is applied with each column rescaled to unit RMS."""
    shape = synth.MoeShape("mx_range", 96, 256, 192, 3, 2, "uniform", True)

    def gen(cfg_id, e, proj, s):
        pk, _ = synth.gen_expert_mx(cfg_id, e, proj, s)
        n, kk = synth.proj_dims(s, proj)
        lo, hi = (67, 147) if proj < 2 else (97, 137)
        sc = np.random.default_rng([cfg_id, e, proj, 99]).integers(lo, hi + 1, (n, kk // 32), dtype=np.uint8)
        return pk, sc

    case = Case(22, shape, nulls=(1,), fmt="mxfp4", gen=gen)
    case.run()
    ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), 3, 256, 192, fmt="mxfp4")
    _check_sort(case, ref)
    n = int(ref["expert_offsets"][-1])
    for name, got, want in (("h", _h2f(case.layer.h)[:n], ref["h"][:n]), ("y", _h2f(case.layer.y)[:n], ref["y"][:n])):
        for e in ref["active_experts"][: ref["active_count"]]:
            lo, hi = int(ref["expert_offsets"][e]), int(ref["expert_offsets"][e + 1])
            g, w = got[lo:hi], want[lo:hi]
            if e == 1:
                assert np.array_equal(g, np.zeros_like(g)), "NULL expert rows"
                continue
            col = np.sqrt(np.mean(w * w, axis=0))
            rel = np.abs(g - w) / (col + np.abs(w) + 1e-300)
            assert rel.max() <= 1e-2, (name, int(e), float(rel.max()))
    say("mx range ok", float(np.abs(ref["h"][:n]).max()), float(np.abs(ref["h"][:n][ref["h"][:n] != 0]).min()))


# ---------------------------------------------------------------- concatenated gate||up twin (next step F4)
@pytest.mark.parametrize("rows,cols,parts", [(1536, 2048, 2), (70, 130, 2), (64, 96, 3)])
def test_transpose_concat_bit_exact(rows, cols, parts):
    say("transpose concat", rows, cols, parts)
    rng = np.random.default_rng(rows + cols)
    srcs = [rng.integers(0, 256, (rows + 3 * p, cols), dtype=np.uint8) for p in range(parts)]
    n_total = sum(a.shape[0] for a in srcs)
    stride = -(-n_total // 16) * 16
    dst = torch.full((cols, stride), 0x5A, dtype=torch.uint8, device="cuda")
    off = 0
    for a in srcs:
        moe.transpose_u8_pitched(torch.from_numpy(a).cuda(), dst, a.shape[0], cols, stride, off)
        off += a.shape[0]
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    want = oracle.transpose_concat(srcs, stride)
    assert np.array_equal(got[:, :n_total], want[:, :n_total])
    assert (got[:, n_total:] == 0x5A).all()  # bytes outside the windows untouched
    # the Python builder zeroes the pad columns
    pt, st, stride2 = moe.transpose_concat_for_gemm(
        [(torch.from_numpy(a).cuda(), torch.from_numpy(a[:, : cols // 8].copy()).cuda(), a.shape[0]) for a in srcs],
        2 * cols, 16, align=16)
    assert stride2 == stride and np.array_equal(pt.cpu().numpy(), want)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_layer_prefill_concat_gate_up_full(fmt):
    """The many-token workload with each expert's gate and up in one
    concatenated K-major twin; h must equal the two-twin launch bit for bit
    (same arithmetic, other addressing) and the oracle to the parity rules."""
    say("layer cfg 5, concatenated gate||up", fmt)
    case = Case(5, fmt=fmt, concat=True)
    _full_check(case, f"cfg5 concat {fmt}")
    h_concat = case.layer.h.clone()
    L = case.layer
    moe.moe_nvfp4_gate_up_silu(case.x, case.shape.k, case.shape.E, case.shape.H, case.shape.I, L.gate, L.up,
                               L.expert_offsets, L.sorted_token_ids, L.active_experts, L.active_count, L.h)
    torch.cuda.synchronize()
    n = int(L.expert_offsets[-1].item())
    assert torch.equal(h_concat[:n], L.h[:n])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("T,H,I,E,k", [(37, 1216, 704, 5, 3), (130, 256, 320, 4, 2)])
def test_ragged_concat_gate_up(T, H, I, E, k, fmt):
    say("ragged concat", T, H, I, E, k, fmt)
    shape = synth.MoeShape(f"ragged_cc_{T}_{H}_{I}_{E}_{k}", T, H, I, E, k, "uniform", True)
    _full_check(Case(23, shape, fmt=fmt, concat=True, nulls=(1,)), f"ragged concat {T},{H},{I},{E},{k},{fmt}")


# ---------------------------------------------------------------- sort fused into the gate+up launch
@pytest.mark.parametrize("T,k,E,H,I,mode", [(1, 8, 128, 2048, 768, "rand"), (4, 2, 4, 256, 512, "rand"),
                                             (2, 8, 1024, 256, 256, "invalid"), (3, 5, 7, 512, 256, "dup"),
                                             (16, 3, 4, 512, 256, "dup"), (2, 32, 64, 256, 384, "rand"),
                                             (32, 6, 128, 2688, 1856, "rand"), (40, 6, 128, 2688, 1856, "invalid"),
                                             (42, 6, 100, 512, 2048, "dup"), (43, 6, 128, 512, 2048, "rand"),
                                             # persistent, 256 pairs over about 225 experts: blocks take
                                             # shares that run into the next slot (two passes per block)
                                             (32, 8, 1024, 256, 512, "rand")])
def test_sort_fused_into_gate_up_matches_two_calls(T, k, E, H, I, mode):
    """moe_nvfp4_sort_gate_up_silu (one launch while P <= 64 and each expert
    fits one pass, or when the gate+up launch is persistent and P <= 256:
    every block then sorts in LDS and block 0 writes the sort outputs; two
    launches otherwise, e.g. 258 pairs) against the two separate calls: sort
    outputs and err_flag equal, h bit for bit; sort outputs against the
    oracle's brute force."""
    L1 = moe.moe_nvfp4_sort_gate_up_launches(T, k, E, H, I, moe.ROW_MAJOR)
    say("launches", L1)
    if T * k in (192, 240, 252, 256):
        assert L1 == 1
    say("fused sort", T, k, E, H, I, mode)
    shape = synth.MoeShape(f"fs_{T}_{k}_{E}", T, H, I, E, k, "uniform", False)
    rng = np.random.default_rng(T * 1000 + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if mode == "dup":
        ids[:, 1] = ids[:, 0]
    if mode == "invalid":
        ids[0, 0] = -1
        ids[-1, -1] = E + 3
    case = Case(24, shape, ids=ids)
    L = case.layer
    outs = []
    for fused in (True, False):
        L.err_flag.zero_()
        L.h.fill_(7.0)
        L.expert_offsets.fill_(-5)
        if fused:
            moe.moe_nvfp4_sort_gate_up_silu(case.ids_d, case.x, E, H, I, L.gate, L.up, L.expert_offsets,
                                            L.sorted_token_ids, L.pair_pos, L.active_experts, L.active_count,
                                            L.err_flag, L.h)
        else:
            moe.moe_nvfp4_sort(case.ids_d, E, L.expert_offsets, L.sorted_token_ids, L.pair_pos, L.active_experts,
                               L.active_count, L.err_flag)
            moe.moe_nvfp4_gate_up_silu(case.x, k, E, H, I, L.gate, L.up, L.expert_offsets, L.sorted_token_ids,
                                       L.active_experts, L.active_count, L.h)
        torch.cuda.synchronize()
        outs.append((case.sort_outputs(), L.h.clone()))
    (s_f, h_f), (s_u, h_u) = outs
    for key in ("expert_offsets", "sorted_token_ids", "pair_pos", "active_experts"):
        assert np.array_equal(s_f[key], s_u[key]), key
    assert s_f["active_count"] == s_u["active_count"] and s_f["err"] == s_u["err"]
    _check_sort(case, oracle.sort_routes(case.ids, E))
    n = int(s_u["expert_offsets"][-1])
    assert torch.equal(h_f[:n], h_u[:n])


# ---------------------------------------------------------------- down + blend in one launch
@pytest.mark.parametrize("T,H,I,E,k,mode", [
    (1, 2048, 768, 128, 8, "cfg"),      # the 1-token decode workload itself
    (1, 256, 512, 4, 2, "rand"),
    (1, 512, 256, 16, 1, "rand"),       # one pair: three waves stream nothing
    (1, 320, 448, 9, 5, "dup"),         # one expert twice, ragged widths
    (1, 256, 256, 80, 64, "rand"),      # k = 64, the most pairs a block takes
    (1, 640, 384, 12, 6, "null"),       # a NULL expert among the pairs
    (2, 256, 512, 8, 3, "invalid"),     # ids outside [0, E) add nothing
    (5, 2048, 256, 64, 4, "rand"),      # two column groups per block
    (32, 2688, 1856, 128, 6, "zipf"),   # many tokens: four column groups, experts shared
    (1, 256, 36736, 4, 1, "rand"),      # the widest h row the staging admits (k = 1)
    (3, 512, 384, 6, 4, "null+invalid"),  # a NULL expert and an id outside [0, E) in one launch
])
def test_down_blend_matches_down_then_blend(T, H, I, E, k, mode):
    """moe_nvfp4_down_blend against moe_nvfp4_down + moe_nvfp4_blend on the
    same h: bit for bit while every expert holds at most 4 routed pairs (the
    grouped kernel then computes each y value in the same order), and against
    the oracle's layer output in every case."""
    say("down+blend", T, H, I, E, k, mode)
    if mode == "cfg":
        case = Case(2)
    else:
        routing = "zipf" if mode == "zipf" else "uniform"
        shape = synth.MoeShape(f"db_{T}_{k}_{E}", T, H, I, E, k, routing, False)
        ids, w = synth.gen_routing(25, shape)
        nulls = ()
        if mode == "dup":
            ids[0, 1] = ids[0, 0]
        elif mode == "invalid":
            ids[0, 0] = -1
            ids[1, 2] = E + 3
        elif mode == "null":
            nulls = (int(ids[0, 1]),)
        elif mode == "null+invalid":
            ids[2, 3] = -1
            nulls = (int(ids[1, 0]),)
        case = Case(25, shape, ids=ids, weights=w, nulls=nulls)
    s, L = case.shape, case.layer
    case.run(fuse_blend=False)
    fused = torch.full_like(L.out, 7.0)
    moe.moe_nvfp4_down_blend(L.h, case.ids_d, case.w_d, L.pair_pos, s.E, s.H, s.I, L.down, fused)
    torch.cuda.synchronize()
    rows = np.diff(L.expert_offsets.cpu().numpy())
    if rows.max() <= 4:
        assert torch.equal(fused.view(torch.int16), L.out.view(torch.int16))
    ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), s.E, s.H, s.I)
    e = parity.assert_parity(_h2f(fused), ref["out"], f"down+blend {T},{H},{I},{E},{k},{mode}")
    say("down+blend", mode, "max rows per expert", int(rows.max()), e)


def test_layer_one_token_fuses_down_blend_or_falls_back():
    """MoeLayer.forward with one token: down and blend in one launch (y left
    untouched); a shape whose 64 activation rows do not fit the staging
    budget (k = 64, I = 2048) is refused with ELIMIT and the layer issues the
    two calls instead (y written).  Both match the oracle."""
    say("layer one token: fused down+blend / fallback")
    for (H, I, E, k), fused in (((2048, 768, 128, 8), True), ((256, 2048, 64, 64), False)):
        shape = synth.MoeShape(f"one_tok_{k}", 1, H, I, E, k, "uniform", False)
        case = Case(26, shape)
        L = case.layer
        L.y.fill_(3.0)
        out = L.forward(case.x, case.ids_d, case.w_d)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(case.x_bits, case.ids, case.w, case.weight_fn(), E, H, I)
        parity.assert_parity(_h2f(out), ref["out"], f"one token k={k}")
        y_touched = bool((L.y != 3.0).any().item())
        assert y_touched != fused, (k, fused)
        if not fused:
            with pytest.raises(moe.MoeNvfp4Error, match="ELIMIT"):
                moe.moe_nvfp4_down_blend(L.h, case.ids_d, case.w_d, L.pair_pos, E, H, I, L.down, L.out)


# ---------------------------------------------------------------- graph capture
def test_layer_graph_replays_match_eager():
    """The decode layer (sort fused into gate+up) captured in a HIP graph: every
    replay, with eager work and synchronisations between replays, gives the
    eager result bit for bit."""
    say("graph replay, 1-token decode layer")
    case = Case(2)
    L = case.layer
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        L.forward(case.x, case.ids_d, case.w_d, stream=stream)
    torch.cuda.synchronize()
    eager_out, eager_h = L.out.clone(), L.h.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        L.forward(case.x, case.ids_d, case.w_d, stream=stream)
    torch.cuda.synchronize()
    for rep in range(3):
        L.out.fill_(9.0)
        L.h.fill_(9.0)
        scratch = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.out, eager_out), rep
        assert torch.equal(L.h[: case.shape.P], eager_h[: case.shape.P]), rep
        del scratch


# ---------------------------------------------------------------- widest admitted rows
@pytest.mark.parametrize("kmajor,H,I", [(False, 36736, 256), (True, 65536, 64)])
def test_widest_hidden_width(kmajor, H, I):
    """The widest activation rows each path admits: the decode kernel stages
    one row of x (fp16) in its LDS budget, so K = H <= 36736 (and I >= 256
    on that path); the K-major GEMM takes the full MOE_NVFP4_MAX_WIDTH =
    65536, here with the narrowest down projection it admits (I = 64):
    393K outputs, each a sum of 64 products of h rounded to fp16."""
    say("widest H", H, "I", I, "kmajor" if kmajor else "row")
    shape = synth.MoeShape(f"wide_h_{H}", 6, H, I, 2, 1, "uniform", kmajor)
    _full_check(Case(25, shape), f"widest H {H}")


# ---------------------------------------------------------------- K-major down: row exponents of h
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_kmajor_down_row_exponents(fmt):
    """The K-major down projection stages h as fp16 with one power of two per
    row, set at the row's first nonzero 32-k step.  Crafted h rows: a first
    step 2^-12 of the rest and a tail grown by 2^20 (a later step exceeds
    the first step's range, so the block runs again with exact exponents),
    zeros up to k = 200, all zeros, and rows at 2^60 and 2^-60.  Each y row
    is compared with the oracle at its own magnitude; zero rows give zero."""
    say("K-major down row exponents", fmt)
    shape = synth.MoeShape(f"down_rows_{fmt}", 40, 512, 384, 2, 2, "uniform", True)
    case = Case(27, shape, fmt=fmt)
    case.run()  # the sort outputs the down launch indexes with
    L, P, I = case.layer, shape.P, shape.I
    h = np.random.default_rng(27).standard_normal((P, I))
    h[0::7, :32] *= 2.0 ** -12
    h[1::7, :200] = 0.0
    h[2::7, :] = 0.0
    h[3::7] *= 2.0 ** 60
    h[4::7] *= 2.0 ** -60
    h[5::7, 300:] *= 2.0 ** 20
    h32 = h.astype(np.float32)
    L.h.copy_(torch.from_numpy(h32).cuda())
    L.y.fill_(7.0)
    moe.moe_nvfp4_down(L.h, shape.T, shape.k, shape.E, shape.H, shape.I, L.down, L.expert_offsets,
                       L.active_experts, L.active_count, L.y)
    torch.cuda.synchronize()
    y = _h2f(L.y)
    offs = L.expert_offsets.cpu().numpy()
    wf = case.weight_fn()
    for e in range(shape.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        Wd = oracle.expert_weights(wf, e, shape.H, shape.I, False, fmt)[2]
        y_ref = oracle.down_rows(h32[lo:hi].astype(np.float64), Wd)
        for p in range(lo, hi):
            if not h32[p].any():
                assert not y[p].any(), p
                continue
            parity.assert_parity_relative(y[p], y_ref[p - lo], f"{fmt} y row {p}")


# ---------------------------------------------------------------- row-major down: row scales of h
def test_rowmajor_down_row_scales():
    """The row-major down projection stages a pass's h rows as fp16 with one
    power of two per row.  With rows read in several batches it reads them
    once, the scale set by the first batch's largest magnitude (with a
    factor 4 of headroom); a row whose later elements pass the fp16 limit at
    that scale, or whose first batch is all zero, makes the block stage again
    from exact maxima.  I = 1856 over two experts (passes of 16 and 8 rows,
    so every pass takes several batches, the first covering at most the
    first 1024 elements).  Crafted rows: the first 32 elements 2^-12 of the
    rest, zeros up to k = 200, all zeros, scaled by 2^60 and 2^-60, a tail
    from k = 1100 grown by 2^20 (overflow at the estimated scale), zeros up
    to k = 1100 (an all-zero first batch), and plain rows.  Each y row is
    compared with the oracle at its own magnitude; zero rows give zero."""
    say("row-major down row scales")
    shape = synth.MoeShape("down_rows_rm", 40, 512, 1856, 2, 2, "uniform", False)
    case = Case(28, shape)
    case.run()  # the sort outputs the down launch indexes with
    L, P, I = case.layer, shape.P, shape.I
    h = np.random.default_rng(28).standard_normal((P, I))
    h[0::8, :32] *= 2.0 ** -12
    h[1::8, :200] = 0.0
    h[2::8, :] = 0.0
    h[3::8] *= 2.0 ** 60
    h[4::8] *= 2.0 ** -60
    h[5::8, 1100:] *= 2.0 ** 20
    h[6::8, :1100] = 0.0
    h32 = h.astype(np.float32)
    L.h.copy_(torch.from_numpy(h32).cuda())
    L.y.fill_(7.0)
    moe.moe_nvfp4_down(L.h, shape.T, shape.k, shape.E, shape.H, shape.I, L.down, L.expert_offsets,
                       L.active_experts, L.active_count, L.y)
    torch.cuda.synchronize()
    y = _h2f(L.y)
    offs = L.expert_offsets.cpu().numpy()
    say("rows per expert", np.diff(offs).tolist())
    wf = case.weight_fn()
    for e in range(shape.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        Wd = oracle.expert_weights(wf, e, shape.H, shape.I, False)[2]
        y_ref = oracle.down_rows(h32[lo:hi].astype(np.float64), Wd)
        for p in range(lo, hi):
            if not h32[p].any():
                assert not y[p].any(), p
                continue
            parity.assert_parity_relative(y[p], y_ref[p - lo], f"row-major y row {p}")
