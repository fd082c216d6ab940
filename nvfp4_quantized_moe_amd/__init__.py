"""Grouped NVFP4 MoE expert projection for MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/moe_nvfp4.h``: the entry
points keep their C names and take torch tensors only for device
memory and streams; every step of the path runs in the HIP kernels of
``libmoe_nvfp4.so``.  There is no CPU fallback: importing works without the
library, but the first call raises if it is missing.

Higher-level helpers:
  * ``ExpertTables``       device pointer tables of one projection across experts
                           (nvfp4_moe_grouped.rs, ``Nvfp4ExpertTables``);
  * ``transpose_for_gemm`` load-time K-major twin of one NVFP4 weight
                           (transpose.rs, ``transpose_for_gemm``);
  * ``MoeLayer``           the four calls of one layer forward on one stream.
"""
from __future__ import annotations

import ctypes
import pathlib
import re
from typing import Optional, Sequence

import torch

__all__ = [
    "ExpertTables",
    "MoeLayer",
    "MoeNvfp4Error",
    "ROW_MAJOR",
    "K_MAJOR",
    "K_MAJOR_MXFP4",
    "FLAG_BAD_EXPERT_ID",
    "lib",
    "header_functions",
    "moe_nvfp4_sort",
    "moe_nvfp4_gate_up_silu",
    "moe_nvfp4_down",
    "moe_nvfp4_blend",
    "moe_nvfp4_down_blend",
    "transpose_u8",
    "transpose_u8_pitched",
    "transpose_for_gemm",
    "transpose_concat_for_gemm",
    "moe_nvfp4_gate_up_silu_concat",
    "moe_nvfp4_sort_gate_up_silu",
    "moe_nvfp4_sort_gate_up_launches",
    "moe_nvfp4_route",
    "moe_nvfp4_stream_read",
    "with_shared_expert",
]

ROW_MAJOR = 0
K_MAJOR = 1
K_MAJOR_MXFP4 = 2  # K-major MXFP4: E8M0 scales, one per 32 k
FLAG_BAD_EXPERT_ID = 1

_PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = _PKG / "libmoe_nvfp4.so"
HEADER = _PKG.parent / "include" / "moe_nvfp4.h"

_ERRNAMES = {-1: "ENULL", -2: "ESHAPE", -3: "ELAYOUT", -4: "ELIMIT"}
_ELIMIT = -4


class MoeNvfp4Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        name = _ERRNAMES.get(code, f"hipError {code}")
        super().__init__(f"{fn} failed: {name} ({code})")
        self.code = code


class _Experts(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("scale2", ctypes.c_void_p),
        ("layout", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m nvfp4_quantized_moe_amd.build`"
            )
        L = ctypes.CDLL(str(LIB_PATH))
        L.moe_nvfp4_sort.argtypes = [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        L.moe_nvfp4_gate_up_silu.argtypes = [_P, _I, _I, _I, _I, _I, _Experts, _Experts, _P, _P, _P, _P, _P, _P]
        L.moe_nvfp4_down.argtypes = [_P, _I, _I, _I, _I, _I, _Experts, _P, _P, _P, _P, _P]
        L.moe_nvfp4_blend.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P]
        L.transpose_u8.argtypes = [_P, _P, _I, _I, _P]
        L.moe_nvfp4_route.argtypes = [_P, _I, _I, _I, _P, _P, _P]
        L.transpose_u8_pitched.argtypes = [_P, _P, _I, _I, ctypes.c_int64, _P]
        L.moe_nvfp4_gate_up_silu_concat.argtypes = [_P, _I, _I, _I, _I, _I, _Experts, _I, _P, _P, _P, _P, _P, _P]
        L.moe_nvfp4_sort_gate_up_silu.argtypes = [_P, _P, _I, _I, _I, _I, _I, _Experts, _Experts, _P, _P, _P, _P,
                                                  _P, _P, _P, _P]
        L.moe_nvfp4_sort_gate_up_launches.argtypes = [_I, _I, _I, _I, _I, _I]
        L.moe_nvfp4_down_blend.argtypes = [_P, _I, _I, _I, _I, _I, _Experts, _P, _P, _P, _P, _P]
        L.moe_nvfp4_stream_read.argtypes = [_P, ctypes.c_int64, _P, _P]
        for fn in ("moe_nvfp4_sort", "moe_nvfp4_gate_up_silu", "moe_nvfp4_down", "moe_nvfp4_blend",
                   "transpose_u8", "moe_nvfp4_route", "moe_nvfp4_abi_version", "transpose_u8_pitched",
                   "moe_nvfp4_gate_up_silu_concat", "moe_nvfp4_sort_gate_up_silu",
                   "moe_nvfp4_sort_gate_up_launches", "moe_nvfp4_down_blend", "moe_nvfp4_stream_read"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions the C header declares."""
    text = HEADER.read_text()
    return re.findall(r"^\s*int\s+(\w+)\s*\(", text, flags=re.M)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoeNvfp4Error(fn, rc)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, numel: int = 0) -> int:
    """Device pointer of t after checking its type, size (at least ``numel``
    elements: the kernels read or write that many), placement and layout."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _x_ptr(x: torch.Tensor, numel: int) -> int:
    """x as bf16, or as int16 holding bf16 bits."""
    if x.dtype == torch.int16:
        return _dev(x, torch.int16, "x (bf16 bits)", numel)
    return _dev(x, torch.bfloat16, "x", numel)


def _out_ptr(out: torch.Tensor, numel: int) -> int:
    """The bf16 output, or int16 holding bf16 bits."""
    if out.dtype == torch.int16:
        return _dev(out, torch.int16, "out (bf16 bits)", numel)
    return _dev(out, torch.bfloat16, "out", numel)


def _table_ptr(t, name: str, device) -> int:
    """Address of an expert's weight tensor: contiguous uint8 on the table's device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.dtype != torch.uint8:
        raise TypeError(f"{name}: expected torch.uint8, got {t.dtype}")
    if t.device.type != torch.device(device).type:
        raise ValueError(f"{name}: on {t.device}, the table is built on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


class ExpertTables:
    """One projection across E experts: device arrays of the experts' packed
    and scale pointers plus their f32 scale_2 values, in one of the layouts
    ROW_MAJOR, K_MAJOR (NVFP4) or K_MAJOR_MXFP4.  ``None`` in ``weights``
    marks an absent (NULL) expert; a present one is ``(packed, scale,
    scale_2)`` with packed and scale contiguous uint8 device tensors.  The
    element counts of every expert's tensors are kept so that each call can
    check them against the (N, K) it is given (``check``) before any launch."""

    def __init__(self, weights: Sequence[Optional[tuple]], layout: int, device="cuda"):
        if layout not in (ROW_MAJOR, K_MAJOR, K_MAJOR_MXFP4):
            raise ValueError(f"ExpertTables: unknown layout {layout}")
        packed, scales, s2, pn, sn = [], [], [], [], []
        self._keep = []
        for e, w in enumerate(weights):
            if w is None:
                packed.append(0)
                scales.append(0)
                s2.append(0.0)
                continue
            pk, sc, sv = w
            if pk is None or sc is None:
                raise ValueError(f"ExpertTables: expert {e} has a packed or scale tensor but not both "
                                 "(pass None for an absent expert)")
            packed.append(_table_ptr(pk, f"expert {e} packed", device))
            scales.append(_table_ptr(sc, f"expert {e} scale", device))
            s2.append(float(sv))
            pn.append(pk.numel())
            sn.append(sc.numel())
            self._keep.append((pk, sc))
        self.packed = torch.tensor(packed, dtype=torch.int64, device=device)
        self.scale = torch.tensor(scales, dtype=torch.int64, device=device)
        self.scale2 = torch.tensor(s2, dtype=torch.float32, device=device)
        self.layout = int(layout)
        self.E = len(weights)
        # Smallest packed / scale element count over the present experts.
        self._min_packed = min(pn) if pn else None
        self._min_scale = min(sn) if sn else None

    @property
    def group(self) -> int:
        """k values per block scale: 32 for MXFP4, 16 for NVFP4."""
        return 32 if self.layout == K_MAJOR_MXFP4 else 16

    def check(self, name: str, E: int, n: int, k: int, pitch: int = 0) -> None:
        """Raise ValueError unless the table covers E experts and every
        present expert holds an [n, k] weight: n*k/2 packed bytes and
        n*k/group scale bytes (a concatenated twin with row pitch ``pitch``:
        k/2 * pitch and k/group * pitch)."""
        if self.E < E:
            raise ValueError(f"{name}: the table holds {self.E} experts, the call reads {E}")
        if self._min_packed is None:
            return
        rows = pitch if pitch else n
        need_p, need_s = (k // 2) * rows, (k // self.group) * rows
        if self._min_packed < need_p or self._min_scale < need_s:
            raise ValueError(f"{name}: an expert holds {self._min_packed} packed / {self._min_scale} scale "
                             f"bytes, a [{n}, {k}] weight needs {need_p} / {need_s}")

    def abi(self) -> _Experts:
        return _Experts(self.packed.data_ptr(), self.scale.data_ptr(), self.scale2.data_ptr(), self.layout)


# --------------------------------------------------------------------------
# The C entry points (argument marshalling only)
# --------------------------------------------------------------------------
def moe_nvfp4_sort(topk_ids, E, expert_offsets, sorted_token_ids, pair_pos, active_experts,
                   active_count, err_flag, stream=None) -> None:
    T, k = topk_ids.shape
    P = T * k
    rc = lib().moe_nvfp4_sort(
        _dev(topk_ids, torch.int32, "topk_ids"), T, k, E,
        _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
        _dev(sorted_token_ids, torch.int32, "sorted_token_ids", P),
        _dev(pair_pos, torch.int32, "pair_pos", P),
        _dev(active_experts, torch.int32, "active_experts", E),
        _dev(active_count, torch.int32, "active_count", 1),
        _dev(err_flag, torch.int32, "err_flag", 1), _stream(stream))
    _check("moe_nvfp4_sort", rc)


def moe_nvfp4_gate_up_silu(x, k, E, H, I, gate: ExpertTables, up: ExpertTables, expert_offsets,
                           sorted_token_ids, active_experts, active_count, h, stream=None) -> None:
    T = x.shape[0]
    P = T * k
    gate.check("gate", E, I, H)
    up.check("up", E, I, H)
    rc = lib().moe_nvfp4_gate_up_silu(
        _x_ptr(x, T * H), T, k, E, H, I, gate.abi(), up.abi(),
        _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
        _dev(sorted_token_ids, torch.int32, "sorted_token_ids", P),
        _dev(active_experts, torch.int32, "active_experts", E),
        _dev(active_count, torch.int32, "active_count", 1),
        _dev(h, torch.float32, "h", P * I), _stream(stream))
    _check("moe_nvfp4_gate_up_silu", rc)


def moe_nvfp4_sort_gate_up_silu(topk_ids, x, E, H, I, gate: ExpertTables, up: ExpertTables, expert_offsets,
                                sorted_token_ids, pair_pos, active_experts, active_count, err_flag, h,
                                stream=None) -> None:
    """Sort then gate+up (one launch in the few-token decode case); see the C header."""
    T, k = topk_ids.shape
    P = T * k
    gate.check("gate", E, I, H)
    up.check("up", E, I, H)
    rc = lib().moe_nvfp4_sort_gate_up_silu(
        _dev(topk_ids, torch.int32, "topk_ids"), _x_ptr(x, T * H),
        T, k, E, H, I, gate.abi(), up.abi(),
        _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
        _dev(sorted_token_ids, torch.int32, "sorted_token_ids", P),
        _dev(pair_pos, torch.int32, "pair_pos", P),
        _dev(active_experts, torch.int32, "active_experts", E),
        _dev(active_count, torch.int32, "active_count", 1),
        _dev(err_flag, torch.int32, "err_flag", 1),
        _dev(h, torch.float32, "h", P * I), _stream(stream))
    _check("moe_nvfp4_sort_gate_up_silu", rc)


def moe_nvfp4_sort_gate_up_launches(T, k, E, H, I, layout) -> int:
    """1 when moe_nvfp4_sort_gate_up_silu runs as one launch for these sizes, else 2."""
    rc = lib().moe_nvfp4_sort_gate_up_launches(T, k, E, H, I, layout)
    if rc < 0:
        raise MoeNvfp4Error("moe_nvfp4_sort_gate_up_launches", rc)
    return rc


def moe_nvfp4_gate_up_silu_concat(x, k, E, H, I, gate_up: ExpertTables, pitch, expert_offsets,
                                  sorted_token_ids, active_experts, active_count, h, stream=None) -> None:
    """Gate+up over a concatenated gate||up K-major twin (rows ``pitch``
    bytes apart, up columns from I on); see the C header."""
    T = x.shape[0]
    P = T * k
    gate_up.check("gate_up", E, 2 * I, H, pitch=int(pitch))
    rc = lib().moe_nvfp4_gate_up_silu_concat(
        _x_ptr(x, T * H), T, k, E, H, I, gate_up.abi(), int(pitch),
        _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
        _dev(sorted_token_ids, torch.int32, "sorted_token_ids", P),
        _dev(active_experts, torch.int32, "active_experts", E),
        _dev(active_count, torch.int32, "active_count", 1),
        _dev(h, torch.float32, "h", P * I), _stream(stream))
    _check("moe_nvfp4_gate_up_silu_concat", rc)


def moe_nvfp4_down(h, T, k, E, H, I, down: ExpertTables, expert_offsets, active_experts, active_count,
                   y, stream=None) -> None:
    P = T * k
    down.check("down", E, H, I)
    rc = lib().moe_nvfp4_down(
        _dev(h, torch.float32, "h", P * I), T, k, E, H, I, down.abi(),
        _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
        _dev(active_experts, torch.int32, "active_experts", E),
        _dev(active_count, torch.int32, "active_count", 1),
        _dev(y, torch.float32, "y", P * H), _stream(stream))
    _check("moe_nvfp4_down", rc)


def moe_nvfp4_blend(y, topk_weights, pair_pos, out, stream=None) -> None:
    T, k = topk_weights.shape
    H = y.shape[1]
    rc = lib().moe_nvfp4_blend(
        _dev(y, torch.float32, "y", T * k * H), _dev(topk_weights, torch.float32, "topk_weights"),
        _dev(pair_pos, torch.int32, "pair_pos", T * k), T, k, H, _out_ptr(out, T * H), _stream(stream))
    _check("moe_nvfp4_blend", rc)


def _down_blend_rc(h, topk_ids, topk_weights, pair_pos, E, H, I, down: ExpertTables, out, stream) -> int:
    T, k = topk_weights.shape
    P = T * k
    down.check("down", E, H, I)
    return lib().moe_nvfp4_down_blend(
        _dev(h, torch.float32, "h", P * I), T, k, E, H, I, down.abi(),
        _dev(topk_ids, torch.int32, "topk_ids", P), _dev(topk_weights, torch.float32, "topk_weights"),
        _dev(pair_pos, torch.int32, "pair_pos", P), _out_ptr(out, T * H), _stream(stream))


def moe_nvfp4_down_blend(h, topk_ids, topk_weights, pair_pos, E, H, I, down: ExpertTables, out,
                         stream=None) -> None:
    """Down projection and top-k blend in one launch (row-major weights; meant
    for decode with one or a few tokens)."""
    _check("moe_nvfp4_down_blend", _down_blend_rc(h, topk_ids, topk_weights, pair_pos, E, H, I, down, out, stream))


def transpose_u8(src, dst, rows, cols, stream=None) -> None:
    if src.numel() != rows * cols or dst.numel() != rows * cols:
        raise ValueError("transpose_u8: tensor sizes do not match rows * cols")
    rc = lib().transpose_u8(_dev(src, torch.uint8, "src"), _dev(dst, torch.uint8, "dst"), rows, cols,
                            _stream(stream))
    _check("transpose_u8", rc)


def transpose_u8_pitched(src, dst, rows, cols, dst_pitch, dst_offset=0, stream=None) -> None:
    """dst.flat[dst_offset + c * dst_pitch + r] = src[r, c] (the C call on
    dst's storage from byte dst_offset on)."""
    if src.numel() != rows * cols:
        raise ValueError("transpose_u8_pitched: src size does not match rows * cols")
    if dst_offset < 0 or dst_pitch < rows or dst.numel() < dst_offset + (cols - 1) * dst_pitch + rows:
        raise ValueError("transpose_u8_pitched: dst too small for the pitched window")
    rc = lib().transpose_u8_pitched(_dev(src, torch.uint8, "src"), _dev(dst, torch.uint8, "dst") + dst_offset,
                                    rows, cols, dst_pitch, _stream(stream))
    _check("transpose_u8_pitched", rc)


def moe_nvfp4_stream_read(src, sink, stream=None) -> None:
    """Read all of ``src`` (a contiguous device tensor) once and discard it:
    the streaming-read ceiling (measurement support; see the C header)."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("moe_nvfp4_stream_read: src must be a contiguous device tensor")
    rc = lib().moe_nvfp4_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                     _dev(sink, torch.int32, "sink", 1), _stream(stream))
    _check("moe_nvfp4_stream_read", rc)


def moe_nvfp4_route(logits, k, topk_ids, topk_weights, stream=None) -> None:
    """Router ahead of the path: top-k experts and renormalised softmax
    weights of each row of f32 logits [T, E] (see the C header)."""
    T, E = logits.shape
    rc = lib().moe_nvfp4_route(_dev(logits, torch.float32, "logits"), T, E, k,
                               _dev(topk_ids, torch.int32, "topk_ids", T * k),
                               _dev(topk_weights, torch.float32, "topk_weights", T * k), _stream(stream))
    _check("moe_nvfp4_route", rc)


def with_shared_expert(topk_ids: torch.Tensor, topk_weights: torch.Tensor, shared_id: int):
    """Routing that also sends every token to a shared expert with weight 1.

    The pages run the shared expert in the same gate+up and down launches as
    the routed ones, as extra block rows over all tokens, and add its output
    in the blend (nvfp4_moe_grouped.rs, doc of
    moe_expert_gate_up_act_nvfp4_grouped: the first block rows are the
    shared expert, written to their own rows).  Here the shared expert is one
    more slot of the expert tables (usually index E of E + 1) and this
    appends it as a (k+1)-th route of every token: the sort gives it all T
    rows, the same launches compute it with the routed experts, and the blend
    adds it last with weight 1.  Returns new int32 [T, k+1] and f32 [T, k+1]
    device tensors; call the layer with E + 1 experts and k + 1.
    """
    T = topk_ids.shape[0]
    dev = topk_ids.device
    ids = torch.cat([topk_ids, torch.full((T, 1), int(shared_id), dtype=torch.int32, device=dev)], dim=1)
    w = torch.cat([topk_weights, torch.ones((T, 1), dtype=torch.float32, device=dev)], dim=1)
    return ids.contiguous(), w.contiguous()


def transpose_for_gemm(packed: torch.Tensor, scale: torch.Tensor, n: int, k: int, group_size: int = 16):
    """Load-time K-major twin (transpose.rs, transpose_for_gemm_gs): new
    buffers packed [K/2, N] and scales [K/group, N]; the inputs are left
    unchanged.  Both transposes run on the current stream, which is
    synchronized before the twin is returned."""
    pt = torch.empty((k // 2, n), dtype=torch.uint8, device=packed.device)
    st = torch.empty((k // group_size, n), dtype=torch.uint8, device=scale.device)
    transpose_u8(packed, pt, n, k // 2)
    transpose_u8(scale, st, n, k // group_size)
    torch.cuda.current_stream().synchronize()
    return pt, st


def transpose_concat_for_gemm(parts, k: int, group_size: int = 16, align: int = 16):
    """Load-time concatenated K-major twin (transpose.rs,
    transpose_concat_for_gemm_padded): parts [(packed [n, K/2], scale
    [n, K/group], n), ...] sharing K, transposed side by side into packed
    [K/2, stride] and scales [K/group, stride], stride = sum(n) rounded up to
    ``align``, pad columns zero.  Returns (packed, scale, stride); the stream
    is synchronized before returning."""
    if not parts:
        raise ValueError("transpose_concat_for_gemm: empty parts")
    n_total = sum(n for _, _, n in parts)
    stride = -(-n_total // align) * align
    dev = parts[0][0].device
    pt = torch.zeros((k // 2, stride), dtype=torch.uint8, device=dev)
    st = torch.zeros((k // group_size, stride), dtype=torch.uint8, device=dev)
    off = 0
    for packed, scale, n in parts:
        transpose_u8_pitched(packed, pt, n, k // 2, stride, off)
        transpose_u8_pitched(scale, st, n, k // group_size, stride, off)
        off += n
    torch.cuda.current_stream().synchronize()
    return pt, st, stride


class MoeLayer:
    """Device buffers and the four calls of one MoE layer forward.

    ``gate``, ``up`` and ``down`` are ExpertTables (the same layout for all
    three).  ``forward`` enqueues sort -> gate_up_silu -> down -> blend on
    the current stream (with sort and gate+up, or down and blend, fused into
    one launch where that pays) and returns the bf16 output [T, H]; the
    intermediate buffers stay available as attributes for inspection.
    """

    def __init__(self, T: int, k: int, E: int, H: int, I: int, gate: ExpertTables, up: ExpertTables,
                 down: ExpertTables, device="cuda", gate_up: Optional[ExpertTables] = None, pitch: int = 0):
        self.T, self.k, self.E, self.H, self.I = T, k, E, H, I
        self.gate, self.up, self.down = gate, up, down
        # Optional concatenated gate||up twin (used instead of gate and up).
        self.gate_up, self.pitch = gate_up, pitch
        P = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.sorted_token_ids = torch.empty(P, **i32)
        self.pair_pos = torch.empty(P, **i32)
        self.active_experts = torch.empty(E, **i32)
        self.active_count = torch.empty(1, **i32)
        self.err_flag = torch.zeros(1, **i32)
        self.h = torch.empty((P, I), dtype=torch.float32, device=device)
        self.y = torch.empty((P, H), dtype=torch.float32, device=device)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=device)

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, stream=None,
                fuse_sort: bool = True, fuse_blend: Optional[bool] = None):
        """``fuse_sort``: sort and gate+up through moe_nvfp4_sort_gate_up_silu
        (one launch for few-token decode); False issues the two calls.
        ``fuse_blend``: down and blend through moe_nvfp4_down_blend (one
        launch, ``y`` is not written); None picks it for one token with
        row-major weights when the library admits the shape, else the two
        calls."""
        s = _stream(stream)
        if self.gate_up is not None:
            moe_nvfp4_sort(topk_ids, self.E, self.expert_offsets, self.sorted_token_ids, self.pair_pos,
                           self.active_experts, self.active_count, self.err_flag, s)
            moe_nvfp4_gate_up_silu_concat(x, self.k, self.E, self.H, self.I, self.gate_up, self.pitch,
                                          self.expert_offsets, self.sorted_token_ids, self.active_experts,
                                          self.active_count, self.h, s)
        elif fuse_sort:
            moe_nvfp4_sort_gate_up_silu(topk_ids, x, self.E, self.H, self.I, self.gate, self.up,
                                        self.expert_offsets, self.sorted_token_ids, self.pair_pos,
                                        self.active_experts, self.active_count, self.err_flag, self.h, s)
        else:
            moe_nvfp4_sort(topk_ids, self.E, self.expert_offsets, self.sorted_token_ids, self.pair_pos,
                           self.active_experts, self.active_count, self.err_flag, s)
            moe_nvfp4_gate_up_silu(x, self.k, self.E, self.H, self.I, self.gate, self.up, self.expert_offsets,
                                   self.sorted_token_ids, self.active_experts, self.active_count, self.h, s)
        if fuse_blend is None:
            fuse_blend = self.T == 1 and self.down.layout == ROW_MAJOR
            if fuse_blend:
                rc = _down_blend_rc(self.h, topk_ids, topk_weights, self.pair_pos, self.E, self.H, self.I,
                                    self.down, self.out, s)
                if rc == 0:
                    return self.out
                if rc != _ELIMIT:  # ELIMIT: the shape is not admitted; issue the two calls
                    _check("moe_nvfp4_down_blend", rc)
        elif fuse_blend:
            moe_nvfp4_down_blend(self.h, topk_ids, topk_weights, self.pair_pos, self.E, self.H, self.I,
                                 self.down, self.out, s)
            return self.out
        moe_nvfp4_down(self.h, self.T, self.k, self.E, self.H, self.I, self.down, self.expert_offsets,
                       self.active_experts, self.active_count, self.y, s)
        moe_nvfp4_blend(self.y, topk_weights, self.pair_pos, self.out, s)
        return self.out
