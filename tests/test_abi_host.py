"""The C-ABI library on the host: it loads, exports every declared entry
point, and rejects bad arguments before launching anything (CPU only: every
call below fails the host-side check, so no GPU work is enqueued)."""
import ctypes

import pytest

import nvfp4_quantized_moe_amd as moe
from nvfp4_quantized_moe_amd import _Experts

ENULL, ESHAPE, ELAYOUT, ELIMIT = -1, -2, -3, -4
D = 0x1000  # a non-NULL dummy address, never dereferenced on these paths


def test_library_exports_every_header_function():
    L = moe.lib()
    names = moe.header_functions()
    assert set(names) >= {"moe_nvfp4_sort", "moe_nvfp4_gate_up_silu", "moe_nvfp4_down", "moe_nvfp4_blend",
                          "transpose_u8", "moe_nvfp4_abi_version", "moe_nvfp4_route", "transpose_u8_pitched",
                          "moe_nvfp4_gate_up_silu_concat", "moe_nvfp4_sort_gate_up_silu",
                          "moe_nvfp4_sort_gate_up_launches", "moe_nvfp4_down_blend", "moe_nvfp4_stream_read"}
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_nvfp4_abi_version() == 7


def _ex(layout=0, null=False):
    return _Experts(0 if null else D, D, D, layout)


def test_sort_rejects():
    L = moe.lib()
    ok = [D, 4, 2, 4, D, D, D, D, D, D, None]
    for i in (0, 4, 5, 6, 7, 8, 9):
        a = list(ok)
        a[i] = None
        assert L.moe_nvfp4_sort(*a) == ENULL
    assert L.moe_nvfp4_sort(D, 0, 2, 4, D, D, D, D, D, D, None) == ESHAPE
    assert L.moe_nvfp4_sort(D, 4, 0, 4, D, D, D, D, D, D, None) == ESHAPE
    assert L.moe_nvfp4_sort(D, 4, 5, 4, D, D, D, D, D, D, None) == ESHAPE    # k > E
    assert L.moe_nvfp4_sort(D, 4, 2, 2000, D, D, D, D, D, D, None) == ELIMIT
    assert L.moe_nvfp4_sort(D, 1 << 21, 8, 16, D, D, D, D, D, D, None) == ELIMIT


def test_gate_up_rejects():
    L = moe.lib()

    def call(x=D, T=4, k=2, E=4, H=256, I=512, g=None, u=None, h=D):
        return L.moe_nvfp4_gate_up_silu(x, T, k, E, H, I, g or _ex(), u or _ex(), D, D, D, D, h, None)

    assert call(x=None) == ENULL
    assert call(h=None) == ENULL
    assert call(g=_ex(null=True)) == ENULL
    assert call(g=_ex(0), u=_ex(1)) == ELAYOUT
    assert call(g=_ex(1), u=_ex(2)) == ELAYOUT          # NVFP4 gate with MXFP4 up
    assert call(g=_ex(7), u=_ex(7)) == ELAYOUT
    assert call(g=_ex(3), u=_ex(3)) == ELAYOUT
    assert call(H=48) == ESHAPE                         # H % 64 != 0
    assert call(H=96) == ESHAPE                         # H % 64 != 0
    assert call(H=192) == ESHAPE                        # row-major needs H >= 256
    assert call(I=528, g=_ex(1), u=_ex(1)) == ESHAPE    # K-major needs I % 64 == 0
    assert call(k=5) == ESHAPE
    assert call(H=1 << 17) == ELIMIT
    assert call(H=36800) == ELIMIT                      # a row-major x row must fit the decode kernel's LDS
    # K-major: x of 4 GiB or more (activation offsets are 32-bit)
    assert call(T=1 << 16, H=1 << 15, g=_ex(1), u=_ex(1)) == ELIMIT
    assert call(T=1 << 16, H=1 << 15, g=_ex(2), u=_ex(2)) == ELIMIT
    assert call(I=528, g=_ex(2), u=_ex(2)) == ESHAPE


def test_down_and_blend_and_transpose_reject():
    L = moe.lib()
    assert L.moe_nvfp4_down(None, 4, 2, 4, 256, 512, _ex(), D, D, D, D, None) == ENULL
    assert L.moe_nvfp4_down(D, 4, 2, 4, 256, 512, _ex(null=True), D, D, D, D, None) == ENULL
    assert L.moe_nvfp4_down(D, 4, 2, 4, 256, 500, _ex(), D, D, D, D, None) == ESHAPE
    # K-major: h of 4 GiB or more
    assert L.moe_nvfp4_down(D, 1 << 20, 4, 4, 256, 1024, _ex(1), D, D, D, D, None) == ELIMIT
    assert L.moe_nvfp4_down(D, 1 << 20, 4, 4, 256, 1024, _ex(2), D, D, D, D, None) == ELIMIT
    assert L.moe_nvfp4_down(D, 4, 2, 4, 256, 512, _ex(4), D, D, D, D, None) == ELAYOUT
    assert L.moe_nvfp4_blend(D, D, None, 4, 2, 256, D, None) == ENULL
    assert L.moe_nvfp4_blend(D, D, D, 0, 2, 256, D, None) == ESHAPE
    assert L.moe_nvfp4_blend(D, D, D, 4, 2, 1 << 17, D, None) == ELIMIT
    assert L.transpose_u8(None, D, 4, 4, None) == ENULL
    assert L.transpose_u8(D, D, 0, 4, None) == ESHAPE


def test_stream_read_rejects():
    L = moe.lib()
    L.moe_nvfp4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert L.moe_nvfp4_stream_read(None, 1024, D, None) == ENULL
    assert L.moe_nvfp4_stream_read(D, 1024, None, None) == ENULL
    assert L.moe_nvfp4_stream_read(D, 8, D, None) == ESHAPE
    assert L.moe_nvfp4_stream_read(D, 1000, D, None) == ESHAPE


def test_python_binding_checks_tensor_arguments():
    import torch

    with pytest.raises(ValueError):
        moe.transpose_u8(torch.zeros(4, dtype=torch.uint8), torch.zeros(4, dtype=torch.uint8), 2, 3)
    with pytest.raises((TypeError, ValueError)):
        moe.transpose_u8(torch.zeros(6, dtype=torch.uint8), torch.zeros(6, dtype=torch.uint8), 2, 3)


def test_python_binding_checks_buffer_sizes():
    """Buffers smaller than the sizes say are refused before any launch (the
    first argument of each call here, so the check runs before the tensors'
    placement is looked at)."""
    import torch

    i32 = dict(dtype=torch.int32)
    with pytest.raises(ValueError, match="y: needs at least 2048"):
        moe.moe_nvfp4_blend(torch.zeros((7, 256)), torch.zeros((4, 2)), torch.zeros(8, **i32),
                            torch.zeros((4, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="h: needs at least 4096"):
        moe.moe_nvfp4_down(torch.zeros((8, 500)), 4, 2, 4, 256, 512, _Table(), torch.zeros(5, **i32),
                           torch.zeros(4, **i32), torch.zeros(1, **i32), torch.zeros((8, 256)))
    with pytest.raises(ValueError, match="x: needs at least 1024"):
        moe.moe_nvfp4_gate_up_silu(torch.zeros((4, 128), dtype=torch.bfloat16), 2, 4, 256, 512, _Table(),
                                   _Table(), torch.zeros(5, **i32), torch.zeros(8, **i32), torch.zeros(4, **i32),
                                   torch.zeros(1, **i32), torch.zeros((8, 512)))


class _Table:
    """Stands in for an ExpertTables where only the argument checks run."""

    def check(self, *args, **kwargs):
        pass

    def abi(self):
        return _ex()


def _cpu_tables(n, k, E, layout=moe.ROW_MAJOR, short=None, missing_scale=None):
    """ExpertTables over CPU tensors (only the host-side checks look at them):
    E experts of [n, k]; expert ``short`` one scale byte short."""
    import torch

    g = 32 if layout == moe.K_MAJOR_MXFP4 else 16
    rows = []
    for e in range(E):
        pk = torch.zeros(n * k // 2, dtype=torch.uint8)
        sc = torch.zeros(n * k // g - (1 if e == short else 0), dtype=torch.uint8)
        rows.append((pk, None if e == missing_scale else sc, 1.0))
    return moe.ExpertTables(rows, layout, device="cpu")


def test_expert_tables_checked_against_the_call():
    """Tables shorter than E, or an expert smaller than the [N, K] weight
    the call reads, are refused before any launch; an expert with packed
    bytes but no scales is refused when the table is built."""
    import torch

    i32 = dict(dtype=torch.int32)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    args = (torch.zeros(5, **i32), torch.zeros(8, **i32), torch.zeros(4, **i32), torch.zeros(1, **i32),
            torch.zeros((8, 512)))
    good = _cpu_tables(512, 256, 4)
    with pytest.raises(ValueError, match="holds 3 experts, the call reads 4"):
        moe.moe_nvfp4_gate_up_silu(x, 2, 4, 256, 512, _cpu_tables(512, 256, 3), good, *args)
    with pytest.raises(ValueError, match="up: an expert holds"):
        moe.moe_nvfp4_gate_up_silu(x, 2, 4, 256, 512, good, _cpu_tables(512, 256, 4, short=2), *args)
    with pytest.raises(ValueError, match="down: an expert holds"):
        moe.moe_nvfp4_down(torch.zeros((8, 512)), 4, 2, 4, 256, 512, _cpu_tables(256, 512, 4, short=0),
                           *args[:1], *args[2:4], torch.zeros((8, 256)))
    with pytest.raises(ValueError, match="down: an expert holds"):   # MXFP4 scale group of 32
        moe.moe_nvfp4_down(torch.zeros((8, 512)), 4, 2, 4, 256, 512,
                           _cpu_tables(256, 512, 4, moe.K_MAJOR_MXFP4, short=3), *args[:1], *args[2:4],
                           torch.zeros((8, 256)))
    with pytest.raises(ValueError, match="packed or scale tensor but not both"):
        _cpu_tables(512, 256, 4, missing_scale=1)
    with pytest.raises(TypeError, match="uint8"):
        moe.ExpertTables([(torch.zeros(8, dtype=torch.int32), torch.zeros(8, dtype=torch.uint8), 1.0)],
                         moe.ROW_MAJOR, device="cpu")
    # the right sizes pass the table checks (and then stop at the CPU tensors)
    with pytest.raises(ValueError, match="expected a device tensor"):
        moe.moe_nvfp4_gate_up_silu(x, 2, 4, 256, 512, good, good, *args)
    # a concatenated twin is checked against its row pitch
    cc = moe.ExpertTables([(torch.zeros(128 * 1040, dtype=torch.uint8), torch.zeros(16 * 1040, dtype=torch.uint8),
                            1.0)] * 4, moe.K_MAJOR, device="cpu")
    with pytest.raises(ValueError, match="gate_up: an expert holds"):
        moe.moe_nvfp4_gate_up_silu_concat(x, 2, 4, 256, 512, cc, 1056, *args)


def test_route_rejects():
    L = moe.lib()
    assert L.moe_nvfp4_route(None, 4, 8, 2, D, D, None) == ENULL
    assert L.moe_nvfp4_route(D, 4, 8, 2, None, D, None) == ENULL
    assert L.moe_nvfp4_route(D, 0, 8, 2, D, D, None) == ESHAPE
    assert L.moe_nvfp4_route(D, 4, 8, 9, D, D, None) == ESHAPE    # k > E
    assert L.moe_nvfp4_route(D, 4, 8, 0, D, D, None) == ESHAPE
    assert L.moe_nvfp4_route(D, 4, 2000, 2, D, D, None) == ELIMIT  # E > MOE_NVFP4_MAX_EXPERTS
    assert L.moe_nvfp4_route(D, 4, 128, 65, D, D, None) == ELIMIT  # k > 64
    assert L.moe_nvfp4_route(D, 1 << 20, 8, 8, D, D, None) == ELIMIT  # T * k > MOE_NVFP4_MAX_PAIRS


def test_concat_gate_up_and_pitched_transpose_reject():
    L = moe.lib()

    def call(x=D, T=4, k=2, E=4, H=256, I=512, gu=None, pitch=1024, h=D):
        return L.moe_nvfp4_gate_up_silu_concat(x, T, k, E, H, I, gu or _ex(1), pitch, D, D, D, D, h, None)

    assert call(x=None) == ENULL
    assert call(gu=_ex(1, null=True)) == ENULL
    assert call(gu=_ex(0)) == ELAYOUT                   # the concatenated twin is K-major
    assert call(gu=_ex(5)) == ELAYOUT
    assert call(pitch=1008) == ESHAPE                   # pitch < 2I
    assert call(pitch=1032) == ESHAPE                   # pitch % 16 != 0
    assert call(H=96) == ESHAPE
    assert call(T=1 << 16, H=1 << 15) == ELIMIT         # x of 4 GiB or more
    assert L.transpose_u8_pitched(None, D, 4, 4, 4, None) == ENULL
    assert L.transpose_u8_pitched(D, D, 4, 4, 3, None) == ESHAPE    # pitch < rows
    assert L.transpose_u8_pitched(D, D, 0, 4, 4, None) == ESHAPE
    assert L.transpose_u8_pitched(D, D, 4, 1 << 30, 1 << 12, None) == ELIMIT


def test_sort_gate_up_rejects():
    L = moe.lib()

    def call(ids=D, x=D, T=4, k=2, E=4, H=256, I=512, g=None, u=None, err=D, h=D):
        return L.moe_nvfp4_sort_gate_up_silu(ids, x, T, k, E, H, I, g or _ex(), u or _ex(), D, D, D, D, D, err, h,
                                             None)

    assert call(ids=None) == ENULL
    assert call(err=None) == ENULL
    assert call(h=None) == ENULL
    assert call(g=_ex(0), u=_ex(1)) == ELAYOUT
    assert call(k=5) == ESHAPE                          # k > E
    assert call(H=192) == ESHAPE                        # row-major needs H >= 256
    assert call(E=2000) == ELIMIT


def test_sort_gate_up_launch_count_query():
    """Host-only query (no GPU work): K-major always sorts in its own launch;
    bad sizes are rejected like the projection's own checks."""
    L = moe.lib()
    assert L.moe_nvfp4_sort_gate_up_launches(2048, 4, 64, 4096, 1536, 1) == 2
    assert L.moe_nvfp4_sort_gate_up_launches(4, 2, 4, 256, 512, 7) == ELAYOUT
    assert L.moe_nvfp4_sort_gate_up_launches(4, 5, 4, 256, 512, 0) == ESHAPE


def test_down_blend_rejects():
    L = moe.lib()

    def call(h=D, T=1, k=8, E=128, H=2048, I=768, d=None, ids=D, w=D, pos=D, out=D):
        return L.moe_nvfp4_down_blend(h, T, k, E, H, I, d or _ex(), ids, w, pos, out, None)

    for kw in ("h", "ids", "w", "pos", "out"):
        assert call(**{kw: None}) == ENULL
    assert call(d=_ex(null=True)) == ENULL
    assert call(d=_ex(1)) == ELAYOUT                    # row-major weights only
    assert call(d=_ex(2)) == ELAYOUT
    assert call(I=500) == ESHAPE
    assert call(k=129) == ESHAPE                        # k > E
    assert call(k=65, E=256) == ELIMIT                  # more pairs than a block takes
    assert call(T=65536) == ELIMIT                      # one block row per token
    assert call(k=64, E=64, H=256, I=2048) == ELIMIT    # 64 staged rows of 2 I bytes exceed the budget
    assert call(k=36, E=64, H=256, I=1024) == ELIMIT    # 36 rows of 2064 bytes > 73728 (35 would fit)


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No CPU fallback: with the HIP library absent every entry point raises."""
    import torch

    monkeypatch.setattr(moe, "LIB_PATH", tmp_path / "libmoe_nvfp4.so")
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()
    with pytest.raises(RuntimeError, match="missing"):
        moe.transpose_u8(torch.zeros(4, dtype=torch.uint8), torch.zeros(4, dtype=torch.uint8), 2, 2)
