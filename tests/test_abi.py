"""C-ABI contract checks that run without a GPU.

The library must load, export every function ``include/hyena_conv.h``
declares, and reject bad arguments on the host before any HIP call (so these
calls are safe on a machine with no GPU: rejected calls never reach the
runtime).  Pointers below are fake, non-dereferenced addresses.
"""
import ctypes
import os
import re

import pytest

import gated_convolution_sequence_amd as hc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyena_conv.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(hc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hc.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyena_conv_\w+)\s*\(", text)))


def test_header_declares_the_python_export_list():
    assert _declared_functions() == sorted(hc.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hc.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_block_len_and_strerror():
    assert hc.lib().hyena_conv_block_len() == 64 == hc.BLOCK_LEN
    for code in list(hc.STATUS) + [-100, 7]:
        assert isinstance(hc.strerror(code), str) and hc.strerror(code)
    assert hc.strerror(0) == "ok"


A = 1 << 20  # fake 16-byte-aligned device addresses, far apart
P = dict(q=A, k=2 * A << 8, v=3 * A << 8, h=4 * A << 8, out=5 * A << 8)


def _call(q=P["q"], k=P["k"], v=P["v"], h=P["h"], B=1, L=128, D=64, gs=16, l_h=7,
          out=P["out"], dtype=hc.DTYPE_BF16, span=0):
    return hc.lib().hyena_conv_fwd_ex(q, k, v, h, B, L, D, gs, l_h, out, dtype, span, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(h=None), -1),
    (dict(out=None), -1),
    (dict(B=-1), -2), (dict(L=-5), -2), (dict(D=-16), -2),
    (dict(L=1 << 40, D=1 << 30), -2),
    (dict(gs=0), -3), (dict(D=64, gs=48), -3),
    (dict(l_h=0), -4), (dict(l_h=129), -4), (dict(l_h=-3), -4),
    (dict(q=P["q"] + 8), -5), (dict(out=P["out"] + 2), -5), (dict(h=P["h"] + 1), -5),
    (dict(dtype=hc.DTYPE_F32, h=P["h"] + 2), -5),
    (dict(out=P["q"]), -6), (dict(out=P["k"] + 64), -6), (dict(out=P["v"] - 16), -6),
    (dict(out=P["h"] - 64), -6),
    # group sizes that are not a multiple of 16 need 16-byte rows
    (dict(D=12, gs=1), -7), (dict(D=36, gs=4), -7), (dict(D=6, gs=3, dtype=hc.DTYPE_F32), -7),
    (dict(dtype=2), -9), (dict(dtype=-1), -9),
])
def test_host_validation_rejects_before_any_gpu_call(kw, code):
    assert _call(**kw) == code


def _call_named(name, q=P["q"], k=P["k"], v=P["v"], h=P["h"], B=1, L=128, D=64, gs=16, l_h=7,
                out=P["out"]):
    return getattr(hc.lib(), name)(q, k, v, h, B, L, D, gs, l_h, out, None)


@pytest.mark.parametrize("name,eb", [("hyena_conv_fwd", 2), ("hyena_conv_fwd_f32", 4)])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(h=None), -1),
    (dict(out=None), -1),
    (dict(B=-1), -2), (dict(L=-5), -2), (dict(D=-16), -2), (dict(L=1 << 40, D=1 << 30), -2),
    (dict(gs=0), -3), (dict(D=64, gs=48), -3),
    (dict(l_h=0), -4), (dict(l_h=129), -4),
    (dict(q=P["q"] + 8), -5), (dict(out=P["out"] + 4), -5),
    (dict(out=P["q"]), -6), (dict(out=P["k"] + 64), -6), (dict(out=P["h"] - 64), -6),
])
def test_named_forward_entry_points_validate_on_host(name, eb, kw, code):
    """The two entry points with the operator's own signature (bf16 and fp32)
    run the same host checks as the explicit-dtype one."""
    assert _call_named(name, **kw) == code


def test_named_forward_entry_points_check_their_own_element_size():
    # a filter aligned for bf16 but not for fp32 is refused only by the fp32 entry
    assert _call_named("hyena_conv_fwd_f32", h=P["h"] + 2) == -5
    assert _call_named("hyena_conv_fwd", h=P["h"] + 1) == -5
    # rows of 24 bytes (12 bf16 or 6 fp32 channels) are not a multiple of 16 off the tile
    assert _call_named("hyena_conv_fwd", D=12, gs=1) == -7
    assert _call_named("hyena_conv_fwd_f32", D=6, gs=3) == -7
    for name in ("hyena_conv_fwd", "hyena_conv_fwd_f32"):
        assert _call_named(name, q=None, k=None, v=None, h=None, out=None, B=0) == 0


def test_empty_problems_are_noops_even_with_null_pointers():
    for B, L, D in [(0, 10, 16), (1, 0, 16), (1, 10, 0)]:
        assert _call(q=None, k=None, v=None, h=None, out=None, B=B, L=L, D=D) == 0


def test_error_precedence_shape_checks_come_first():
    # sizes are judged before pointers: a bad l_h with NULL pointers reports l_h
    assert _call(q=None, l_h=0) == -4
    assert _call(q=None, gs=3, D=64) == -3


def test_binding_raises_with_status():
    with pytest.raises(hc.HyenaError) as ei:
        hc.plan(1, 128, 12, 1, 7)
    assert ei.value.status == -7


@pytest.mark.parametrize("B,L,D,l_h,dtype,span,expect_span", [
    # SE (l_h <= 33) in bf16: 256-channel slabs, spans up to 8 chunks while
    # the grid keeps at least 256 workgroups
    (1, 8192, 4096, 7, 0, 0, 8), (1, 16384, 4096, 7, 0, 0, 8), (1, 4096, 4096, 7, 0, 0, 4),
    (1, 2048, 4096, 7, 0, 0, 2), (1, 1024, 4096, 7, 0, 0, 1), (4, 8192, 4096, 33, 0, 0, 8),
    (1, 8192, 4096, 7, 1, 0, 2), (1, 8192, 4096, 128, 0, 0, 8),
    (4, 32768, 4096, 128, 0, 0, 8), (1, 1024, 256, 7, 1, 0, 2),
    (1, 1000, 64, 7, 0, 3, 2), (1, 1000, 64, 7, 0, 7, 4), (1, 100, 64, 7, 0, 50, 2),
    (1, 1 << 20, 4096, 128, 0, 0, 8), (1, 1 << 20, 4096, 128, 1, 0, 4),
    (1, 1 << 20, 4096, 128, 0, 1000, 32), (1, 1 << 20, 4096, 128, 1, 1000, 4),
    (1, 130, 64, 7, 0, 0, 1), (1, 60, 64, 128, 0, 0, 1), (1, 8192, 4096, 66, 0, 0, 4),
    (1, 8192, 4096, 1, 0, 0, 8),
])
def test_plan_split(B, L, D, l_h, dtype, span, expect_span):
    s, wgs = hc.plan(B, L, D, 16, l_h, dtype, span)
    assert s == expect_span
    chunks = -(-L // 64)
    # the 16-wave kernel: bf16 SE always, longer filters from 1024 workgroups
    # at 8-chunk spans
    wide = dtype == hc.DTYPE_BF16 and (l_h <= 33 or B * (-(-D // 256)) * (-(-chunks // 8)) >= 1024)
    slab = hc.WIDE_SLAB if wide else hc.SLAB
    assert wgs == B * (-(-D // slab)) * (-(-chunks // s))


@pytest.mark.parametrize("B,L,D,gs,l_h,dtype,span,expect_span", [
    # group sizes off the 16-channel tile, filters longer than 8 taps (the
    # chunk-direction GEMMs): spans of whole 256-row blocks (4 chunks each), by
    # default long enough for about one workgroup per CU
    (1, 8192, 4096, 1, 128, 0, 0, 32), (1, 8192, 4096, 8, 33, 1, 0, 64), (4, 32768, 4096, 2, 128, 0, 0, 512),
    (1, 100, 64, 1, 128, 0, 0, 4), (1, 1000, 72, 24, 65, 0, 0, 4), (1, 1 << 20, 4096, 1, 128, 0, 0, 4096),
    (1, 1000, 64, 1, 9, 0, 9, 12), (2, 1000, 96, 3, 9, 1, 3, 4),
])
def test_plan_split_chunk_direction(B, L, D, gs, l_h, dtype, span, expect_span):
    s, wgs = hc.plan(B, L, D, gs, l_h, dtype, span)
    assert s == expect_span
    slab = 32 if dtype == hc.DTYPE_F32 else 64  # 8 waves x one 16-byte row segment each
    blocks = -(-L // 256)
    assert wgs == B * (-(-D // slab)) * (-(-blocks // (s // 4)))


@pytest.mark.parametrize("B,L,D,gs,l_h,dtype,span,expect_span", [
    # off the tile with at most 8 taps (the direct kernel): one 64-lane
    # workgroup per 256 channels and span; spans of 256 rows halved (down to
    # 64) while there are fewer than 1024 workgroups, or the requested chunks
    # (at most the sequence)
    (1, 8192, 4096, 1, 7, 0, 0, 2), (1, 8192, 4096, 1, 8, 1, 0, 2), (4, 32768, 4096, 2, 4, 0, 0, 4),
    (1, 100, 64, 1, 7, 0, 0, 1), (1, 1 << 20, 4096, 2, 1, 0, 0, 4),
    (2, 1000, 96, 3, 7, 1, 3, 3), (1, 1000, 64, 1, 7, 0, 9, 9), (1, 1 << 20, 4096, 2, 2, 0, 1000, 1000),
    (1, 3000, 64, 1, 7, 0, 10 ** 6, 47),
])
def test_plan_split_direct(B, L, D, gs, l_h, dtype, span, expect_span):
    s, wgs = hc.plan(B, L, D, gs, l_h, dtype, span)
    assert s == expect_span
    assert wgs == B * (-(-D // 256)) * (-(-L // (64 * s)))


def test_plan_chunk_direction_window():
    # buffer windows are per block: any span length; only a row of 384
    # rows x D elements must stay below 2^31 bytes
    s, _ = hc.plan(1, 1 << 16, 1 << 20, 1, 128, hc.DTYPE_BF16, 0)
    assert s == (1 << 16) // 64
    with pytest.raises(hc.HyenaError):
        hc.plan(1, 256, 1 << 22, 2, 65, hc.DTYPE_F32, 0)
    # the direct kernel's window is a span plus 8 rows: default spans shrink
    # (down to one chunk) to keep it below 2^31 bytes
    s, _ = hc.plan(1, 256, 1 << 21, 2, 7, hc.DTYPE_F32, 0)
    assert s == 2
    s, _ = hc.plan(1, 256, 1 << 22, 2, 7, hc.DTYPE_F32, 0)
    assert s == 1
    with pytest.raises(hc.HyenaError):
        hc.plan(1, 256, 1 << 24, 2, 7, hc.DTYPE_F32, 0)
    with pytest.raises(hc.HyenaError):
        hc.plan(1, 256, 1 << 22, 2, 7, hc.DTYPE_F32, 4)


def test_plan_keeps_the_window_addressable():
    # a very wide row forces short spans: (span*64 + history + 64) * D * 2 < 2^31
    D = 1 << 20
    s, _ = hc.plan(1, 1 << 16, D, 16, 128, hc.DTYPE_BF16, 0)
    assert (s * 64 + 128 + 64) * D * 2 < 1 << 31
    with pytest.raises(hc.HyenaError):
        hc.plan(1, 64, 1 << 24, 16, 128, hc.DTYPE_F32, 0)


def test_binding_validates_tensors_on_host():
    import torch
    q = torch.zeros(1, 8, 16)
    with pytest.raises(ValueError):
        hc.conv_fwd(q, q, q, torch.zeros(1, 3), 16)  # CPU tensors are refused


def _halo(kp=P["k"] + (64 << 20), vp=P["v"] + (64 << 20), Pn=127, out=P["out"], **kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], h=P["h"], B=1, L=128, D=64, gs=16, l_h=7,
             dtype=hc.DTYPE_BF16, span=0)
    a.update(kw)
    return hc.lib().hyena_conv_fwd_halo(a["q"], a["k"], a["v"], a["h"], kp, vp, Pn, a["B"], a["L"],
                                        a["D"], a["gs"], a["l_h"], out, a["dtype"], a["span"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Pn=-1), -2), (dict(kp=None), -1), (dict(vp=None), -1),
    (dict(kp=P["k"] + (64 << 20) + 8), -5), (dict(vp=P["v"] + (64 << 20) + 4), -5),
    (dict(out=P["k"] + (64 << 20)), -6), (dict(out=P["v"] + (64 << 20) - 16), -6),
    (dict(l_h=200), -4), (dict(D=12, gs=3, l_h=9), -7),
])
def test_halo_entry_validates_its_prefix_on_host(kw, code):
    assert _halo(**kw) == code


def test_halo_entry_without_prefix_needs_no_prefix_pointers():
    # P = 0: same checks as the plain entry point; still rejected before launch
    assert _halo(kp=None, vp=None, Pn=0, q=None) == -1


def _bwd(q=P["q"], k=P["k"], v=P["v"], h=P["h"], dy=P["out"] + (64 << 20), B=1, L=128, D=64,
         gs=16, l_h=7, dq=P["out"], dk=P["out"] + (16 << 20), dv=P["out"] + (32 << 20),
         dh=P["out"] + (48 << 20), ws=P["out"] + (96 << 20), ws_n=1 << 20, dtype=hc.DTYPE_BF16):
    return hc.lib().hyena_conv_bwd(q, k, v, h, dy, B, L, D, gs, l_h, dq, dk, dv, dh, ws, ws_n,
                                   dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), -1), (dict(q=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(dh=P["out"] + (48 << 20) + 2), -5), (dict(dq=P["out"] + 8), -5),
    (dict(ws=P["out"] + (96 << 20) + 4), -5),
    (dict(dq=P["q"]), -6), (dict(dk=P["out"]), -6), (dict(dh=P["k"] + 64), -6),
    (dict(ws=P["v"]), -6), (dict(ws=P["out"] + (16 << 20)), -6),
    (dict(ws=None), -10), (dict(ws_n=16), -10),
    (dict(l_h=0), -4), (dict(D=12, gs=3, l_h=9), -7), (dict(D=12, gs=1, l_h=7), -7), (dict(dtype=5), -9),
])
def test_backward_validates_on_host(kw, code):
    assert _bwd(**kw) == code


def test_backward_workspace_size():
    # one float per (batch row, span of the filter-gradient pass, 16-channel tile, tap)
    n = hc.bwd_workspace_bytes(1, 8192, 4096, 16, 128)
    assert n == 1 * (8192 // (64 * 16)) * (4096 // 16) * 128 * 4
    assert hc.bwd_workspace_bytes(0, 8192, 4096, 16, 128) == 0
    with pytest.raises(hc.HyenaError):
        hc.bwd_workspace_bytes(1, 64, 64, 16, 300)
    # off the 16-channel tile, at most 8 taps: one partial row of l_h floats
    # per span (the direct plan's), batch row and channel; longer filters are
    # not supported there
    for B, L, D, gs, l_h in ((1, 8192, 4096, 1, 7), (2, 1000, 96, 3, 5), (1, 100, 8, 2, 1)):
        span, _ = hc.plan(B, L, D, gs, l_h)
        assert hc.bwd_workspace_bytes(B, L, D, gs, l_h) == B * (-(-L // (64 * span))) * D * l_h * 4
    # longer filters off the tile: one partial row per 1024-row span, batch
    # row and channel (the lag-product pass); rows of 24 bytes are refused
    for B, L, D, gs, l_h in ((1, 8192, 4096, 8, 9), (2, 1000, 96, 3, 128), (3, 2049, 64, 1, 65)):
        assert hc.bwd_workspace_bytes(B, L, D, gs, l_h) == B * (-(-L // 1024)) * D * l_h * 4
    with pytest.raises(hc.HyenaError):
        hc.bwd_workspace_bytes(1, 8192, 12, 3, 9)
    # very wide rows: the lag-product pass addresses a span's rows, and the
    # 160 rows of history before it, with 32-bit byte offsets, so its spans
    # shrink in 64-row chunks to keep that window below 2^31 bytes
    D = 1 << 20
    for code, eb in ((hc.DTYPE_BF16, 2), (hc.DTYPE_F32, 4)):
        rows = ((2 ** 31 - 1) // (eb * D) - 160) // 64 * 64
        assert rows in (832, 320)
        assert hc.bwd_workspace_bytes(1, 8192, D, 8, 100, code) == (-(-8192 // rows)) * D * 100 * 4


def _long(q=P["q"], k=P["k"], v=P["v"], h=P["h"], B=1, L=128, D=64, gs=16, l_h=1000,
          out=P["out"], dtype=hc.DTYPE_BF16, ws=P["out"] + (64 << 20), ws_n=1 << 30):
    return hc.lib().hyena_conv_fwd_long(q, k, v, h, B, L, D, gs, l_h, out, dtype, ws, ws_n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(h=None), -1), (dict(out=None), -1),
    (dict(B=-1), -2), (dict(gs=0), -3), (dict(D=64, gs=48), -3), (dict(l_h=0), -4),
    (dict(D=63, gs=1), -7), (dict(L=1 << 23), -7),
    (dict(q=P["q"] + 8), -5), (dict(h=P["h"] + 1), -5), (dict(ws=P["out"] + (64 << 20) + 4), -5),
    (dict(out=P["k"]), -6), (dict(ws=P["v"]), -6), (dict(ws=P["out"]), -6),
    (dict(ws=None), -10), (dict(ws_n=1024), -10), (dict(dtype=3), -9),
])
def test_long_filter_entry_validates_on_host(kw, code):
    assert _long(**kw) == code


def test_long_filter_workspace_size():
    # N = 2^ceil(log2(L + min(l_h, L) - 1)); 8 N (max(B D/2, G'/2) + G') bytes
    def expect(B, L, D, gs, l_h):
        n = 1 << max(2, (L + min(l_h, L) - 2).bit_length())
        G = D // gs
        Gp = G + (G & 1)
        return 8 * n * (max(B * D // 2, Gp // 2) + Gp)
    for args in [(1, 8192, 4096, 16, 8192), (2, 1000, 64, 1, 37), (1, 5, 6, 3, 1000), (3, 1, 2, 1, 1)]:
        assert hc.long_workspace_bytes(*args) == expect(*args), args
    assert hc.long_workspace_bytes(0, 8192, 4096, 16, 8192) == 0
    with pytest.raises(hc.HyenaError):
        hc.long_workspace_bytes(1, 100, 7, 1, 10)  # odd D


def test_long_filter_plan_rejects_unaddressable_sizes():
    """Filter lengths past a 32-bit row pitch, element counts past 2^60 and
    workspace sizes past 2^63 bytes are refused on the host."""
    n = ctypes.c_int64(-1)
    ws = lambda B, L, D, gs, l_h: hc.lib().hyena_conv_fwd_long_workspace(B, L, D, gs, l_h, hc.DTYPE_BF16,
                                                                         ctypes.byref(n))
    assert ws(1, 100, 64, 16, (1 << 31)) == -7          # l_h past a 32-bit pitch
    assert ws(1, 100, 64, 16, (1 << 31) - 1) == 0       # (taps past L never contribute)
    assert ws(1 << 40, 1 << 20, 1 << 20, 16, 7) == -2   # B L D overflows
    assert ws(1, 1 << 62, 64, 16, 7) == -7              # longer than one transform
    assert ws(1 << 30, 1, (1 << 30) - 2, 1, 1) == -2    # workspace bytes overflow
    assert ws(1, 100, (1 << 30) - 2, 1, (1 << 31) - 1) == -2  # G l_h taps overflow
    assert _long(l_h=1 << 31) == -7
    assert _long(B=1 << 40, L=1 << 20, D=1 << 20) == -2


def test_long_filter_spectra_flag_is_checked_on_host():
    lib = hc.lib()
    a = dict(q=P["q"], k=P["k"], v=P["v"], h=P["h"], out=P["out"], ws=P["out"] + (64 << 20))
    call = lambda h, flag: lib.hyena_conv_fwd_long_ex(a["q"], a["k"], a["v"], h, 1, 128, 64, 16, 1000,
                                                      a["out"], hc.DTYPE_BF16, a["ws"], 1 << 10, flag, None)
    assert call(a["h"], 2) == -2 and call(a["h"], -1) == -2
    assert call(None, 0) == -1          # the spectra are computed from h
    assert call(None, 1) == -10         # h is not needed with kept spectra; the workspace still is


def _bwd_long(q=P["q"], k=P["k"], v=P["v"], h=P["h"], dy=P["out"] + (128 << 20), B=1, L=128, D=64, gs=16,
              l_h=1000, dq=P["out"], dk=P["out"] + (1 << 20), dv=P["out"] + (2 << 20),
              dh=P["out"] + (3 << 20), dtype=hc.DTYPE_BF16, ws=P["out"] + (64 << 20), ws_n=1 << 30):
    return hc.lib().hyena_conv_bwd_long(q, k, v, h, dy, B, L, D, gs, l_h, dq, dk, dv, dh, dtype, ws, ws_n,
                                        None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(dy=None), -1), (dict(h=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(B=-1), -2), (dict(gs=0), -3), (dict(D=64, gs=48), -3), (dict(l_h=0), -4),
    (dict(D=63, gs=1), -7), (dict(L=1 << 23), -7),
    (dict(q=P["q"] + 8), -5), (dict(dq=P["out"] + 8), -5), (dict(dh=P["out"] + (3 << 20) + 2), -5),
    (dict(ws=P["out"] + (64 << 20) + 4), -5),
    (dict(dq=P["k"]), -6), (dict(dh=P["h"]), -6), (dict(ws=P["v"]), -6), (dict(ws=P["out"]), -6),
    (dict(dk=P["out"] + (2 << 20), dv=P["out"] + (2 << 20)), -6),
    (dict(ws=None), -10), (dict(ws_n=1024), -10), (dict(dtype=3), -9),
])
def test_long_filter_backward_validates_on_host(kw, code):
    assert _bwd_long(**kw) == code


def test_long_filter_backward_without_outputs_is_a_host_no_op():
    assert _bwd_long(dq=None, dk=None, dv=None, dh=None, ws=None, ws_n=0) == 0


def test_long_filter_backward_workspace_size():
    # 8 N (G' + B D + B T S): spectra, the x and dz work areas, and the
    # filter gradient's partial sums (T column tiles of P channel pairs, S
    # group slots per tile).  P: the largest power of two <= 64 with c N1 P <=
    # 4096 complex values of LDS, no larger than needed for D / 2 pairs; c = 2
    # for even group sizes (single columns), 4 otherwise (column pairs); both
    # transformed in place.
    def expect(B, L, D, gs, l_h):
        n = 1 << max(2, (L + min(l_h, L) - 2).bit_length())
        log_n = n.bit_length() - 1
        log1 = (log_n + 2) // 3 if log_n > 16 else (log_n + 1) // 2
        n1 = 1 << log1
        P = 64
        while P > 1 and (2 if gs % 2 == 0 else 4) * n1 * P > 4096:
            P //= 2
        while P > 1 and P // 2 >= D // 2:
            P //= 2
        G = D // gs
        Gp = G + (G & 1)
        T = (D // 2 + P - 1) // P
        S = min(G, (2 * P - 1 + gs - 1) // gs + 1)
        assert T * S <= G + D
        return 8 * n * (Gp + B * D + B * T * S)
    for args in [(1, 8192, 4096, 16, 8192), (2, 1000, 64, 1, 37), (1, 5, 6, 3, 1000), (3, 1, 2, 1, 1),
                 (1, 1 << 20, 64, 64, 1 << 20), (2, 3000, 10, 5, 100)]:
        assert hc.bwd_long_workspace_bytes(*args) == expect(*args), args
    assert hc.bwd_long_workspace_bytes(0, 8192, 4096, 16, 8192) == 0
    with pytest.raises(hc.HyenaError):
        hc.bwd_long_workspace_bytes(1, 100, 7, 1, 10)  # odd D


def test_long_filter_backward_spectra_flag_is_checked_on_host():
    lib = hc.lib()
    a = dict(q=P["q"], k=P["k"], v=P["v"], h=P["h"], dy=P["out"] + (128 << 20), dq=P["out"],
             dk=P["out"] + (1 << 20), dv=P["out"] + (2 << 20), dh=P["out"] + (3 << 20), ws=P["out"] + (64 << 20))
    call = lambda h, flag: lib.hyena_conv_bwd_long_ex(a["q"], a["k"], a["v"], h, a["dy"], 1, 128, 64, 16, 1000,
                                                      a["dq"], a["dk"], a["dv"], a["dh"], hc.DTYPE_BF16, a["ws"],
                                                      1 << 10, flag, None)
    assert call(a["h"], 2) == -2 and call(a["h"], -1) == -2
    assert call(None, 0) == -1          # the spectra are computed from h
    assert call(None, 1) == -10         # h is not needed with kept spectra; the workspace still is
