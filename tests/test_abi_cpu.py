"""C ABI checks that need no GPU: exports, geometry helper, argument validation.

Validation runs before any HIP call, so invalid calls return their status here
without a device.  These tests pass fake addresses only to calls that must be
rejected; they are skipped where a GPU is visible so that a validation bug
could never turn into a launch on a fake pointer.
"""
import ctypes
import os
import re

import pytest
import torch

from dynamic_convolution_amd import _native as N

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dwconv.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation only without a GPU")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(N.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = N.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in N.STATUS:
        s = N.status_str(code)
        assert s and s != "unknown status"
    assert N.status_str(12345) == "unknown status"


def _geo(n=2, ic=3, ih=9, iw=7, oc=3, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1):
    return [n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw]


def out_size(*geo):
    oh, ow = ctypes.c_int64(-1), ctypes.c_int64(-1)
    rc = N.lib().dwconv2d_out_size(*geo, ctypes.byref(oh), ctypes.byref(ow))
    return rc, oh.value, ow.value


def test_out_size_matches_oracle(orc):
    import itertools
    for ih, kh, sh, ph, dh in itertools.product((1, 2, 5, 8, 13), (1, 2, 3, 5, 7), (1, 2, 3), (0, 1, 3), (1, 2, 3)):
        rc, oh, ow = out_size(*_geo(ih=ih, iw=ih + 1, kh=kh, kw=kh, sh=sh, sw=sh, ph=ph, pw=ph, dh=dh, dw=dh))
        want_h = orc.out_size(ih, kh, sh, ph, dh)
        want_w = orc.out_size(ih + 1, kh, sh, ph, dh)
        if want_h < 1 or want_w < 1:
            assert rc == -2
        else:
            assert (rc, oh, ow) == (0, want_h, want_w)


@pytest.mark.parametrize("bad,code", [
    (dict(n=0), -2), (dict(ic=0), -2), (dict(kh=0), -2), (dict(sh=0), -2), (dict(dw=0), -2),
    (dict(ph=-1), -2), (dict(ih=2, kh=5, ph=0), -2), (dict(oc=4), -3), (dict(oc=7, ic=3), -3),
    (dict(n=1 << 31), -6), (dict(n=4096, ic=4096, ih=512, iw=512, oc=4096), -6),
])
def test_out_size_rejects(bad, code):
    assert out_size(*_geo(**bad))[0] == code


FAKE = 1 << 40  # never dereferenced: every call below must fail validation


@no_gpu
def test_fwd_validation():
    L = N.lib()
    g = _geo()
    assert L.dwconv2d_fwd(FAKE, FAKE, None, FAKE + 4096, *g, 7, None) == -4      # dtype
    assert L.dwconv2d_fwd(None, FAKE, None, FAKE + 4096, *g, 0, None) == -1      # null x
    assert L.dwconv2d_fwd(FAKE, FAKE, None, None, *g, 0, None) == -1             # null y
    assert L.dwconv2d_fwd(FAKE + 2, FAKE, None, FAKE + 4096, *g, 0, None) == -1  # misaligned f32
    assert L.dwconv2d_fwd(FAKE, FAKE + 1, None, FAKE + 4096, *g, 1, None) == -1  # misaligned f16
    assert L.dwconv2d_fwd(FAKE, FAKE, None, FAKE, *g, 0, None) == -7             # y aliases x
    assert L.dwconv2d_fwd(FAKE, FAKE + 4096, FAKE + 8, FAKE + 4096 - 8, *g, 0, None) == -7  # y overlaps w
    assert L.dwconv2d_fwd(FAKE, FAKE, None, FAKE + 4096, *_geo(oc=4), 0, None) == -3
    assert L.dwconv2d_fwd(FAKE, FAKE, None, FAKE + 4096, *_geo(ih=1, ph=0), 0, None) == -2


@no_gpu
def test_bwd_input_validation():
    L = N.lib()
    g = _geo()
    assert L.dwconv2d_bwd_input(FAKE, FAKE, FAKE + 4096, *g, 3, None) == -4
    assert L.dwconv2d_bwd_input(None, FAKE, FAKE + 4096, *g, 0, None) == -1
    assert L.dwconv2d_bwd_input(FAKE, FAKE, FAKE, *g, 0, None) == -7
    assert L.dwconv2d_bwd_input(FAKE, FAKE, FAKE + 4096, *_geo(n=-1), 0, None) == -2


@no_gpu
def test_bwd_weight_validation():
    L = N.lib()
    g = _geo()
    need = ctypes.c_size_t()
    assert L.dwconv2d_bwd_weight_workspace_bytes(*g, 0, ctypes.byref(need)) == 0
    assert need.value > 0
    ws = FAKE + (1 << 20)
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, None, ws, need.value, *g, 9, None) == -4
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, None, None, ws, need.value, *g, 0, None) == -1
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, None, None, need.value, *g, 0, None) == -5
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, None, ws, need.value - 1, *g, 0, None) == -5
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, None, ws + 4, need.value, *g, 0, None) == -5
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE, None, ws, need.value, *g, 0, None) == -7
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, FAKE + 8192, ws, need.value, *g, 0, None) == -7
    assert L.dwconv2d_bwd_weight(FAKE, FAKE, FAKE + 8192, None, FAKE, need.value, *g, 0, None) == -7


def test_workspace_bytes_positive_and_valid(orc):
    L = N.lib()
    for g in (_geo(), _geo(n=128, ic=32, ih=112, iw=112, oc=32), _geo(n=64, ic=384, ih=64, iw=64, oc=384,
                                                                      kh=31, kw=31, ph=15, pw=15),
              _geo(n=128, ic=256, ih=56, iw=56, oc=512, kh=5, kw=5, sh=2, sw=2, ph=4, pw=4, dh=2, dw=2)):
        for dt in (0, 1, 2):
            need = ctypes.c_size_t()
            assert L.dwconv2d_bwd_weight_workspace_bytes(*g, dt, ctypes.byref(need)) == 0
            assert 0 < need.value < (64 << 20)
    assert L.dwconv2d_bwd_weight_workspace_bytes(*_geo(oc=4), 0, ctypes.byref(need)) == -3


@no_gpu
def test_dynconv_validation():
    L = N.lib()
    f3 = (ctypes.c_void_p * 3)(FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24))
    d3 = (ctypes.c_int32 * 3)(1, 3, 5)
    y = FAKE + (8 << 24)
    dyn = L.dynconv_multidil_fwd
    assert dyn(FAKE, f3, d3, 3, y, 1, 4, 8, 8, 3, 5, None) == -4
    assert dyn(FAKE, f3, d3, 3, y, 1, 4, 8, 8, 4, 0, None) == -9        # even k
    assert dyn(FAKE, f3, d3, 0, y, 1, 4, 8, 8, 3, 0, None) == -9        # nb = 0
    assert dyn(FAKE, f3, d3, 5, y, 1, 4, 8, 8, 3, 0, None) == -9        # nb > 4
    bad = (ctypes.c_int32 * 3)(1, 0, 5)
    assert dyn(FAKE, f3, bad, 3, y, 1, 4, 8, 8, 3, 0, None) == -9       # dilation 0
    assert dyn(None, f3, d3, 3, y, 1, 4, 8, 8, 3, 0, None) == -1
    fnull = (ctypes.c_void_p * 3)(FAKE + (1 << 24), None, FAKE + (3 << 24))
    assert dyn(FAKE, fnull, d3, 3, y, 1, 4, 8, 8, 3, 0, None) == -1
    assert dyn(FAKE, f3, d3, 3, FAKE, 1, 4, 8, 8, 3, 0, None) == -7     # y aliases x
    assert dyn(FAKE, f3, d3, 3, FAKE + (1 << 24), 1, 4, 8, 8, 3, 0, None) == -7  # y aliases a filter
    assert dyn(FAKE, f3, d3, 3, y, 0, 4, 8, 8, 3, 0, None) == -2


@no_gpu
def test_dynconv_bwd_validation():
    L = N.lib()
    f3 = (ctypes.c_void_p * 3)(FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24))
    d3 = (ctypes.c_int32 * 3)(1, 3, 5)
    dy = FAKE + (8 << 24)
    dx = FAKE + (9 << 24)
    g3 = (ctypes.c_void_p * 3)(FAKE + (10 << 24), FAKE + (11 << 24), FAKE + (12 << 24))
    bwd = L.dynconv_multidil_bwd
    geo = (1, 4, 8, 8, 3)
    assert bwd(FAKE, f3, dy, d3, 3, dx, g3, *geo, 5, None) == -4              # dtype
    assert bwd(FAKE, f3, dy, d3, 3, dx, g3, 1, 4, 8, 8, 2, 0, None) == -9     # even k
    assert bwd(FAKE, f3, dy, d3, 0, dx, g3, *geo, 0, None) == -9              # nb = 0
    bad = (ctypes.c_int32 * 3)(1, -3, 5)
    assert bwd(FAKE, f3, dy, bad, 3, dx, g3, *geo, 0, None) == -9             # dilation < 1
    assert bwd(FAKE, f3, None, d3, 3, dx, g3, *geo, 0, None) == -1            # null dy
    assert bwd(None, f3, dy, d3, 3, dx, g3, *geo, 0, None) == -1              # null x
    assert bwd(FAKE, f3, dy + 2, d3, 3, dx, g3, *geo, 0, None) == -1          # misaligned dy
    assert bwd(FAKE, f3, dy, d3, 3, dx + 1, g3, *geo, 1, None) == -1          # misaligned dx (f16)
    assert bwd(FAKE, f3, dy, d3, 3, FAKE, g3, *geo, 0, None) == -7            # dx aliases x
    assert bwd(FAKE, f3, dy, d3, 3, dy, g3, *geo, 0, None) == -7              # dx aliases dy
    assert bwd(FAKE, f3, dy, d3, 3, FAKE + (2 << 24), None, *geo, 0, None) == -7  # dx aliases a filter
    galias = (ctypes.c_void_p * 3)(FAKE + (10 << 24), FAKE + (10 << 24) + 64, FAKE + (12 << 24))
    assert bwd(FAKE, f3, dy, d3, 3, dx, galias, *geo, 0, None) == -7          # two filter gradients overlap
    gx = (ctypes.c_void_p * 3)(None, dx, None)
    assert bwd(FAKE, f3, dy, d3, 3, dx, gx, *geo, 0, None) == -7              # filter gradient aliases dx
    assert bwd(FAKE, f3, dy, d3, 3, dx, g3, 0, 4, 8, 8, 3, 0, None) == -2     # n = 0
    # nothing requested: validated, nothing launched (safe without a device)
    none3 = (ctypes.c_void_p * 3)(None, None, None)
    assert bwd(FAKE, f3, dy, d3, 3, None, None, *geo, 0, None) == 0
    assert bwd(FAKE, f3, dy, d3, 3, None, none3, *geo, 0, None) == 0


@no_gpu
def test_dynconv_into_validation():
    L = N.lib()
    f3 = (ctypes.c_void_p * 3)(FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24))
    d3 = (ctypes.c_int32 * 3)(1, 3, 5)
    y = FAKE + (8 << 24)
    into = L.dynconv_multidil_fwd_into
    geo = (1, 4, 8, 8, 3)
    assert into(FAKE, f3, d3, 3, y, 12, -1, *geo, 0, None) == -2       # negative offset
    assert into(FAKE, f3, d3, 3, y, 12, 1, *geo, 0, None) == -2        # offset + nb*c past the channels
    assert into(FAKE, f3, d3, 3, y, 0, 0, *geo, 0, None) == -2         # no channels
    assert into(FAKE, f3, d3, 3, None, 20, 4, *geo, 0, None) == -1     # null y
    assert into(FAKE, f3, d3, 3, y + 2, 20, 4, *geo, 0, None) == -1    # misaligned y
    assert into(FAKE, f3, d3, 3, FAKE - 4096, 20, 4, *geo, 0, None) == -7  # larger y reaches x
    assert into(FAKE, f3, d3, 3, y, 20, 4, *geo, 9, None) == -4        # dtype
    frm = L.dynconv_multidil_bwd_from
    dx = FAKE + (9 << 24)
    assert frm(FAKE, f3, y, 12, 1, d3, 3, dx, None, *geo, 0, None) == -2
    assert frm(FAKE, f3, y, 20, -2, d3, 3, dx, None, *geo, 0, None) == -2
    assert frm(FAKE, f3, None, 20, 4, d3, 3, dx, None, *geo, 0, None) == -1
    assert frm(FAKE, f3, y, 20, 4, d3, 3, y + 64, None, *geo, 0, None) == -7   # dx inside the larger dy
    assert frm(FAKE, f3, y, 20, 4, d3, 3, None, None, *geo, 0, None) == 0      # nothing requested


@pytest.mark.parametrize("pass_,geo,dtype,must", [
    (0, ((128, 128, 56, 56), (128, 3, 3), 1, 1, 1), torch.float32, {"rowwalk_3x3", "band_3x3_s1", "band_generic"}),
    (1, ((128, 128, 56, 56), (128, 3, 3), 2, 1, 1), torch.float32, {"rowwalk_3x3", "band_generic"}),
    (2, ((128, 1024, 7, 7), (1024, 3, 3), 2, 1, 1), torch.float32, {"channelgroup_small"}),
    (0, ((64, 384, 64, 64), (384, 31, 31), 1, 15, 1), torch.float16, {"largek_roll16", "largek_mfma", "largek_regtile"}),
    (1, ((64, 384, 48, 48), (384, 31, 31), 1, 15, 1), torch.bfloat16, {"largek_roll16", "largek_mfma", "largek_regtile"}),
    (2, ((64, 384, 64, 64), (384, 31, 31), 1, 15, 1), torch.bfloat16, {"largek_roll16", "largek_mfma", "largek_regtile"}),
    (2, ((64, 384, 48, 48), (384, 7, 7), 1, 3, 1), torch.float32, {"stream_7x7", "largek_regtile"}),
    (1, ((128, 256, 56, 56), (512, 5, 5), 2, 4, 2), torch.bfloat16, {"decimated_s2d2", "band_generic"}),
])
def test_algo_candidates_and_selection_table(pass_, geo, dtype, must):
    cands = N.dwconv2d_algo_candidates(pass_, *geo, dtype=dtype)
    assert must <= set(cands), cands
    default = N.dwconv2d_algo(pass_, *geo, dtype=dtype)
    assert default in cands
    try:
        for name in cands:
            N.dwconv2d_set_algo(pass_, *geo, dtype=dtype, algo=name)
            assert N.dwconv2d_algo(pass_, *geo, dtype=dtype) == name
        with pytest.raises(N.DwconvError):
            N.dwconv2d_set_algo(pass_, *geo, dtype=dtype, algo="no_such_family")
        # another dtype or pass of the same geometry is a different key
        other = 0 if pass_ else 1
        assert N.dwconv2d_algo(other, *geo, dtype=dtype) == N.dwconv2d_algo(other, *geo, dtype=dtype)
    finally:
        N.dwconv2d_set_algo(pass_, *geo, dtype=dtype, algo=None)
    assert N.dwconv2d_algo(pass_, *geo, dtype=dtype) == default


@pytest.mark.parametrize("pass_,geo,dtype,want", [
    (0, ((64, 384, 48, 48), (384, 13, 13), 1, 6, 1), torch.float16, "largek_roll16"),
    (1, ((64, 384, 64, 64), (384, 7, 7), 1, 3, 1), torch.bfloat16, "largek_roll16"),
    (0, ((64, 384, 32, 32), (384, 7, 7), 1, 3, 1), torch.bfloat16, "largek_roll16"),
    (1, ((8, 64, 16, 16), (64, 13, 13), 1, 6, 1), torch.float16, None),   # below 32 x 32: the tiles
    (0, ((8, 64, 100, 24), (64, 13, 13), 1, 6, 1), torch.float16, None),  # rows under 32 columns
    (0, ((64, 384, 48, 48), (384, 31, 31), 1, 15, 1), torch.float32, "largek_roll_f32"),
    (1, ((64, 384, 32, 32), (384, 31, 31), 1, 15, 1), torch.float32, "largek_roll_f32"),
    (1, ((8, 64, 16, 16), (64, 31, 31), 1, 15, 1), torch.float32, None),   # below 32 x 32
])
def test_default_row_streaming(pass_, geo, dtype, want):
    """16-bit 7 x 7 and 13 x 13, and fp32 31 x 31, stream input rows on planes of at least 32 x 32."""
    fam = "largek_roll16" if dtype != torch.float32 else "largek_roll_f32"
    default = N.dwconv2d_algo(pass_, *geo, dtype=dtype)
    if want:
        assert default == want
    else:
        assert default != fam
        assert fam in N.dwconv2d_algo_candidates(pass_, *geo, dtype=dtype)


def test_algo_candidates_validation():
    L = N.lib()
    names = (ctypes.c_char_p * 4)()
    g = _geo()
    assert L.dwconv2d_algo_candidates(3, *g, 0, names, 4) == -2       # no such pass
    assert L.dwconv2d_algo_candidates(0, *g, 7, names, 4) == -4       # dtype
    assert L.dwconv2d_algo_candidates(0, *g, 0, None, 4) == -1        # names needed when cap > 0
    cnt = L.dwconv2d_algo_candidates(0, *g, 0, None, 0)               # count only
    assert cnt >= 1 and L.dwconv2d_algo_candidates(0, *g, 0, names, 1) == cnt
    assert L.dwconv2d_algo_candidates(0, *_geo(oc=4), 0, names, 4) == -3
    assert L.dwconv2d_set_algo(0, *g, 0, b"band_generic") == 0
    assert L.dwconv2d_set_algo(0, *g, 0, None) == 0
    assert L.dwconv2d_set_algo(0, *g, 0, b"largek_mfma") == -10        # cannot run a 3x3 fp32 layer


def test_workspace_covers_every_candidate():
    import torch as T
    for geo, dt in ((((64, 384, 64, 64), (384, 31, 31), 1, 15, 1), T.float16),
                    (((128, 32, 112, 112), (32, 3, 3), 1, 1, 1), T.float32)):
        need = N.dwconv2d_bwd_weight_workspace_bytes(*geo, dt)
        try:
            for name in N.dwconv2d_algo_candidates(2, *geo, dtype=dt):
                N.dwconv2d_set_algo(2, *geo, dtype=dt, algo=name)
                assert N.dwconv2d_bwd_weight_workspace_bytes(*geo, dt) == need
        finally:
            N.dwconv2d_set_algo(2, *geo, dtype=dt, algo=None)

def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 2, 5, 5)
    w = torch.zeros(2, 3, 3)
    with pytest.raises(ValueError, match="GPU tensor"):
        N.dwconv2d_fwd(x, w, None, 1, 1, 1)


def test_binding_checks_caller_buffers():
    """Caller-supplied outputs, bias and workspace must match the geometry, dtype and device
    before any pointer reaches the library (which writes that many elements of that type)."""
    x = torch.zeros(1, 2, 5, 5)
    w = torch.zeros(2, 3, 3)
    dy = torch.zeros(1, 2, 5, 5)
    with pytest.raises(ValueError, match="bias has shape"):
        N.dwconv2d_fwd(x, w, torch.zeros(3), 1, 1, 1)
    with pytest.raises(TypeError, match="bias dtype"):
        N.dwconv2d_fwd(x, w, torch.zeros(2, dtype=torch.float16), 1, 1, 1)
    with pytest.raises(ValueError, match="out has shape"):
        N.dwconv2d_fwd(x, w, None, 1, 1, 1, out=torch.zeros(1, 2, 4, 5))
    with pytest.raises(ValueError, match="out has shape"):
        N.dwconv2d_bwd_input(dy, w, x.shape, 1, 1, 1, out=torch.zeros(1, 2, 5, 4))
    with pytest.raises(ValueError, match="dy has shape"):
        N.dwconv2d_bwd_input(torch.zeros(1, 2, 4, 4), w, x.shape, 1, 1, 1)
    with pytest.raises(ValueError, match="out has shape"):
        N.dwconv2d_bwd_weight(x, dy, w.shape, 1, 1, 1, out=torch.zeros(2, 3, 2))
    with pytest.raises(TypeError, match="out dtype"):
        N.dwconv2d_bwd_weight(x, dy, w.shape, 1, 1, 1, out=torch.zeros(2, 3, 3, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out_bias has shape"):
        N.dwconv2d_bwd_weight(x, dy, w.shape, 1, 1, 1, out=torch.zeros(2, 3, 3), out_bias=torch.zeros(1))
    with pytest.raises(TypeError, match="out_bias dtype"):
        N.dwconv2d_bwd_weight(x, dy, w.shape, 1, 1, 1, out=torch.zeros(2, 3, 3),
                              out_bias=torch.zeros(2, dtype=torch.float16))
    with pytest.raises(ValueError, match="dy has shape"):
        N.dwconv2d_bwd_weight(x, torch.zeros(1, 2, 5, 6), w.shape, 1, 1, 1)
    with pytest.raises(ValueError, match="dy has shape"):
        N.dwconv2d_tune_bwd_weight(x, torch.zeros(1, 2, 5, 6), w.shape, 1, 1, 1)
    with pytest.raises(ValueError, match="bias has shape"):
        N.dwconv2d_tune_fwd(x, w, torch.zeros(5), 1, 1, 1)


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16])
def test_every_valid_geometry_has_a_family(dt):
    """No valid geometry is refused: each pass names a kernel family (direct kernels take rows
    too wide for any family's LDS staging) and the grad-weight workspace is positive."""
    import itertools
    import random
    rng = random.Random(7)
    geos = [((1, 4, 64, 600), (4, 31, 31), 1, 15, 1), ((1, 4, 512, 512), (4, 31, 31), 1, 15, 1),
            ((1, 4, 8, 8192), (4, 3, 3), 1, 1, 1), ((1, 1, 4, 16384), (1, 3, 3), 1, 1, 1),
            ((1, 1, 4, 16400), (1, 3, 3), 1, 1, 1), ((1, 2, 24, 600), (2, 31, 31), 1, 15, 1),
            ((1, 1, 520, 520), (1, 31, 31), 1, 15, 1), ((2, 3, 3, 20000), (6, 5, 5), (1, 2), (2, 4), (1, 3))]
    for _ in range(300):
        k = rng.choice([1, 2, 3, 5, 7, 9, 13, 31])
        s = rng.choice([1, 2, 3])
        d = rng.choice([1, 2, 3])
        p = rng.randint(0, k)
        h = rng.randint(1, 300)
        w = rng.choice([rng.randint(1, 300), rng.randint(1000, 30000)])
        m = rng.choice([1, 2, 3])
        c = rng.randint(1, 8)
        geos.append(((rng.randint(1, 3), c, h, w), (c * m, k, k), s, p, d))
    checked = 0
    for geo in geos:
        try:
            N.dwconv2d_out_size(*geo)
        except N.DwconvError:
            continue
        for pass_ in (0, 1, 2):
            assert N.dwconv2d_algo(pass_, *geo, dtype=dt), (pass_, geo)
        assert N.dwconv2d_bwd_weight_workspace_bytes(*geo, dt) > 0
        checked += 1
    assert checked > 100
    for geo in geos[:7]:
        assert "direct" in {N.dwconv2d_algo(p_, *geo, dtype=dt) for p_ in (0, 1, 2)} or geo[1][1] == 31


def test_bwd_weight_noalloc_validation():
    """The allocation-free grad-weight validates like dwconv2d_bwd_weight, and
    refuses geometries whose partial sums exceed its fixed device scratch
    before any HIP call."""
    L = N.lib()
    g = _geo()
    f = L.dwconv2d_bwd_weight_noalloc
    assert f(FAKE, FAKE, FAKE + 8192, None, *g, 9, None) == -4                  # dtype
    assert f(FAKE, FAKE, None, None, *g, 0, None) == -1                         # no dw
    assert f(FAKE, FAKE, FAKE + 8194, None, *g, 0, None) == -1                  # misaligned dw
    assert f(FAKE, FAKE, FAKE, None, *g, 0, None) == -7                         # dw inside x
    assert f(FAKE, FAKE, FAKE + 8192, FAKE + 8192, *g, 0, None) == -7           # db inside dw
    assert f(FAKE, FAKE, FAKE + 8192, None, *_geo(oc=4), 0, None) == -3         # multiplier
    assert f(FAKE, FAKE, FAKE + 8192, None, *_geo(ph=-1), 0, None) == -2        # geometry
    # multiplier 8 at 31 x 31 over 2048 channels: some 60 MiB of partial sums
    big = _geo(n=1, ic=2048, ih=8, iw=8, oc=16384, kh=31, kw=31, ph=15, pw=15)
    need = ctypes.c_size_t()
    assert L.dwconv2d_bwd_weight_workspace_bytes(*big, 0, ctypes.byref(need)) == 0
    assert need.value > N.NOALLOC_SCRATCH_BYTES
    dwp = FAKE + (1 << 30)
    assert f(FAKE, FAKE + (1 << 29), dwp, None, *big, 0, None) == -11
    assert "scratch" in N.status_str(-11)
    hdr = open(HEADER).read()
    m = re.search(r"#define DWCONV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == N.NOALLOC_SCRATCH_BYTES
