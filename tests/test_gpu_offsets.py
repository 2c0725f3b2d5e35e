"""Tensors that start at an element offset inside a larger allocation.

The ABI asks only for element alignment.  The kernels take their 16-byte
vector paths when every pointer of a call is 16-byte aligned and fall back to
element or narrower accesses otherwise; these tests put every input and output
of a call one (or three) elements past a 16-byte boundary and compare with the
oracle, for a geometry of each kernel family, and check that nothing outside
the views is written."""
import pytest
import torch

import dynamic_convolution_amd as dc
from dynamic_convolution_amd import synth
from oracle import oracle as O
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = synth.DTYPES
GUARD = 1024.0  # exactly representable in every I/O dtype


def note(msg):
    print("[case] " + msg, flush=True)


def at_offset(t, off):
    """(buffer, view): a device copy of t starting `off` elements into a buffer whose
    other elements hold GUARD."""
    n = t.numel()
    buf = torch.full((n + off + 8,), GUARD, dtype=t.dtype, device=DEV)
    v = buf[off:off + n].view(t.shape)
    v.copy_(t.to(DEV))
    return buf, v


def out_at_offset(shape, dtype, off):
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + off + 8,), GUARD, dtype=dtype, device=DEV)
    v = buf[off:off + n].view(shape)
    v.fill_(float("nan"))
    return buf, v


def assert_guards(buf, off, n, what):
    assert torch.all(buf[:off] == GUARD) and torch.all(buf[off + n:] == GUARD), what + ": written outside its view"


STATIC = [
    # n, c, h, w, M, k, s, p, d, dtype            family the geometry selects
    (2, 4, 60, 60, 1, 3, 1, 1, 1, "f32"),         # row-walk 3x3 stride 1
    (2, 4, 60, 64, 1, 3, 2, 1, 1, "bf16"),        # row-walk 3x3 stride 2
    (2, 3, 24, 40, 2, 5, 2, 4, 2, "bf16"),        # even grid (stride 2, dilation 2, pad k-1)
    (2, 3, 20, 22, 1, 5, 1, 2, 1, "f32"),         # band kernels
    (4, 40, 7, 7, 1, 3, 1, 1, 1, "f32"),          # small-plane channel groups
    (4, 40, 14, 14, 1, 3, 2, 1, 1, "f16"),        # small-plane channel groups, stride 2
    (1, 2, 40, 40, 1, 13, 1, 6, 1, "f32"),        # large-kernel register tiles
    (2, 2, 32, 32, 1, 31, 1, 15, 1, "f16"),       # large kernels on the matrix cores
    (2, 2, 32, 36, 1, 31, 1, 15, 1, "f32"),       # 31 x 31 fp32 on the matrix cores (input-row stream)
    (2, 2, 40, 40, 1, 13, 1, 6, 1, "bf16"),       # 16-bit 13 x 13 input-row stream (and its grad-weight)
    (2, 2, 33, 34, 1, 7, 1, 3, 1, "f16"),         # 16-bit 7 x 7 input-row stream
]


@pytest.mark.parametrize("off", [1, 3])
@pytest.mark.parametrize("case", STATIC)
def test_static_passes_at_element_offsets(case, off):
    n, c, h, w, M, k, s, p, d, dts = case
    dt = DT[dts]
    seed = 1300 + sum(case[:9]) + off
    x = synth.draw((n, c, h, w), ("U", -1.0, 1.0), seed, "x", dt)
    wt = synth.draw((c * M, k, k), ("N", 0.0, 1.0 / (k * k)), seed, "w", dt)
    b = synth.draw((c * M,), ("U", -0.1, 0.1), seed, "b", dt)
    oh, ow = dc.dwconv2d_out_size(x.shape, wt.shape, s, p, d)
    dy = synth.draw((n, c * M, oh, ow), ("N", 0.0, 1.0), seed, "dy", dt)
    tag = "offset %d: %s" % (off, case)
    _, xv = at_offset(x, off)
    _, wv = at_offset(wt, off)
    _, bv = at_offset(b, off)
    _, dyv = at_offset(dy, off)
    note(tag + " fwd")
    ybuf, y = out_at_offset((n, c * M, oh, ow), dt, off)
    dc.dwconv2d_fwd(xv, wv, bv, s, p, d, out=y)
    note(tag + " bwd_input")
    dxbuf, dx = out_at_offset(x.shape, dt, off)
    dc.dwconv2d_bwd_input(dyv, wv, x.shape, s, p, d, out=dx)
    note(tag + " bwd_weight")
    gwbuf, gw = out_at_offset(wt.shape, dt, off)
    gbbuf, gb = out_at_offset((c * M,), dt, off)
    wsbuf = torch.empty((dc.dwconv2d_bwd_weight_workspace_bytes(x.shape, wt.shape, s, p, d, dt) + 64,),
                        dtype=torch.uint8, device=DEV)
    dc.dwconv2d_bwd_weight(xv, dyv, wt.shape, s, p, d, out=gw, out_bias=gb, workspace=wsbuf[16:])
    torch.cuda.synchronize()
    assert_close(y, O.dwconv2d_fwd(x, wt, b, s, p, d), k * k, dt, tag + " fwd")
    assert_close(dx, O.dwconv2d_bwd_input(dy, wt, x.shape, s, p, d), M * k * k, dt, tag + " bwd_input")
    ow_, ob_ = O.dwconv2d_bwd_weight(x, dy, wt.shape, s, p, d)
    assert_close(gw, ow_, n * oh * ow, dt, tag + " bwd_weight")
    assert_close(gb, ob_, n * oh * ow, dt, tag + " bwd_bias")
    for buf, v, what in ((ybuf, y, "y"), (dxbuf, dx, "dx"), (gwbuf, gw, "dw"), (gbbuf, gb, "db")):
        assert_guards(buf, off, v.numel(), tag + " " + what)


@pytest.mark.parametrize("off", [1, 3])
@pytest.mark.parametrize("dts", ["f32", "bf16"])
def test_dynamic_at_element_offsets(dts, off):
    dt = DT[dts]
    n, c, h, w, k, dils = 1, 3, 21, 24, 3, (1, 3, 5)
    seed = 1400 + off
    x = synth.draw((n, c, h, w), ("N", 0.0, 1.0), seed, "x", dt)
    fs = [synth.draw((n, c, k * k, h, w), ("N", 0.0, 1.0 / 9), seed, "f%d" % i, dt) for i in range(3)]
    dy = synth.draw((n, 3 * c, h, w), ("N", 0.0, 1.0), seed, "dy", dt)
    tag = "dynamic offset %d %s" % (off, dts)
    _, xv = at_offset(x, off)
    fvs = [at_offset(f, off)[1] for f in fs]
    _, dyv = at_offset(dy, off)
    note(tag + " fwd")
    ybuf, y = out_at_offset((n, 3 * c, h, w), dt, off)
    dc.dynconv_multidil_fwd(xv, fvs, dils, out=y)
    note(tag + " bwd")
    dxbuf, dx = out_at_offset(x.shape, dt, off)
    dfb = [out_at_offset(f.shape, dt, off) for f in fs]
    dc.dynconv_multidil_bwd(xv, fvs, dyv, dils, out_dx=dx, out_dfilters=[v for _b, v in dfb])
    torch.cuda.synchronize()
    assert_close(y, O.dynconv_multidil_fwd(x, fs, dils), k * k, dt, tag + " fwd")
    odx, odf = O.dynconv_multidil_bwd(x, fs, dy, dils)
    assert_close(dx, odx, 3 * k * k, dt, tag + " dx")
    for i, ((_b, g), o) in enumerate(zip(dfb, odf)):
        assert_close(g, o, 1, dt, tag + " dF%d" % i)
    assert_guards(ybuf, off, y.numel(), tag + " y")
    assert_guards(dxbuf, off, dx.numel(), tag + " dx")
    for i, (bf, v) in enumerate(dfb):
        assert_guards(bf, off, v.numel(), tag + " dF%d" % i)


def test_strided_views_are_refused():
    x = torch.randn(2, 3, 16, 16, device=DEV)
    w = torch.randn(3, 3, 3, device=DEV)
    with pytest.raises(ValueError, match="contiguous"):
        dc.dwconv2d_fwd(x.transpose(2, 3), w, None, 1, 1, 1)
    y = torch.empty(2, 3, 16, 32, device=DEV)[..., ::2]
    with pytest.raises(ValueError, match="contiguous"):
        dc.dwconv2d_fwd(x, w, None, 1, 1, 1, out=y)
    fs = [torch.randn(2, 3, 9, 16, 16, device=DEV) for _ in range(3)]
    with pytest.raises(ValueError, match="contiguous"):
        dc.dynconv_multidil_fwd(x, [fs[0], fs[1].transpose(3, 4), fs[2]], (1, 3, 5))
