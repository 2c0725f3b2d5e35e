"""HIP path vs the CPU oracle, element by element, through the C ABI.

Inputs come from dynamic_convolution_amd.synth (seeded); the oracle sees the
exact fp64 upcast of the same tensors the kernels read.  Sizes are small
enough for the oracle to finish in seconds while spanning several workgroup
tiles and ragged tails; the full-size workloads are checked on sampled planes
and channels in the same launch configuration the benchmark times.
"""
import math
import random
import sys

import numpy as np
import pytest
import torch

import dynamic_convolution_amd as dc
from dynamic_convolution_amd import synth
from oracle import oracle as O
from tolerance import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = synth.DTYPES


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def _ks(k):
    return k if isinstance(k, tuple) else (k, k)


def static_case(n, ic, h, w, mult, k, s, p, d, dtype, seed, dists=None, bias=True):
    kh, kw = _ks(k)
    dists = dists or dict(x=("U", -1.0, 1.0), w=("N", 0.0, 1.0 / (kh * kw)), b=("U", -0.1, 0.1),
                          dy=("N", 0.0, 1.0))
    x = synth.draw((n, ic, h, w), dists["x"], seed, "x", dtype)
    wt = synth.draw((ic * mult, kh, kw), dists["w"], seed, "w", dtype)
    b = synth.draw((ic * mult,), dists["b"], seed, "b", dtype) if bias else None
    oh, ow = dc.dwconv2d_out_size(x.shape, wt.shape, s, p, d)
    assert (oh, ow) == (O.out_size(h, kh, _ks(s)[0], _ks(p)[0], _ks(d)[0]),
                        O.out_size(w, kw, _ks(s)[1], _ks(p)[1], _ks(d)[1]))
    dy = synth.draw((n, ic * mult, oh, ow), dists["dy"], seed, "dy", dtype)
    return x, wt, b, dy


def check_static(x, wt, b, dy, s, p, d, tag, passes=("fwd", "bwd_in", "bwd_w")):
    dtype = x.dtype
    n, ic, h, w = x.shape
    oc, kh, kw = wt.shape
    M = oc // ic
    oh, ow = dy.shape[2:]
    xd, wd, dyd = x.to(DEV), wt.to(DEV), dy.to(DEV)
    bd = b.to(DEV) if b is not None else None
    worst = {}
    if "fwd" in passes:
        note(tag + " fwd")
        y = dc.dwconv2d_fwd(xd, wd, bd, s, p, d)
        torch.cuda.synchronize()
        worst["fwd"] = assert_close(y, O.dwconv2d_fwd(x, wt, b, s, p, d), kh * kw, dtype, tag + " fwd")
    if "bwd_in" in passes:
        note(tag + " bwd_input")
        dx = dc.dwconv2d_bwd_input(dyd, wd, x.shape, s, p, d)
        torch.cuda.synchronize()
        worst["bwd_in"] = assert_close(dx, O.dwconv2d_bwd_input(dy, wt, x.shape, s, p, d), M * kh * kw,
                                       dtype, tag + " bwd_input")
    if "bwd_w" in passes:
        note(tag + " bwd_weight")
        gw, gb = dc.dwconv2d_bwd_weight(xd, dyd, wt.shape, s, p, d, with_bias=True)
        torch.cuda.synchronize()
        ow_, ob_ = O.dwconv2d_bwd_weight(x, dy, wt.shape, s, p, d)
        worst["bwd_w"] = assert_close(gw, ow_, n * oh * ow, dtype, tag + " bwd_weight")
        worst["bwd_b"] = assert_close(gb, ob_, n * oh * ow, dtype, tag + " bwd_bias")
    return worst


# ------------------------------------------------------------------ workloads
def test_tiny_workload():
    t = synth.TINY
    x, wt, b, dy = static_case(1, 8, 16, 16, 1, 3, 1, 1, 1, torch.float32, 1,
                               dists=dict(x=t["x"], w=t["w"], b=t["b"], dy=t["dy"]))
    check_static(x, wt, b, dy, 1, 1, 1, "tiny")


@pytest.mark.parametrize("stride", [1, 2])
@pytest.mark.parametrize("c,hw", synth.MOBILENET_LAYERS)
def test_mobilenet_layers(c, hw, stride):
    m = synth.MOBILENET
    n = 2 if c * hw * hw <= 200_000 else 1
    x, wt, b, dy = static_case(n, c, hw, hw, 1, 3, stride, 1, 1, torch.float32, 100 + c + stride,
                               dists=dict(x=m["x"], w=m["w"], b=("U", -0.1, 0.1), dy=m["dy"]))
    check_static(x, wt, None, dy, stride, 1, 1, "mobilenet C%d H%d s%d" % (c, hw, stride))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_mult_dil_workload(dtype):
    m = synth.MULT_DIL
    x, wt, b, dy = static_case(2, m["c"], m["h"], m["h"], m["mult"], m["k"], m["stride"], m["pad"], m["dil"],
                               DT[dtype], 200, dists=dict(x=m["x"], w=m["w"], b=("U", -0.1, 0.1), dy=m["dy"]))
    check_static(x, wt, b, dy, m["stride"], m["pad"], m["dil"], "multdil " + dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("k", [7, 13, 31])
@pytest.mark.parametrize("hw", [32, 48, 64])
def test_large_kernel(hw, k, dtype):
    L = synth.LARGE_K
    x, wt, b, dy = static_case(1, 4, hw, hw, 1, k, 1, k // 2, 1, DT[dtype], 300 + hw + k,
                               dists=dict(x=L["x"], w=("N", 0.0, 1.0 / k ** 2), b=("U", -0.1, 0.1), dy=L["dy"]))
    check_static(x, wt, b, dy, 1, k // 2, 1, "largek H%d k%d %s" % (hw, k, dtype))


def dyn_inputs(n, c, h, w, k, dils, dtype, seed, fdist=("N", 0.0, 1.0 / 9)):
    x = synth.draw((n, c, h, w), ("N", 0.0, 1.0), seed, "x", dtype)
    fs = [synth.draw((n, c, k * k, h, w), fdist, seed, "f%d" % i, dtype) for i in range(len(dils))]
    return x, fs


def check_dyn(x, fs, dils, tag):
    k = int(round(fs[0].shape[2] ** 0.5))
    note(tag)
    y = dc.dynconv_multidil_fwd(x.to(DEV), [f.to(DEV) for f in fs], dils)
    torch.cuda.synchronize()
    return assert_close(y, O.dynconv_multidil_fwd(x, fs, dils), k * k, x.dtype, tag)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,hw", [(1, 128), (2, 128), (1, 256)])
def test_dynamic_workload(n, hw, dtype):
    x, fs = dyn_inputs(n, 4, hw, hw, 3, (1, 3, 5), DT[dtype], 400 + n + hw)
    check_dyn(x, fs, (1, 3, 5), "dynamic N%d H%d %s" % (n, hw, dtype))


@pytest.mark.parametrize("shape,k,dils", [
    ((1, 3, 37, 53), 3, (1, 3, 5)),     # ragged rows, width not a vector multiple
    ((2, 2, 20, 16), 5, (1, 2)),        # k = 5
    ((1, 2, 9, 130), 3, (2, 4, 6, 8)),  # four branches, halo wider than the image height
    ((1, 1, 1, 1), 3, (1,)),            # single pixel
    ((1, 2, 12, 12), 1, (1, 7)),        # k = 1
    ((1, 2, 11, 14), 7, (3,)),          # runtime k
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dynamic_shapes(shape, k, dils, dtype):
    x, fs = dyn_inputs(*shape, k, dils, DT[dtype], 450 + sum(shape) + k, fdist=("N", 0.0, 1.0 / (k * k)))
    check_dyn(x, fs, dils, "dynamic %s k%d %s %s" % (shape, k, dils, dtype))



# ------------------------------------------------------------------ dynamic filter backward
def check_dyn_bwd(x, fs, dy, dils, tag, need_dx=True, need_df=True, df_mask=None):
    """dx and every requested dF_b against the oracle's chain rule; returns the device results."""
    k = int(round(fs[0].shape[2] ** 0.5))
    note(tag)
    xd, fsd, dyd = x.to(DEV), [f.to(DEV) for f in fs], dy.to(DEV)
    outs = None
    if need_df and df_mask is not None:
        outs = [torch.full_like(f, float("nan")) if m else None for f, m in zip(fsd, df_mask)]
    dx, dfs = dc.dynconv_multidil_bwd(xd, fsd, dyd, dils, need_dx=need_dx, need_dfilters=need_df,
                                      out_dfilters=outs)
    torch.cuda.synchronize()
    odx, odf = O.dynconv_multidil_bwd(x, fs, dy, dils)
    if need_dx:
        assert_close(dx, odx, len(dils) * k * k, x.dtype, tag + " dx")
    else:
        assert dx is None
    if need_df:
        for b, (g, o) in enumerate(zip(dfs, odf)):
            if g is not None:
                assert_close(g, o, 1, x.dtype, tag + " dF%d" % b)
    return dx, dfs


def dyn_bwd_inputs(n, c, h, w, k, dils, dtype, seed, fdist=("N", 0.0, 1.0 / 9)):
    x, fs = dyn_inputs(n, c, h, w, k, dils, dtype, seed, fdist)
    dy = synth.draw((n, len(dils) * c, h, w), ("N", 0.0, 1.0), seed, "dy", dtype)
    return x, fs, dy


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,hw", [(1, 128), (2, 128), (1, 256)])
def test_dynamic_bwd_workload(n, hw, dtype):
    x, fs, dy = dyn_bwd_inputs(n, 4, hw, hw, 3, (1, 3, 5), DT[dtype], 420 + n + hw)
    check_dyn_bwd(x, fs, dy, (1, 3, 5), "dynamic-bwd N%d H%d %s" % (n, hw, dtype))


@pytest.mark.parametrize("shape,k,dils", [
    ((1, 3, 37, 53), 3, (1, 3, 5)),     # ragged rows, width not a vector multiple: element paths
    ((2, 2, 20, 16), 5, (1, 2)),        # k = 5 register path
    ((2, 2, 13, 24), 5, (1, 3, 5)),     # k = 5, three branches, 16-bit strips of 8 fit 24
    ((1, 2, 9, 130), 3, (2, 4, 6, 8)),  # four branches, halo wider than the image height
    ((1, 1, 1, 1), 3, (1,)),            # single pixel
    ((1, 2, 12, 12), 1, (1, 7)),        # k = 1
    ((1, 2, 11, 14), 7, (3,)),          # runtime k
    ((1, 2, 24, 64), 3, (1, 3, 5)),     # several row bands on the register path
    ((1, 1, 40, 256), 3, (1, 3, 5)),    # one wave of strips per row
    ((3, 2, 17, 40), 3, (1, 3, 5)),     # partial last band
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dynamic_bwd_shapes(shape, k, dils, dtype):
    x, fs, dy = dyn_bwd_inputs(*shape, k, dils, DT[dtype], 470 + sum(shape) + k,
                               fdist=("N", 0.0, 1.0 / (k * k)))
    check_dyn_bwd(x, fs, dy, dils, "dynamic-bwd %s k%d %s %s" % (shape, k, dils, dtype))


@pytest.mark.parametrize("need_dx,need_df,mask", [
    (True, False, None), (False, True, None), (True, True, (True, False, True)), (False, True, (False, True, False)),
])
def test_dynamic_bwd_partial_requests(need_dx, need_df, mask):
    x, fs, dy = dyn_bwd_inputs(2, 3, 21, 32, 3, (1, 3, 5), torch.float32, 31)
    dx, dfs = check_dyn_bwd(x, fs, dy, (1, 3, 5), "dynamic-bwd partial %s %s %s" % (need_dx, need_df, mask),
                            need_dx, need_df, mask)
    if mask is not None:
        for g, m in zip(dfs, mask):
            assert (g is not None) == m


def test_dynamic_bwd_deterministic():
    x, fs, dy = dyn_bwd_inputs(2, 4, 64, 64, 3, (1, 3, 5), torch.float32, 37)
    xd, fsd, dyd = x.to(DEV), [f.to(DEV) for f in fs], dy.to(DEV)
    note("dynamic-bwd determinism")
    a = dc.dynconv_multidil_bwd(xd, fsd, dyd, (1, 3, 5))
    b = dc.dynconv_multidil_bwd(xd, fsd, dyd, (1, 3, 5))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    for g1, g2 in zip(a[1], b[1]):
        assert torch.equal(g1, g2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dynamic_bwd_guard_bands(dtype):
    margin = 64
    n, c, h, w = 2, 3, 21, 24
    x, fs, dy = dyn_bwd_inputs(n, c, h, w, 3, (1, 3, 5), DT[dtype], 41)
    dxbuf, dx = _guarded((n, c, h, w), DT[dtype])
    gb = [_guarded((n, c, 9, h, w), DT[dtype]) for _ in range(3)]
    note("dynamic-bwd guard " + dtype)
    dc.dynconv_multidil_bwd(x.to(DEV), [f.to(DEV) for f in fs], dy.to(DEV), (1, 3, 5), out_dx=dx,
                            out_dfilters=[t for _, t in gb])
    torch.cuda.synchronize()
    for buf, t in [(dxbuf, dx)] + gb:
        assert torch.isfinite(t).all(), "unwritten output element"
        assert torch.all(buf[:margin] == 1024.0) and torch.all(buf[-margin:] == -2048.0), "guard band written"


@pytest.mark.parametrize("shape,k,dils,off,extra,dtype", [
    ((2, 3, 21, 24), 3, (1, 3, 5), 5, 2, "f32"),     # branches in the middle of a larger concatenation
    ((1, 4, 32, 32), 5, (1, 3, 5), 0, 3, "bf16"),    # k = 5, offset 0, channels after
    ((2, 2, 20, 16), 5, (1, 2), 7, 0, "f16"),        # k = 5, the last channels of the tensor
    ((1, 3, 37, 53), 3, (1, 3, 5), 4, 1, "bf16"),    # ragged rows
])
def test_dynamic_into_larger_concat(shape, k, dils, off, extra, dtype):
    n, c, h, w = shape
    nb = len(dils)
    ctot = off + nb * c + extra
    x, fs, dy = dyn_bwd_inputs(*shape, k, dils, DT[dtype], 520 + sum(shape) + k + off,
                               fdist=("N", 0.0, 1.0 / (k * k)))
    note("dynamic-into %s k%d off%d of %d %s" % (shape, k, off, ctot, dtype))
    xd, fsd = x.to(DEV), [f.to(DEV) for f in fs]
    y = torch.full((n, ctot, h, w), 777.0, dtype=DT[dtype], device=DEV)
    dc.dynconv_multidil_fwd_into(xd, fsd, y, off, dils)
    # the gradient of the larger tensor: this op's branches at the same channels
    gbig = torch.full((n, ctot, h, w), 555.0, dtype=DT[dtype], device=DEV)
    gbig[:, off:off + nb * c] = dy.to(DEV)
    dx, dfs = dc.dynconv_multidil_bwd_from(xd, fsd, gbig, off, dils)
    torch.cuda.synchronize()
    assert torch.all(y[:, :off] == 777.0) and torch.all(y[:, off + nb * c:] == 777.0), "channel outside the slice written"
    assert_close(y[:, off:off + nb * c], O.dynconv_multidil_fwd(x, fs, dils), k * k, DT[dtype], "dynamic-into y")
    odx, odf = O.dynconv_multidil_bwd(x, fs, dy, dils)
    assert_close(dx, odx, nb * k * k, DT[dtype], "dynamic-from dx")
    for b in range(nb):
        assert_close(dfs[b], odf[b], 1, DT[dtype], "dynamic-from dF%d" % b)
    # the plain entry points are the special case offset 0, channels nb*c: identical results
    y0 = dc.dynconv_multidil_fwd(xd, fsd, dils)
    dx0, dfs0 = dc.dynconv_multidil_bwd(xd, fsd, dy.to(DEV), dils)
    torch.cuda.synchronize()
    assert torch.equal(y0, y[:, off:off + nb * c]) and torch.equal(dx0, dx)
    for a_, b_ in zip(dfs0, dfs):
        assert torch.equal(a_, b_)


# ------------------------------------------------------------------ every kernel family a geometry can run
SELECT_CASES = [
    (2, 6, 20, 24, 1, 3, 1, 1, 1, "f32"),      # 3x3 stride 1: row-walk, band 3x3, band generic
    (2, 6, 28, 28, 1, 3, 2, 1, 1, "f32"),      # 3x3 stride 2
    (2, 3, 20, 22, 2, 5, 2, 4, 2, "bf16"),     # multiplier 2, dilation 2, stride 2: even grid and band kernels
    (1, 2, 40, 40, 1, 31, 1, 15, 1, "f16"),    # 31x31: matrix cores, register tiles, band kernels
    (3, 20, 7, 7, 1, 3, 1, 1, 1, "f32"),       # small planes: channel groups, row-walk, band
    (1, 2, 33, 36, 1, 13, 1, 6, 1, "bf16"),    # 13x13
]


@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d,dt", SELECT_CASES)
def test_every_candidate_family_matches_oracle(n, c, h, w, mult, k, s, p, d, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 1100 + h + w + k)
    geo = (x.shape, wt.shape, s, p, d)
    passes = {0: "fwd", 1: "bwd_in", 2: "bwd_w"}
    try:
        for pi, pname in passes.items():
            cands = dc.dwconv2d_algo_candidates(pi, *geo, dtype=DT[dt])
            assert len(cands) >= 1
            for name in cands:
                dc.dwconv2d_set_algo(pi, *geo, dtype=DT[dt], algo=name)
                check_static(x, wt, b, dy, s, p, d, "family %s %s n%d c%d %dx%d k%d s%d %s"
                             % (pname, name, n, c, h, w, k, s, dt), passes=(pname,))
            dc.dwconv2d_set_algo(pi, *geo, dtype=DT[dt], algo=None)
    finally:
        for pi in passes:
            dc.dwconv2d_set_algo(pi, *geo, dtype=DT[dt], algo=None)


@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d,dt", [SELECT_CASES[0], SELECT_CASES[3]])
def test_tuned_selection_is_used_and_correct(n, c, h, w, mult, k, s, p, d, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 1200 + h + k)
    xd, wd, bd, dyd = x.to(DEV), wt.to(DEV), b.to(DEV), dy.to(DEV)
    geo = (x.shape, wt.shape, s, p, d)
    note("tune n%d c%d %dx%d k%d %s" % (n, c, h, w, k, dt))
    try:
        got = [dc.dwconv2d_tune_fwd(xd, wd, bd, s, p, d, reps=3),
               dc.dwconv2d_tune_bwd_input(dyd, wd, x.shape, s, p, d, reps=3),
               dc.dwconv2d_tune_bwd_weight(xd, dyd, wt.shape, s, p, d, reps=3)]
        for pi, name in enumerate(got):
            assert name in dc.dwconv2d_algo_candidates(pi, *geo, dtype=DT[dt])
            assert dc.dwconv2d_algo(pi, *geo, dtype=DT[dt]) == name
        check_static(x, wt, b, dy, s, p, d, "tuned %s" % (got,))
    finally:
        for pi in range(3):
            dc.dwconv2d_set_algo(pi, *geo, dtype=DT[dt], algo=None)

def fuzz_cases(count=48, seed=2024):
    r = random.Random(seed)
    out = []
    while len(out) < count:
        kh = r.choice([1, 2, 3, 3, 4, 5, 5, 7, 9, 11, 31]) if len(out) % 6 else 3
        kw = kh if r.random() < 0.6 else r.choice([1, 2, 3, 5, 6, 7])
        sh, sw = r.randint(1, 3), r.randint(1, 3)
        dh, dw = r.randint(1, 5), r.randint(1, 5)
        ph, pw = r.randint(0, (kh - 1) * dh), r.randint(0, (kw - 1) * dw)
        h, w = r.randint(1, 41), r.randint(1, 41)
        if O.out_size(h, kh, sh, ph, dh) < 1 or O.out_size(w, kw, sw, pw, dw) < 1:
            continue
        n, ic, mult = r.randint(1, 3), r.randint(1, 5), r.randint(1, 3)
        out.append((n, ic, h, w, mult, (kh, kw), (sh, sw), (ph, pw), (dh, dw), r.choice(["f32", "f16", "bf16"])))
    return out


@pytest.mark.parametrize("case", fuzz_cases(), ids=lambda c: "n%d_c%d_%dx%d_m%d_k%s_s%s_p%s_d%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8], c[9]))
def test_fuzz_geometry(case):
    n, ic, h, w, mult, k, s, p, d, dt = case
    x, wt, b, dy = static_case(n, ic, h, w, mult, k, s, p, d, DT[dt], 500 + h * 41 + w)
    check_static(x, wt, b, dy, s, p, d, "fuzz %s" % (case,))


# ------------------------------------------------------------------ exact cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_delta_filter_exact(dtype):
    n, ic, h, w, M, k, s, p, d = 2, 3, 19, 23, 2, (3, 5), (2, 1), (1, 3), (1, 2)
    x = synth.draw((n, ic, h, w), ("N", 0.0, 1.0), 7, "x", DT[dtype])
    for i0, j0 in [(0, 0), (1, 2), (2, 4)]:
        wt = torch.zeros((ic * M, 3, 5), dtype=DT[dtype])
        wt[:, i0, j0] = 1
        note("delta %s %d %d" % (dtype, i0, j0))
        y = dc.dwconv2d_fwd(x.to(DEV), wt.to(DEV), None, s, p, d).cpu().double().numpy()
        want = O.dwconv2d_fwd(x, wt, None, s, p, d)
        assert np.array_equal(y, want)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_ones_count_and_bias_exact(dtype):
    n, ic, h, w, k, s, p, d = 1, 4, 40, 37, 31, 1, 15, 1
    x = torch.ones((n, ic, h, w), dtype=DT[dtype])
    wt = torch.ones((ic, k, k), dtype=DT[dtype])
    note("ones " + dtype)
    y = dc.dwconv2d_fwd(x.to(DEV), wt.to(DEV), None, s, p, d).cpu()
    want = torch.from_numpy(O.dwconv2d_fwd(x, wt, None, s, p, d)).to(DT[dtype])  # counts, rounded once
    assert torch.equal(y, want)
    b = synth.draw((ic,), ("U", -1.0, 1.0), 8, "b", DT[dtype])
    wr = synth.draw((ic, 3, 3), ("N", 0.0, 1.0), 8, "w", DT[dtype])
    y0 = dc.dwconv2d_fwd(torch.zeros((2, ic, 9, 9), dtype=DT[dtype], device=DEV), wr.to(DEV), b.to(DEV), 1, 1, 1)
    assert torch.equal(y0.cpu(), b.view(1, ic, 1, 1).expand(2, ic, 9, 9))


def test_structural_zero_rows_exact():
    m = synth.MULT_DIL
    x, wt, b, dy = static_case(1, 8, 30, 26, 2, 5, 2, 4, 2, torch.bfloat16, 9)
    note("structural zeros")
    dx = dc.dwconv2d_bwd_input(dy.to(DEV), wt.to(DEV), x.shape, 2, 4, 2).cpu()
    assert torch.all(dx[:, :, 1::2, :] == 0) and torch.all(dx[:, :, :, 1::2] == 0)
    assert torch.count_nonzero(dx[:, :, 0::2, 0::2]) > 0.9 * dx[:, :, 0::2, 0::2].numel()


def test_bwd_weight_deterministic():
    x, wt, b, dy = static_case(8, 16, 56, 56, 1, 3, 1, 1, 1, torch.float32, 11)
    xd, dyd = x.to(DEV), dy.to(DEV)
    outs = []
    for _ in range(3):
        gw, gb = dc.dwconv2d_bwd_weight(xd, dyd, wt.shape, 1, 1, 1)
        outs.append((gw.clone(), gb.clone()))
    torch.cuda.synchronize()
    for gw, gb in outs[1:]:
        assert torch.equal(gw, outs[0][0]) and torch.equal(gb, outs[0][1])


def _guarded(shape, dtype, margin=64):
    numel = int(np.prod(shape))
    buf = torch.full((numel + 2 * margin,), float("nan"), dtype=dtype, device=DEV)
    buf[:margin] = 1024.0   # exactly representable in every I/O dtype
    buf[margin + numel:] = -2048.0
    return buf, buf[margin:margin + numel].view(shape)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_and_poison(dtype):
    margin = 64
    n, ic, h, w, M, k, s, p, d = 3, 5, 29, 31, 2, 5, 2, 4, 2
    x, wt, b, dy = static_case(n, ic, h, w, M, k, s, p, d, DT[dtype], 12)
    oh, ow = dy.shape[2:]
    ybuf, y = _guarded((n, ic * M, oh, ow), DT[dtype])
    dxbuf, dx = _guarded((n, ic, h, w), DT[dtype])
    gwbuf, gw = _guarded((ic * M, k, k), DT[dtype])
    gbbuf, gb = _guarded((ic * M,), DT[dtype])
    note("guard " + dtype)
    dc.dwconv2d_fwd(x.to(DEV), wt.to(DEV), b.to(DEV), s, p, d, out=y)
    dc.dwconv2d_bwd_input(dy.to(DEV), wt.to(DEV), x.shape, s, p, d, out=dx)
    dc.dwconv2d_bwd_weight(x.to(DEV), dy.to(DEV), wt.shape, s, p, d, out=gw, out_bias=gb)
    xq, fs = dyn_inputs(2, 3, 21, 18, 3, (1, 3, 5), DT[dtype], 13)
    ydbuf, yd = _guarded((2, 9, 21, 18), DT[dtype])
    dc.dynconv_multidil_fwd(xq.to(DEV), [f.to(DEV) for f in fs], (1, 3, 5), out=yd)
    torch.cuda.synchronize()
    for buf, t in ((ybuf, y), (dxbuf, dx), (gwbuf, gw), (gbbuf, gb), (ydbuf, yd)):
        assert torch.isfinite(t).all(), "unwritten output element"
        assert torch.all(buf[:margin] == 1024.0) and torch.all(buf[-margin:] == -2048.0), "guard band written"


# ------------------------------------------------------------------ full-size workloads, sampled
def _sample_idx(count, k, seed):
    r = random.Random(seed)
    return sorted(set([0, count - 1] + [r.randrange(count) for _ in range(k)]))


def full_static_sampled(n, ic, hw, M, k, s, p, d, dtype, dists, seed, tag):
    gen = lambda shape, name: synth.draw(shape, dists[name], seed, name, dtype, device=DEV)
    x = gen((n, ic, hw, hw), "x")
    wt = gen((ic * M, k, k), "w")
    oh, ow = dc.dwconv2d_out_size(x.shape, wt.shape, s, p, d)
    dy = gen((n, ic * M, oh, ow), "dy")
    note(tag + " full-size launch")
    y = dc.dwconv2d_fwd(x, wt, None, s, p, d)
    dx = dc.dwconv2d_bwd_input(dy, wt, x.shape, s, p, d)
    gw, gb = dc.dwconv2d_bwd_weight(x, dy, wt.shape, s, p, d)
    torch.cuda.synchronize()
    wc = wt.cpu()
    for nn in _sample_idx(n, 2, seed):
        for g in _sample_idx(ic, 2, seed + 1):
            xs = x[nn:nn + 1, g:g + 1].cpu()
            ws = wc[g * M:(g + 1) * M]
            assert_close(y[nn:nn + 1, g * M:(g + 1) * M], O.dwconv2d_fwd(xs, ws, None, s, p, d), k * k, dtype,
                         tag + " fwd n%d g%d" % (nn, g))
            dys = dy[nn:nn + 1, g * M:(g + 1) * M].cpu()
            assert_close(dx[nn:nn + 1, g:g + 1], O.dwconv2d_bwd_input(dys, ws, xs.shape, s, p, d), M * k * k,
                         dtype, tag + " bwd_input n%d g%d" % (nn, g))
    for g in _sample_idx(ic, 1, seed + 2):
        ow_, ob_ = O.dwconv2d_bwd_weight(x[:, g:g + 1].cpu(), dy[:, g * M:(g + 1) * M].cpu(), (M, k, k), s, p, d)
        assert_close(gw[g * M:(g + 1) * M], ow_, n * oh * ow, dtype, tag + " bwd_weight g%d" % g)
        assert_close(gb[g * M:(g + 1) * M], ob_, n * oh * ow, dtype, tag + " bwd_bias g%d" % g)


@pytest.mark.parametrize("c,hw,s", [(32, 112, 1), (64, 112, 2), (1024, 7, 2), (512, 14, 1)])
def test_full_size_mobilenet_sampled(c, hw, s):
    m = synth.MOBILENET
    full_static_sampled(128, c, hw, 1, 3, s, 1, 1, torch.float32, dict(x=m["x"], w=m["w"], dy=m["dy"]),
                        700 + c + s, "mobilenet-full C%d H%d s%d" % (c, hw, s))


def test_full_size_mult_dil_sampled():
    m = synth.MULT_DIL
    full_static_sampled(m["n"], m["c"], m["h"], m["mult"], m["k"], m["stride"], m["pad"], m["dil"], torch.bfloat16,
                        dict(x=m["x"], w=m["w"], dy=m["dy"]), 800, "multdil-full")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_full_size_large_kernel_sampled(dtype):
    L = synth.LARGE_K
    full_static_sampled(L["n"], L["c"], 64, 1, 31, 1, 15, 1, DT[dtype],
                        dict(x=L["x"], w=("N", 0.0, 1.0 / 961), dy=L["dy"]), 900, "largek-full H64 k31 " + dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_size_dynamic_sampled(dtype):
    D = synth.DYNAMIC
    n, c, hw = 2, D["c"], 256
    x = synth.draw((n, c, hw, hw), D["x"], 950, "x", DT[dtype], device=DEV)
    fs = [synth.draw((n, c, 9, hw, hw), D["f"], 950, "f%d" % i, DT[dtype], device=DEV) for i in range(3)]
    note("dynamic-full " + dtype)
    y = dc.dynconv_multidil_fwd(x, fs, D["dilations"])
    torch.cuda.synchronize()
    for nn in range(n):
        for ch in _sample_idx(c, 3, 951):
            want = O.dynconv_multidil_fwd(x[nn:nn + 1, ch:ch + 1].cpu(),
                                          [f[nn:nn + 1, ch:ch + 1].cpu() for f in fs], D["dilations"])
            got = torch.stack([y[nn, b * c + ch] for b in range(3)]).unsqueeze(0)
            assert_close(got, want, 9, DT[dtype], "dynamic-full n%d c%d" % (nn, ch))



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_size_dynamic_bwd_sampled(dtype):
    D = synth.DYNAMIC
    n, c, hw = 2, D["c"], 256
    x = synth.draw((n, c, hw, hw), D["x"], 960, "x", DT[dtype], device=DEV)
    fs = [synth.draw((n, c, 9, hw, hw), D["f"], 960, "f%d" % i, DT[dtype], device=DEV) for i in range(3)]
    dy = synth.draw((n, 3 * c, hw, hw), D["dy"], 960, "dy", DT[dtype], device=DEV)
    note("dynamic-bwd-full " + dtype)
    dx, dfs = dc.dynconv_multidil_bwd(x, fs, dy, D["dilations"])
    torch.cuda.synchronize()
    for nn in range(n):
        for ch in _sample_idx(c, 3, 961):
            sl = lambda t: t[nn:nn + 1, ch:ch + 1].cpu()
            dys = torch.stack([dy[nn, b * c + ch] for b in range(3)]).unsqueeze(0).cpu()
            odx, odf = O.dynconv_multidil_bwd(sl(x), [sl(f) for f in fs], dys, D["dilations"])
            assert_close(dx[nn:nn + 1, ch:ch + 1], odx, 27, DT[dtype], "dynamic-bwd-full dx n%d c%d" % (nn, ch))
            for b in range(3):
                assert_close(dfs[b][nn:nn + 1, ch:ch + 1], odf[b], 1, DT[dtype],
                             "dynamic-bwd-full dF%d n%d c%d" % (b, nn, ch))

# ------------------------------------------------------------------ streaming 3x3 path edges
@pytest.mark.parametrize("n,c,h,w,mult,s,dt", [
    (2, 3, 9, 13, 1, 1, "f32"), (2, 3, 9, 13, 1, 2, "f32"),     # odd sizes, scalar loads
    (1, 4, 17, 256, 1, 1, "f32"),                               # 64 strips: widest row of one wave
    (1, 2, 10, 257, 1, 1, "f32"),                               # one column too wide: band kernels
    (1, 2, 12, 512, 1, 2, "f32"),                               # stride 2, 64 output strips
    (3, 5, 23, 40, 2, 1, "f32"), (3, 5, 23, 40, 2, 2, "f32"),   # multiplier 2
    (2, 3, 31, 64, 1, 1, "f16"), (2, 3, 31, 64, 2, 2, "bf16"),  # 16-bit strips of 8
    (1, 2, 6, 512, 1, 1, "bf16"), (1, 2, 5, 1030, 1, 2, "f16"),
    (4, 1, 1, 1, 1, 1, "f32"), (2, 2, 2, 3, 1, 2, "f32"),       # degenerate planes
    # rows whose byte length is not a multiple of 16: narrower clamped vector accesses
    (2, 3, 19, 58, 1, 1, "f32"), (2, 3, 19, 58, 1, 2, "f32"),   # 232-byte rows: 8-byte vectors
    (2, 2, 15, 57, 1, 1, "f32"), (2, 2, 15, 57, 2, 2, "f32"),   # 228-byte rows: 4-byte vectors
    (2, 3, 14, 58, 1, 1, "bf16"), (2, 3, 14, 60, 2, 1, "f16"),  # 116 / 120-byte rows
    (2, 2, 13, 57, 1, 1, "bf16"), (2, 2, 13, 57, 1, 2, "f16"),  # odd 16-bit rows: 2-byte vectors
    (3, 4, 14, 14, 1, 1, "f32"), (3, 4, 28, 28, 1, 2, "f32"),   # narrow planes (grad-input s2)
    (3, 4, 14, 14, 2, 2, "bf16"), (2, 3, 7, 7, 1, 1, "f32"),
])
def test_streaming_3x3_shapes(n, c, h, w, mult, s, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, 3, s, 1, 1, DT[dt], 600 + h * 7 + w)
    check_static(x, wt, b, dy, s, 1, 1, "stream3x3 n%d c%d %dx%d m%d s%d %s" % (n, c, h, w, mult, s, dt))


# ------------------------------------------------------------------ HIP graph replay
def test_graph_replay_matches_eager():
    """Every entry point captured in a HIP graph: each of several replays, with eager
    work and synchronisation in between, reproduces the eager result bitwise."""
    # streaming and band paths (fp32 3x3), and the 16-bit 31x31 matrix-core path
    cases = [(4, 8, 112, 112, 1, 3, 1, 1, torch.float32), (4, 8, 56, 56, 2, 3, 2, 1, torch.float32),
             (3, 5, 14, 14, 1, 3, 2, 1, torch.float32), (5, 2, 64, 64, 1, 31, 1, 15, torch.float16)]
    work = []
    for n, c, h, w, mult, k, s, p, dt in cases:
        x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, 1, dt, 17 + h + k)
        xd, wd, bd, dyd = x.to(DEV), wt.to(DEV), b.to(DEV), dy.to(DEV)
        y = torch.empty((n, c * mult) + tuple(dy.shape[2:]), device=DEV, dtype=dt)
        dx, gw, gb = torch.empty_like(xd), torch.empty_like(wd), torch.empty_like(bd)
        ws = torch.empty((dc.dwconv2d_bwd_weight_workspace_bytes(x.shape, wt.shape, s, p, 1, dt),),
                         dtype=torch.uint8, device=DEV)
        work.append(lambda xd=xd, wd=wd, bd=bd, dyd=dyd, y=y, dx=dx, gw=gw, gb=gb, ws=ws, s=s, p=p: (
            dc.dwconv2d_fwd(xd, wd, bd, s, p, 1, out=y),
            dc.dwconv2d_bwd_input(dyd, wd, xd.shape, s, p, 1, out=dx),
            dc.dwconv2d_bwd_weight(xd, dyd, wd.shape, s, p, 1, out=gw, out_bias=gb, workspace=ws)))
        work[-1].outs = (y, dx, gw, gb)
    xq, fs = dyn_inputs(1, 4, 64, 64, 3, (1, 3, 5), torch.float32, 19)
    xqd, fsd = xq.to(DEV), [f.to(DEV) for f in fs]
    gq = synth.draw((1, 12, 64, 64), ("N", 0.0, 1.0), 19, "dy", device=DEV)
    yq = torch.empty((1, 12, 64, 64), device=DEV)
    dxq = torch.empty_like(xqd)
    dfq = [torch.empty_like(f) for f in fsd]

    def dynf():
        dc.dynconv_multidil_fwd(xqd, fsd, (1, 3, 5), out=yq)
        dc.dynconv_multidil_bwd(xqd, fsd, gq, (1, 3, 5), out_dx=dxq, out_dfilters=dfq)
    dyn_outs = (yq, dxq) + tuple(dfq)
    note("graph eager")
    for fn in work:
        fn()
    dynf()
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in fn.outs) for fn in work] + [tuple(t.clone() for t in dyn_outs)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in work:
            fn()
        dynf()
    for rep in range(4):
        for fn in work:  # poison outputs eagerly between replays
            for t in fn.outs:
                t.fill_(float("nan"))
        for t in dyn_outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        note("graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = [fn.outs for fn in work] + [dyn_outs]
        for a_, b_ in zip(got, ref):
            for t1, t2 in zip(a_, b_):
                assert torch.equal(t1, t2), "replay %d differs from eager" % rep


@pytest.mark.parametrize("n,c,h,k,p,dt", [(5, 3, 64, 31, 15, "f16"), (4, 2, 48, 13, 6, "bf16"),
                                          (3, 2, 32, 7, 3, "f16")])
def test_large_kernel_matrix_core_deterministic(n, c, h, k, p, dt):
    """The matrix-core passes give bitwise identical results run to run."""
    x, wt, b, dy = static_case(n, c, h, h, 1, k, 1, p, 1, DT[dt], 1300 + h + k)
    xd, wd, bd, dyd = x.to(DEV), wt.to(DEV), b.to(DEV), dy.to(DEV)
    note("mfma determinism k%d %s" % (k, dt))
    runs = []
    for _ in range(3):
        y = dc.dwconv2d_fwd(xd, wd, bd, 1, p, 1)
        dx = dc.dwconv2d_bwd_input(dyd, wd, xd.shape, 1, p, 1)
        gw, gb = dc.dwconv2d_bwd_weight(xd, dyd, wd.shape, 1, p, 1)
        torch.cuda.synchronize()
        runs.append((y, dx, gw, gb))
    for r in runs[1:]:
        for t1, t2 in zip(runs[0], r):
            assert torch.equal(t1, t2)


# ------------------------------------------------------------------ large-kernel path edges
@pytest.mark.parametrize("n,c,h,w,mult,k,p,dt", [
    (2, 3, 37, 50, 1, 7, 3, "f32"),      # ragged sizes, column tile of 4
    (1, 2, 20, 70, 1, 13, 0, "f32"),     # no padding
    (1, 2, 40, 33, 1, 13, 12, "f32"),    # pad k-1: grad-input pad 0
    (1, 2, 64, 64, 2, 31, 15, "f32"),    # multiplier 2 (forward on the matrix cores, others fall back)
    (1, 3, 48, 48, 1, 31, 15, "bf16"),
    (2, 2, 9, 9, 1, 31, 15, "f16"),      # kernel wider than the image
    (1, 1, 130, 24, 1, 7, 3, "f32"),     # several row bands
    (1, 2, 100, 64, 1, 13, 6, "f16"),    # several grad-weight bands, 16-bit filter staged as fp32
])
def test_large_kernel_shapes(n, c, h, w, mult, k, p, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, k, 1, p, 1, DT[dt], 650 + h + w + k)
    check_static(x, wt, b, dy, 1, p, 1, "largek n%d c%d %dx%d m%d k%d p%d %s" % (n, c, h, w, mult, k, p, dt))



# ------------------------------------------------------------------ large kernels on the matrix cores (16-bit I/O)
@pytest.mark.parametrize("n,c,h,w,mult,k,p,dt,fwd_mfma,bin_mfma", [
    (5, 2, 64, 64, 1, 31, 15, "f16", True, True),     # 2 x 2 tiles, two images per workgroup: last group partial
    (3, 3, 48, 48, 1, 31, 15, "bf16", True, True),    # 48 x 48 in 2 x 2 tiles (masked stores)
    (6, 2, 32, 32, 1, 31, 15, "bf16", True, True),    # one tile, four images per workgroup: last group partial
    (2, 2, 64, 64, 2, 31, 15, "f16", True, False),    # multiplier 2: forward on the matrix cores
    (3, 2, 64, 40, 1, 13, 6, "f16", True, True),      # 2 x 2 tiles, ragged width (element staging and stores)
    (2, 3, 33, 36, 1, 13, 0, "bf16", True, True),     # no padding (forward output 21 x 24)
    (2, 2, 20, 22, 1, 13, 12, "f16", True, True),     # pad k - 1: grad-input pad 0
    (4, 2, 47, 47, 1, 7, 2, "bf16", True, True),      # k = 7, odd sizes
    (2, 2, 9, 9, 1, 31, 15, "f16", True, True),       # kernel wider than the image
    (1, 2, 100, 24, 1, 13, 6, "f16", False, False),   # more than 64 rows, under 32 columns: register-tile kernels
])
def test_large_kernel_mfma(n, c, h, w, mult, k, p, dt, fwd_mfma, bin_mfma):
    """The 32 x 32-tile family (at k = 7 on planes over 32 the 16 x 16 tiles are the default, so it is forced)."""
    geo = ((n, c, h, w), (c * mult, k, k), 1, p, 1)
    mfma = ("largek_mfma", "largek_mfma_h16", "largek_roll16")
    assert (dc.dwconv2d_algo(0, *geo, dtype=DT[dt]) in mfma) == fwd_mfma
    assert (dc.dwconv2d_algo(1, *geo, dtype=DT[dt]) in mfma) == bin_mfma
    x, wt, b, dy = static_case(n, c, h, w, mult, k, 1, p, 1, DT[dt], 680 + h + w + k)
    try:
        if fwd_mfma:
            dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo="largek_mfma")
        if bin_mfma:
            dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo="largek_mfma")
        check_static(x, wt, b, dy, 1, p, 1, "largek-mfma n%d c%d %dx%d m%d k%d p%d %s" % (n, c, h, w, mult, k, p, dt),
                     passes=("fwd", "bwd_in"))
    finally:
        dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo=None)
        dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo=None)


@pytest.mark.parametrize("n,c,h,w,k,p,dt", [
    (7, 2048, 16, 16, 7, 3, "f16"),    # four images a group, two groups a workgroup, the last one partial
    (7, 1200, 40, 40, 7, 3, "bf16"),   # 2 x 2 tiles, two images a group, two groups a workgroup
])
def test_large_kernel_mfma_group_chunks(n, c, h, w, k, p, dt):
    """Workgroups that walk several image groups load the next group's planes during the matrix work."""
    geo = ((n, c, h, w), (c, k, k), 1, p, 1)
    x, wt, b, dy = static_case(n, c, h, w, 1, k, 1, p, 1, DT[dt], 690 + h + w + k)
    try:
        for pass_ in (0, 1):
            dc.dwconv2d_set_algo(pass_, *geo, dtype=DT[dt], algo="largek_mfma")
        check_static(x, wt, b, dy, 1, p, 1, "largek-mfma-chunks n%d c%d %dx%d k%d %s" % (n, c, h, w, k, dt),
                     passes=("fwd", "bwd_in"))
    finally:
        for pass_ in (0, 1):
            dc.dwconv2d_set_algo(pass_, *geo, dtype=DT[dt], algo=None)


@pytest.mark.parametrize("n,c,h,w,k,p,dt,bw_mfma", [
    (5, 2, 64, 64, 31, 15, "f16", True),     # two 32-row bands, chunks of images
    (3, 3, 48, 48, 31, 15, "bf16", True),    # a full band and a partial band
    (6, 2, 32, 32, 31, 15, "f16", True),     # one band
    (3, 2, 64, 40, 13, 6, "bf16", True),     # ragged width: element staging
    (2, 3, 33, 36, 13, 0, "f16", True),      # no padding
    (2, 2, 20, 22, 13, 12, "bf16", True),    # pad k - 1
    (2, 2, 9, 9, 31, 15, "f16", True),       # kernel wider than the image
    (3, 2, 70, 40, 13, 6, "f16", True),      # 70 dy rows: three bands
    (2, 2, 47, 47, 7, 2, "bf16", False),     # k = 7: register tiles (the matrix cores measured slower)
    (3, 2, 64, 64, 7, 3, "f16", False),      # k = 7, 64 x 64
    (2, 2, 20, 18, 7, 6, "bf16", False),     # k = 7, pad k - 1
    (1, 2, 40, 100, 13, 6, "f16", False),    # rows of 100: register tiles
])
def test_large_kernel_mfma_grad_weight(n, c, h, w, k, p, dt, bw_mfma):
    """The 32 x 32-tile family (forced: the row-streaming family is the 16-bit default at k = 13 and 31)."""
    geo = ((n, c, h, w), (c, k, k), 1, p, 1)
    default = dc.dwconv2d_algo(2, *geo, dtype=DT[dt])
    if bw_mfma:
        assert default == "largek_roll16"
        assert "largek_mfma" in dc.dwconv2d_algo_candidates(2, *geo, dtype=DT[dt])
    else:
        assert default not in ("largek_mfma", "largek_roll16")
    x, wt, b, dy = static_case(n, c, h, w, 1, k, 1, p, 1, DT[dt], 690 + h + w + k)
    try:
        if bw_mfma:
            dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo="largek_mfma")
        check_static(x, wt, b, dy, 1, p, 1, "largek-mfma-bw n%d c%d %dx%d k%d p%d %s" % (n, c, h, w, k, p, dt),
                     passes=("bwd_w",))
    finally:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo=None)

# ------------------------------------------------------------------ stride 2 / dilation 2 / pad k-1 (even-grid) path
@pytest.mark.parametrize("n,c,h,w,mult,k,dt", [
    (2, 3, 29, 31, 2, 5, "bf16"), (2, 3, 29, 31, 1, 5, "f32"),   # odd sizes
    (1, 2, 20, 22, 1, 3, "f32"), (2, 2, 17, 9, 2, 3, "f16"),
    (1, 2, 6, 512, 2, 5, "bf16"),                                # 64 strips of decimated columns
    (1, 2, 6, 514, 1, 5, "f32"),                                 # one strip too many: band kernels
    (3, 1, 1, 1, 1, 3, "f32"), (1, 2, 2, 3, 2, 5, "f32"),        # tiny planes
    # width a multiple of 8: whole-vector loads and stores
    (2, 5, 24, 40, 2, 5, "bf16"), (3, 3, 15, 16, 1, 3, "f16"),   # odd height: last dx row has no zero row
    (2, 4, 16, 24, 2, 3, "f32"), (1, 2, 9, 8, 2, 5, "bf16"),
    (5, 7, 20, 56, 1, 5, "bf16"),                                # images x bands not a multiple of a wave's units
    # few planes of many rows: several row bands (band heights rounded to k or 2k rows)
    (1, 2, 120, 40, 2, 5, "bf16"), (1, 3, 90, 24, 1, 3, "f32"), (2, 2, 64, 32, 1, 5, "f16"),
])
def test_even_grid_shapes(n, c, h, w, mult, k, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, k, 2, k - 1, 2, DT[dt], 670 + h + w + k)
    check_static(x, wt, b, dy, 2, k - 1, 2, "evengrid n%d c%d %dx%d m%d k%d %s" % (n, c, h, w, mult, k, dt))


# ------------------------------------------------------------------ small planes (grad-weight by channel groups)
@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d,dt", [
    (6, 40, 7, 7, 1, 3, 1, 1, 1, "f32"),      # two channel groups, the second partial; two images per chunk
    (9, 1024, 7, 7, 1, 3, 1, 1, 1, "f32"),    # 7x7 MobileNet plane, three images per chunk
    (4, 512, 14, 14, 1, 3, 2, 1, 1, "f32"),   # 14x14 -> 7x7
    (5, 72, 14, 14, 1, 3, 2, 1, 1, "bf16"),   # group size cut to whole 16-byte vectors of both ranges
    (4, 24, 7, 7, 2, 3, 2, 1, 1, "f16"),      # 7x7 -> 4x4 with multiplier 2
    (3, 20, 7, 9, 1, 5, 1, 2, 1, "f32"),      # 5x5, rows of 9 outputs
    (4, 10, 11, 11, 1, 5, 2, 4, 2, "f32"),    # 5x5 stride 2 dilation 2; ranges not whole vectors
    (3, 9, 4, 16, 1, 3, 1, 1, 1, "bf16"),     # rows of 16 outputs
    (2, 7, 5, 5, 1, 3, 1, 1, 1, "f32"),       # element staging
    (5, 20, 14, 14, 1, 3, 1, 1, 1, "f32"),    # 14x14 outputs: rows of 14 in 16-wide windows
    (4, 12, 28, 28, 1, 3, 2, 1, 1, "bf16"),   # 28x28 -> 14x14
    (3, 8, 16, 16, 2, 5, 1, 2, 1, "f16"),     # 256 outputs per plane, multiplier 2, 5x5
])
def test_small_plane_shapes(n, c, h, w, mult, k, s, p, d, dt):
    assert dc.dwconv2d_algo(2, (n, c, h, w), (c * mult, k, k), s, p, d, dtype=DT[dt]) == "channelgroup_small"
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 900 + c + h * 3 + k)
    check_static(x, wt, b, dy, s, p, d, "smallplane n%d c%d %dx%d m%d k%d s%d %s" % (n, c, h, w, mult, k, s, dt),
                 passes=("bwd_w",))


# ------------------------------------------------------------------ small planes (forward and grad-input by channel groups)
@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d,dt,fwd_cg", [
    (6, 40, 7, 7, 1, 3, 1, 1, 1, "f32", True),       # two channel groups, the second partial
    (9, 1024, 7, 7, 1, 3, 2, 1, 1, "f32", True),     # 7x7 -> 4x4, odd padding at stride 2
    (4, 512, 14, 14, 1, 3, 2, 1, 1, "f32", True),    # 14x14 -> 7x7
    (5, 72, 14, 14, 1, 3, 1, 1, 1, "bf16", True),    # group size cut to whole 16-byte vectors
    (4, 24, 28, 28, 1, 3, 2, 1, 1, "f16", False),    # dx rows of 28 in 32-wide windows (grad-input only)
    (3, 20, 7, 9, 2, 5, 1, 2, 1, "f32", True),       # 5x5, multiplier 2
    (4, 10, 11, 11, 1, 5, 2, 2, 2, "f32", True),     # 5x5 stride 2 dilation 2, even padding; element staging
    (3, 9, 12, 16, 1, 3, 2, 0, 1, "bf16", True),     # stride 2 without padding
    (2, 7, 5, 5, 2, 3, 1, 1, 1, "f16", True),        # element staging, multiplier 2
    (3, 6, 20, 30, 1, 5, 2, 3, 2, "f32", False),     # 5x5 stride 2 dilation 2, odd padding, dx rows of 30
    (2, 3, 13, 15, 2, 3, 1, 1, 1, "f32", True),      # rows of 15 in 16-wide windows, multiplier 2
    (2, 5, 8, 32, 1, 3, 1, 1, 1, "bf16", False),     # stride 1, dx rows of 32
])
def test_small_plane_fwd_bwd_input(n, c, h, w, mult, k, s, p, d, dt, fwd_cg):
    geo = ((n, c, h, w), (c * mult, k, k), s, p, d)
    assert dc.dwconv2d_algo(1, *geo, dtype=DT[dt]) == "channelgroup_small"
    assert (dc.dwconv2d_algo(0, *geo, dtype=DT[dt]) == "channelgroup_small") == fwd_cg
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 950 + c + h * 3 + k + s)
    check_static(x, wt, b, dy, s, p, d, "smallplane-fb n%d c%d %dx%d m%d k%d s%d p%d %s" % (n, c, h, w, mult, k, s, p, dt),
                 passes=("fwd", "bwd_in"))


# ------------------------------------------------------------------ 31 x 31 fp32 grad-weight on the matrix cores
@pytest.mark.parametrize("n,c,h,w,p", [
    (5, 2, 64, 64, 15),     # two 32-row bands, chunks of images
    (3, 3, 48, 48, 15),     # a full band and a partial band
    (6, 2, 32, 32, 15),     # one band
    (2, 2, 9, 9, 15),       # kernel wider than the image; rows not whole 16-byte vectors
    (2, 2, 40, 36, 0),      # no padding: 6 x 10 dy
    (2, 2, 20, 22, 30),     # pad k - 1
    (2, 2, 70, 40, 15),     # three bands
    (1, 1, 33, 17, 7),      # odd sizes, asymmetric output
])
def test_large_kernel_grad_weight_f32_matrix(n, c, h, w, p):
    geo = ((n, c, h, w), (c, 31, 31), 1, p, 1)
    assert dc.dwconv2d_algo(2, *geo, dtype=torch.float32) == "largek_mfma_f32"
    x, wt, b, dy = static_case(n, c, h, w, 1, 31, 1, p, 1, torch.float32, 1500 + h + w + p)
    check_static(x, wt, b, dy, 1, p, 1, "largek-mfma32-bw n%d c%d %dx%d p%d" % (n, c, h, w, p), passes=("bwd_w",))


# ------------------------------------------------------------------ 31 x 31 fp32 forward / grad-input on the matrix cores
@pytest.mark.parametrize("n,c,h,w,mult,p,bin_m", [
    (2, 2, 64, 64, 1, 15, True),      # two 32-row bands, two 32-column tiles
    (3, 3, 64, 56, 1, 15, True),      # partial band and partial column tile
    (2, 2, 32, 32, 1, 15, True),      # one band, one column tile
    (2, 2, 9, 9, 1, 15, True),        # kernel wider than the image; rows not whole 16-byte vectors
    (2, 2, 40, 36, 1, 0, True),       # no padding: 10 x 6 output; grad-input pad 30
    (2, 2, 20, 22, 1, 30, True),      # pad k - 1: grad-input pad 0
    (1, 2, 64, 64, 2, 15, False),     # multiplier 2: forward only
    (1, 1, 70, 100, 1, 15, True),     # four column tiles, six bands
    (5, 1, 33, 30, 1, 7, True),       # odd sizes
    (2, 3, 48, 48, 1, 15, True),      # 16-column tiles: three a row
    (2, 2, 40, 80, 1, 15, True),      # five 16-column tiles, two bands
    (1, 1, 20, 144, 1, 15, True),     # nine 16-column tiles
    (2, 2, 48, 48, 2, 15, False),     # 16-column tiles, multiplier 2
])
def test_large_kernel_fwd_f32_matrix(n, c, h, w, mult, p, bin_m):
    """Forward and grad-input of the family, selected through the table (the built-in
    rules prefer it only where its 32-column tiles are mostly input)."""
    geo = ((n, c, h, w), (c * mult, 31, 31), 1, p, 1)
    dt = torch.float32
    assert "largek_mfma_f32" in dc.dwconv2d_algo_candidates(0, *geo, dtype=dt)
    assert ("largek_mfma_f32" in dc.dwconv2d_algo_candidates(1, *geo, dtype=dt)) == bin_m
    x, wt, b, dy = static_case(n, c, h, w, mult, 31, 1, p, 1, dt, 1550 + h + w + p)
    try:
        dc.dwconv2d_set_algo(0, *geo, dtype=dt, algo="largek_mfma_f32")
        if bin_m:
            dc.dwconv2d_set_algo(1, *geo, dtype=dt, algo="largek_mfma_f32")
        check_static(x, wt, b, dy, 1, p, 1, "largek-mfma32 n%d c%d %dx%d m%d p%d" % (n, c, h, w, mult, p),
                     passes=("fwd", "bwd_in"))
    finally:
        for pass_ in (0, 1):
            dc.dwconv2d_set_algo(pass_, *geo, dtype=dt, algo=None)


def test_large_kernel_f32_matrix_deterministic():
    """The fp32 matrix-core passes give bitwise identical results run to run."""
    x, wt, b, dy = static_case(3, 2, 40, 44, 1, 31, 1, 15, 1, torch.float32, 1590)
    xd, wd, bd, dyd = x.to(DEV), wt.to(DEV), b.to(DEV), dy.to(DEV)
    note("fp32 mfma determinism")
    runs = []
    for _ in range(3):
        y = dc.dwconv2d_fwd(xd, wd, bd, 1, 15, 1)
        dx = dc.dwconv2d_bwd_input(dyd, wd, xd.shape, 1, 15, 1)
        gw, gb = dc.dwconv2d_bwd_weight(xd, dyd, wd.shape, 1, 15, 1)
        torch.cuda.synchronize()
        runs.append((y, dx, gw, gb))
    for r in runs[1:]:
        for t1, t2 in zip(runs[0], r):
            assert torch.equal(t1, t2)


# ------------------------------------------------------------------ direct kernels: every valid geometry
@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d,dt", [
    (1, 2, 24, 600, 1, 31, 1, 15, 1, "f32"),      # 31 x 31 over rows of 600
    (1, 1, 520, 520, 1, 31, 1, 15, 1, "f32"),     # 31 x 31 over a 520 x 520 plane
    (1, 1, 4, 16400, 1, 3, 1, 1, 1, "f32"),       # 3 x 3 over rows of 16400
    (1, 1, 4, 16400, 1, 3, 1, 1, 1, "f16"),
    (1, 4, 8, 8192, 1, 3, 1, 1, 1, "f32"),
    (2, 3, 3, 20000, 2, 5, (1, 2), (2, 4), (1, 3), "bf16"),  # per-axis stride, pad, dilation; multiplier 2
])
def test_wide_rows(n, c, h, w, mult, k, s, p, d, dt):
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 1600 + h + w + k)
    check_static(x, wt, b, dy, s, p, d, "wide n%d c%d %dx%d m%d k%d s%s p%s d%s %s" % (n, c, h, w, mult, k, s, p, d, dt))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,c,h,w,mult,k,s,p,d", [
    (2, 3, 17, 23, 1, 3, 1, 1, 1), (2, 2, 20, 18, 2, 5, 2, 4, 2), (1, 2, 13, 29, 3, 7, (2, 1), (3, 0), (1, 2)),
    (3, 2, 9, 9, 1, 31, 1, 15, 1), (1, 1, 1, 1, 1, 3, 1, 1, 1), (2, 2, 11, 12, 1, 4, 3, 2, 1),
])
def test_direct_family_forced(n, c, h, w, mult, k, s, p, d, dt):
    """The direct kernels on ordinary geometries, selected through the table."""
    geo = ((n, c, h, w), (c * mult, k, k), s, p, d)
    x, wt, b, dy = static_case(n, c, h, w, mult, k, s, p, d, DT[dt], 1650 + h + w + k)
    try:
        for pass_ in (0, 1, 2):
            dc.dwconv2d_set_algo(pass_, *geo, dtype=DT[dt], algo="direct")
        check_static(x, wt, b, dy, s, p, d, "direct n%d c%d %dx%d m%d k%d %s" % (n, c, h, w, mult, k, dt))
    finally:
        for pass_ in (0, 1, 2):
            dc.dwconv2d_set_algo(pass_, *geo, dtype=DT[dt], algo=None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,k,dils", [((1, 2, 6, 12000), 3, (1, 3, 5)), ((1, 1, 3, 20000), 5, (1, 2))])
def test_dynamic_wide_rows(shape, k, dils, dtype):
    """Rows too wide for the staged band run on the direct dynamic kernels."""
    x, fs, dy = dyn_bwd_inputs(*shape, k, dils, DT[dtype], 1700 + sum(shape) + k, fdist=("N", 0.0, 1.0 / (k * k)))
    check_dyn(x, fs, dils, "dynamic-wide %s k%d %s" % (shape, k, dtype))
    check_dyn_bwd(x, fs, dy, dils, "dynamic-wide-bwd %s k%d %s" % (shape, k, dtype))


# ------------------------------------------------------------------ 13 x 13 grad-weight on 16 x 16 matrix tiles
@pytest.mark.parametrize("n,c,h,w,p,dt", [
    (3, 2, 64, 64, 6, "f32"),     # two bands of 32 dy rows, register prefetch
    (2, 3, 48, 48, 6, "f32"),     # a full and a partial band
    (4, 2, 32, 32, 6, "f16"),
    (2, 2, 40, 72, 6, "bf16"),    # rows of 72: staged without prefetch
    (2, 2, 33, 30, 0, "f32"),     # no padding, ragged width: element staging
    (2, 2, 20, 22, 12, "f32"),    # pad k - 1
    (2, 2, 9, 9, 6, "f32"),       # filter wider than the image
    (1, 2, 70, 64, 3, "f32"),     # 70 dy rows: three bands
])
def test_grad_weight_13_matrix_tiles(n, c, h, w, p, dt):
    geo = ((n, c, h, w), (c, 13, 13), 1, p, 1)
    assert "largek_mfma_t16" in dc.dwconv2d_algo_candidates(2, *geo, dtype=DT[dt])
    x, wt, b, dy = static_case(n, c, h, w, 1, 13, 1, p, 1, DT[dt], 1750 + h + w + p)
    try:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo="largek_mfma_t16")
        check_static(x, wt, b, dy, 1, p, 1, "wgrad16 n%d c%d %dx%d p%d %s" % (n, c, h, w, p, dt), passes=("bwd_w",))
    finally:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo=None)


# ------------------------------------------------------------------ 7 x 7 grad-weight as a register row stream
@pytest.mark.parametrize("n,c,h,w,dt", [
    (2, 3, 64, 64, "f32"),     # 16 lanes a row, 4 planes a wave, 16-byte rows
    (2, 3, 48, 48, "f16"),     # plane rows of 12 lanes across the wave's 16-lane rows
    (4, 2, 17, 100, "bf16"),   # 25 lanes a row, 2 planes a wave
    (3, 2, 30, 45, "f16"),     # ragged rows: element loads
    (2, 2, 20, 22, "bf16"),
    (2, 2, 33, 32, "f32"),     # a ragged band
    (2, 2, 5, 5, "f32"),       # filter wider than the image
    (1, 2, 100, 256, "f32"),   # rows of 256: one plane a wave, several bands
    (32, 520, 2, 132, "f32"),  # two rounds of units a chunk, bands of 2 rows
])
def test_grad_weight_7_row_stream(n, c, h, w, dt):
    geo = ((n, c, h, w), (c, 7, 7), 1, 3, 1)
    assert "stream_7x7" in dc.dwconv2d_algo_candidates(2, *geo, dtype=DT[dt])
    x, wt, b, dy = static_case(n, c, h, w, 1, 7, 1, 3, 1, DT[dt], 1800 + h + w)
    try:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo="stream_7x7")
        check_static(x, wt, b, dy, 1, 3, 1, "stream7 n%d c%d %dx%d %s" % (n, c, h, w, dt), passes=("bwd_w",))
    finally:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo=None)


# ------------------------------------------------------------------ 16-bit grad-weight of k <= 16 on 16 x 16 matrix tiles
@pytest.mark.parametrize("n,c,h,w,k,p,dt", [
    (3, 2, 64, 64, 13, 6, "f16"),     # two bands, three 32-column window steps
    (2, 3, 48, 48, 13, 6, "bf16"),    # a full and a partial band, two steps
    (4, 2, 32, 32, 7, 3, "f16"),
    (5, 2, 64, 64, 7, 3, "bf16"),
    (2, 2, 20, 22, 13, 12, "bf16"),   # pad k - 1, rows of 22: element staging
    (2, 2, 9, 9, 13, 6, "f16"),       # kernel wider than the image, one step
    (3, 2, 70, 40, 13, 6, "f16"),     # 70 dy rows: three bands
    (2, 2, 33, 30, 7, 0, "bf16"),     # no padding
])
def test_grad_weight_16bit_small_matrix_tiles(n, c, h, w, k, p, dt):
    geo = ((n, c, h, w), (c, k, k), 1, p, 1)
    assert "largek_mfma_h16" in dc.dwconv2d_algo_candidates(2, *geo, dtype=DT[dt])
    x, wt, b, dy = static_case(n, c, h, w, 1, k, 1, p, 1, DT[dt], 1850 + h + w + k + p)
    try:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo="largek_mfma_h16")
        check_static(x, wt, b, dy, 1, p, 1, "wgrad-h16 n%d c%d %dx%d k%d p%d %s" % (n, c, h, w, k, p, dt),
                     passes=("bwd_w",))
    finally:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo=None)


# ------------------------------------------------------------------ 16-bit large kernels on 16 x 16 matrix tiles
@pytest.mark.parametrize("n,c,h,w,mult,k,p,dt,bin_h", [
    (5, 2, 64, 64, 1, 31, 15, "f16", True),     # four 16-row tiles a plane, one image a group
    (3, 3, 48, 48, 1, 31, 15, "bf16", True),    # 3 x 3 tiles
    (6, 2, 32, 32, 1, 31, 15, "bf16", True),    # two images a group, the last group partial
    (2, 2, 64, 64, 2, 31, 15, "f16", False),    # multiplier 2: forward only
    (3, 2, 64, 40, 1, 13, 6, "f16", True),      # 4 x 3 tiles
    (2, 3, 33, 36, 1, 13, 0, "bf16", True),     # no padding, rows of 36: element staging
    (2, 2, 20, 22, 1, 13, 12, "f16", True),     # pad k - 1: grad-input pad 0
    (4, 2, 47, 47, 1, 7, 2, "bf16", True),      # k = 7, odd sizes
    (2, 2, 9, 9, 1, 31, 15, "f16", True),       # kernel wider than the image
    (7, 2048, 16, 16, 1, 7, 3, "f16", True),    # two groups a workgroup: the next group's planes prefetched
])
def test_large_kernel_16bit_small_tiles(n, c, h, w, mult, k, p, dt, bin_h):
    geo = ((n, c, h, w), (c * mult, k, k), 1, p, 1)
    assert "largek_mfma_h16" in dc.dwconv2d_algo_candidates(0, *geo, dtype=DT[dt])
    assert ("largek_mfma_h16" in dc.dwconv2d_algo_candidates(1, *geo, dtype=DT[dt])) == bin_h
    x, wt, b, dy = static_case(n, c, h, w, mult, k, 1, p, 1, DT[dt], 1900 + h + w + k + p)
    try:
        dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo="largek_mfma_h16")
        if bin_h:
            dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo="largek_mfma_h16")
        check_static(x, wt, b, dy, 1, p, 1, "largek-h16 n%d c%d %dx%d m%d k%d p%d %s" % (n, c, h, w, mult, k, p, dt),
                     passes=("fwd", "bwd_in") if bin_h else ("fwd",))
    finally:
        dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo=None)
        if bin_h:
            dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo=None)


# 16-bit 31 x 31 forward / grad-input streaming input rows through rotating
# filter rows (forced family): the large-kernel workload's planes, odd and
# element-staged widths, several column chunks with a ragged last one, pad 0
# and pad k - 1, a multiplier, a kernel wider than the image, input heights
# that are not a multiple of 4, and enough planes that each wave walks two images.
@pytest.mark.gpu
@pytest.mark.parametrize("n,c,h,w,mult,p,dt,bin_ok", [
    (2, 3, 32, 32, 1, 15, "f16", True),
    (2, 2, 48, 48, 1, 15, "bf16", True),
    (2, 2, 64, 64, 1, 15, "f16", True),
    (1, 2, 47, 47, 1, 15, "f16", True),     # element staging, ragged 16-column tile
    (2, 1, 33, 29, 1, 15, "bf16", True),
    (1, 2, 21, 150, 1, 15, "f16", True),    # three column chunks, the last ragged
    (1, 1, 12, 264, 1, 15, "bf16", True),   # five chunks, vector staging
    (2, 2, 40, 40, 1, 0, "f16", True),      # pad 0: grad-input pad 30
    (2, 2, 26, 22, 1, 30, "bf16", True),    # pad k - 1: grad-input pad 0
    (2, 2, 30, 34, 2, 15, "f16", False),    # multiplier 2 (forward only)
    (2, 2, 9, 9, 1, 15, "bf16", True),      # kernel wider than the image
    (1, 2, 5, 70, 1, 15, "f16", True),      # fewer input rows than one batch of four
    (8, 2048, 16, 16, 1, 15, "f16", True),  # many waves of few rows
    (4, 131073, 1, 1, 1, 15, "bf16", True),  # over 2^19 planes: two images a wave
])
def test_large_kernel_row_stream_16bit(n, c, h, w, mult, p, dt, bin_ok):
    run_row_stream_16bit(n, c, h, w, mult, 31, p, dt, bin_ok)


# fp32 31 x 31 forward / grad-input on the same streaming (forced family): the
# workload's planes, element-staged widths (not a multiple of 4), column chunks
# with a ragged last one, pad 0 and pad k - 1, a multiplier, a kernel wider
# than the image, fewer input rows than one batch, and more than 2^19 planes
# (each wave then walks two images).
@pytest.mark.gpu
@pytest.mark.parametrize("n,c,h,w,mult,p,bin_ok", [
    (2, 3, 32, 32, 1, 15, True),
    (2, 2, 48, 48, 1, 15, True),
    (2, 2, 64, 64, 1, 15, True),
    (1, 2, 47, 47, 1, 15, True),     # element staging, ragged 16-column tile
    (2, 1, 33, 29, 1, 15, True),
    (1, 2, 21, 150, 1, 15, True),    # three column chunks, the last ragged
    (1, 1, 12, 264, 1, 15, True),    # five chunks, vector staging
    (2, 2, 40, 40, 1, 0, True),      # pad 0: grad-input pad 30
    (2, 2, 26, 22, 1, 30, True),     # pad k - 1: grad-input pad 0
    (2, 2, 30, 34, 2, 15, False),    # multiplier 2 (forward only)
    (2, 2, 9, 9, 1, 15, True),       # kernel wider than the image
    (1, 2, 5, 70, 1, 15, True),      # fewer input rows than one batch
    (4, 131073, 1, 1, 1, 15, True),  # over 2^19 planes: two images a wave
    (2, 2, 64, 40, 1, 7, True),      # pad 7 (grad-input pad 23), H != W
    (1, 3, 37, 61, 3, 15, False),    # multiplier 3, element staging
    (2, 2, 50, 33, 1, 20, True),     # pad 20: output 60 x 43
])
def test_large_kernel_row_stream_f32(n, c, h, w, mult, p, bin_ok):
    geo = ((n, c, h, w), (c * mult, 31, 31), 1, p, 1)
    assert "largek_roll_f32" in dc.dwconv2d_algo_candidates(0, *geo, dtype=torch.float32)
    assert ("largek_roll_f32" in dc.dwconv2d_algo_candidates(1, *geo, dtype=torch.float32)) == bin_ok
    x, wt, b, dy = static_case(n, c, h, w, mult, 31, 1, p, 1, torch.float32, 2400 + h + w + p + mult)
    try:
        dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo="largek_roll_f32")
        if bin_ok:
            dc.dwconv2d_set_algo(1, *geo, dtype=torch.float32, algo="largek_roll_f32")
        check_static(x, wt, b, dy, 1, p, 1, "largek-roll-f32 n%d c%d %dx%d m%d p%d" % (n, c, h, w, mult, p),
                     passes=("fwd", "bwd_in") if bin_ok else ("fwd",))
    finally:
        dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo=None)
        if bin_ok:
            dc.dwconv2d_set_algo(1, *geo, dtype=torch.float32, algo=None)


@pytest.mark.gpu
def test_large_kernel_row_stream_f32_no_bias():
    """The fp32 stream's forward without a bias starts every output row at zero."""
    n, c, h, w, p = 2, 3, 48, 48, 15
    geo = ((n, c, h, w), (c, 31, 31), 1, p, 1)
    x, wt, b, dy = static_case(n, c, h, w, 1, 31, 1, p, 1, torch.float32, 2490, bias=False)
    assert b is None
    try:
        dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo="largek_roll_f32")
        check_static(x, wt, b, dy, 1, p, 1, "largek-roll-f32 no bias", passes=("fwd",))
    finally:
        dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo=None)


# k = 7 and 13 on the same streaming: four input rows (k = 7) or two (k = 13)
# per contraction; odd heights, element staging, chunks, pad 0 and k - 1, a
# multiplier, kernels wider than the image.
@pytest.mark.gpu
@pytest.mark.parametrize("n,c,h,w,mult,k,p,dt,bin_ok", [
    (2, 3, 32, 32, 1, 7, 3, "f16", True),
    (2, 2, 48, 48, 1, 7, 3, "bf16", True),
    (2, 2, 64, 64, 1, 13, 6, "f16", True),
    (2, 2, 48, 48, 1, 13, 6, "bf16", True),
    (1, 2, 47, 45, 1, 7, 3, "f16", True),     # element staging, ragged tiles
    (2, 1, 33, 29, 1, 13, 6, "bf16", True),
    (1, 2, 21, 150, 1, 13, 6, "f16", True),   # three column chunks
    (1, 1, 14, 264, 1, 7, 3, "bf16", True),   # five chunks, vector staging
    (2, 2, 40, 40, 1, 7, 0, "f16", True),     # pad 0: grad-input pad 6
    (2, 2, 26, 22, 1, 13, 12, "bf16", True),  # pad k - 1: grad-input pad 0
    (2, 2, 20, 24, 1, 7, 6, "f16", True),     # pad k - 1
    (2, 2, 30, 34, 2, 13, 6, "f16", False),   # multiplier 2 (forward only)
    (2, 2, 5, 9, 1, 13, 6, "bf16", True),     # kernel wider than the image
    (1, 2, 3, 70, 1, 7, 3, "f16", True),      # fewer input rows than one step
])
def test_small_kernel_row_stream_16bit(n, c, h, w, mult, k, p, dt, bin_ok):
    run_row_stream_16bit(n, c, h, w, mult, k, p, dt, bin_ok)


def run_row_stream_16bit(n, c, h, w, mult, k, p, dt, bin_ok):
    geo = ((n, c, h, w), (c * mult, k, k), 1, p, 1)
    assert "largek_roll16" in dc.dwconv2d_algo_candidates(0, *geo, dtype=DT[dt])
    assert ("largek_roll16" in dc.dwconv2d_algo_candidates(1, *geo, dtype=DT[dt])) == bin_ok
    x, wt, b, dy = static_case(n, c, h, w, mult, k, 1, p, 1, DT[dt], 2300 + h + w + p + mult)
    try:
        dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo="largek_roll16")
        if bin_ok:
            dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo="largek_roll16")
        check_static(x, wt, b, dy, 1, p, 1, "largek-roll16 n%d c%d %dx%d m%d k%d p%d %s" % (n, c, h, w, mult, k, p, dt),
                     passes=("fwd", "bwd_in") if bin_ok else ("fwd",))
    finally:
        dc.dwconv2d_set_algo(0, *geo, dtype=DT[dt], algo=None)
        if bin_ok:
            dc.dwconv2d_set_algo(1, *geo, dtype=DT[dt], algo=None)


# 16-bit grad-weight streaming input rows, the dy rows moving through the
# filter-row slots (forced family): the workload's planes, element-staged
# widths, pad 0 and pad k - 1, a kernel wider than the image, dy rows shorter
# than 32 (one contraction step), and enough planes that each wave walks two images.
@pytest.mark.gpu
@pytest.mark.parametrize("n,c,h,w,k,p,dt", [
    (3, 2, 64, 64, 31, 15, "f16"),
    (2, 3, 48, 48, 31, 15, "bf16"),
    (3, 2, 32, 32, 31, 15, "f16"),
    (3, 2, 64, 64, 13, 6, "bf16"),
    (2, 3, 48, 48, 13, 6, "f16"),
    (2, 2, 47, 45, 31, 15, "bf16"),   # element staging
    (2, 2, 33, 30, 13, 0, "f16"),     # no padding
    (2, 2, 20, 24, 31, 30, "bf16"),   # pad k - 1 (output rows of 54)
    (2, 2, 9, 9, 31, 15, "f16"),      # kernel wider than the image
    (3, 2, 70, 20, 13, 6, "bf16"),    # 70 rows, one contraction step
    (8, 2048, 16, 16, 31, 15, "f16"),  # two images a wave
])
def test_grad_weight_row_stream_16bit(n, c, h, w, k, p, dt):
    geo = ((n, c, h, w), (c, k, k), 1, p, 1)
    assert "largek_roll16" in dc.dwconv2d_algo_candidates(2, *geo, dtype=DT[dt])
    x, wt, b, dy = static_case(n, c, h, w, 1, k, 1, p, 1, DT[dt], 2500 + h + w + k + p)
    try:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo="largek_roll16")
        check_static(x, wt, b, dy, 1, p, 1, "wgrad-roll16 n%d c%d %dx%d k%d p%d %s" % (n, c, h, w, k, p, dt),
                     passes=("bwd_w",))
    finally:
        dc.dwconv2d_set_algo(2, *geo, dtype=DT[dt], algo=None)
