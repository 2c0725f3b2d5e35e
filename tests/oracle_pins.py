"""Pins that tie the CPU oracle to facts other than itself.

Each ``check_*`` takes an :class:`oracle.oracle.Oracle` and raises
AssertionError when the oracle disagrees with an independent fact:

* a different algorithm on tiny inputs (dense operator matrices built from
  Kronecker products of 0/1 selection matrices, in numpy fp64);
* a library routine the problem reduces to (torch CPU float64 conv2d with
  groups=ic, its autograd, and F.unfold for the dynamic filter);
* closed forms: a one-hot (delta) filter returns the shifted input, all-ones
  input and filter give the in-bounds tap count, zero input gives the bias,
  db is the plain sum of dy;
* adjoint identities <dy, fwd(x, w)> = <bwd_input(dy, w), x> = <bwd_weight(x, dy), w>;
* the dynamic filter equals the static depthwise convolution when every pixel
  carries the same filter; its backward satisfies <dy, y> = <dx, x> =
  sum_b <dF_b, F_b>, matches torch autograd of the unfold formulation and gives
  shifted copies of dy (dx) and products dy * shifted x (dF) for one-hot filters;
* the page-printed geometry chain in tests/golden/.

The same checks run against builds of the oracle with planted mistakes
(test_oracle_pins.py) to show that each mistake is caught.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tiny geometries: (n, ic, ih, iw, mult, (kh, kw), (sh, sw), (ph, pw), (dh, dw)).
# Non-square kernels, unequal strides/pads/dilations, multipliers and kernels
# wider than the image, so that transposed or swapped indices change results.
CASES = [
    (2, 3, 9, 7, 1, (3, 3), (1, 1), (1, 1), (1, 1)),
    (2, 2, 9, 8, 2, (3, 5), (2, 1), (1, 2), (1, 2)),
    (1, 3, 10, 9, 3, (5, 3), (2, 3), (4, 0), (2, 1)),
    (2, 2, 5, 6, 1, (7, 7), (1, 1), (3, 3), (1, 1)),
    (1, 2, 11, 6, 2, (2, 4), (3, 2), (0, 3), (3, 1)),
    (1, 1, 4, 13, 1, (1, 1), (1, 2), (0, 0), (1, 1)),
]


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(case, seed, bias=True):
    n, ic, ih, iw, m, k, s, p, d = case
    r = _rng(seed)
    x = r.uniform(-1, 1, (n, ic, ih, iw))
    w = r.normal(0, 1, (ic * m, k[0], k[1]))
    b = r.uniform(-0.5, 0.5, (ic * m,)) if bias else None
    return x, w, b


def _sel(out_n, in_n, s, p, d, i):
    """0/1 matrix S[o, h] = 1 iff h == o*s - p + i*d (the rows/cols tap i reads)."""
    S = np.zeros((out_n, in_n))
    for o in range(out_n):
        h = o * s - p + i * d
        if 0 <= h < in_n:
            S[o, h] = 1.0
    return S


def _out_len(in_n, k, s, p, d):
    return (in_n + 2 * p - d * (k - 1) - 1) // s + 1


def dense_operator(w_oc, ih, iw, k, s, p, d):
    """A with y_flat = A @ x_flat for one output channel: sum_ij w[i,j] kron(S_i, T_j)."""
    oh = _out_len(ih, k[0], s[0], p[0], d[0])
    ow = _out_len(iw, k[1], s[1], p[1], d[1])
    A = np.zeros((oh * ow, ih * iw))
    for i in range(k[0]):
        Si = _sel(oh, ih, s[0], p[0], d[0], i)
        for j in range(k[1]):
            Tj = _sel(ow, iw, s[1], p[1], d[1], j)
            A += w_oc[i, j] * np.kron(Si, Tj)
    return A, oh, ow


def _torch():
    import torch
    import torch.nn.functional as F
    return torch, F


# ---------------------------------------------------------------- geometry
def check_out_size_closed_form(orc):
    for in_n in range(1, 20):
        for k in range(1, 8):
            for s in range(1, 4):
                for p in range(0, 5):
                    for d in range(1, 4):
                        num = in_n + 2 * p - d * (k - 1) - 1
                        want = num // s + 1 if num >= 0 else 0
                        got = orc.out_size(in_n, k, s, p, d)
                        assert got == want, (in_n, k, s, p, d, got, want)


def check_out_size_torch(orc):
    torch, F = _torch()
    for case in CASES:
        n, ic, ih, iw, m, k, s, p, d = case
        x = torch.zeros(n, ic, ih, iw, dtype=torch.float64)
        w = torch.zeros(ic * m, 1, *k, dtype=torch.float64)
        y = F.conv2d(x, w, None, s, p, d, groups=ic)
        assert tuple(y.shape[2:]) == (orc.out_size(ih, k[0], s[0], p[0], d[0]),
                                      orc.out_size(iw, k[1], s[1], p[1], d[1])), case


def check_golden_mobilenet_geometry(orc):
    with open(os.path.join(GOLDEN, "mobilenet_geometry.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = orc.out_size(c["in"], g["kernel"], c["stride"], g["pad"], g["dilation"])
        assert got == c["out"], (c, got)


# ---------------------------------------------------------------- forward
def check_fwd_dense_bruteforce(orc):
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        x, w, b = _rand_case(case, 10 + ci)
        y = orc.dwconv2d_fwd(x, w, b, s, p, d)
        for nn in range(n):
            for o in range(ic * m):
                A, oh, ow = dense_operator(w[o], ih, iw, k, s, p, d)
                want = A @ x[nn, o // m].reshape(-1) + b[o]
                np.testing.assert_allclose(y[nn, o].reshape(-1), want, rtol=1e-12, atol=1e-12,
                                           err_msg=str(case))


def check_fwd_torch(orc):
    torch, F = _torch()
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        x, w, b = _rand_case(case, 20 + ci)
        want = F.conv2d(torch.from_numpy(x), torch.from_numpy(w).unsqueeze(1),
                        torch.from_numpy(b), s, p, d, groups=ic).numpy()
        got = orc.dwconv2d_fwd(x, w, b, s, p, d)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12, err_msg=str(case))


def check_fwd_delta_filter(orc):
    """A one-hot filter at (i0, j0) returns the input sampled at oh*s - p + i0*d, exactly."""
    for case in CASES:
        n, ic, ih, iw, m, k, s, p, d = case
        x, _, _ = _rand_case(case, 30)
        for i0 in range(k[0]):
            for j0 in range(k[1]):
                w = np.zeros((ic * m, k[0], k[1]))
                w[:, i0, j0] = 1.0
                y = orc.dwconv2d_fwd(x, w, None, s, p, d)
                oh, ow = y.shape[2:]
                want = np.zeros_like(y)
                for a in range(oh):
                    h = a * s[0] - p[0] + i0 * d[0]
                    for bb in range(ow):
                        c = bb * s[1] - p[1] + j0 * d[1]
                        if 0 <= h < ih and 0 <= c < iw:
                            want[:, :, a, bb] = np.repeat(x[:, :, h, c], m, axis=1)
                assert np.array_equal(y, want), (case, i0, j0)


def _count(out_n, in_n, k, s, p, d):
    """In-bounds tap count per output position along one axis (arithmetic, no loops over taps)."""
    o = np.arange(out_n)
    first = o * s - p
    # taps i with 0 <= first + i*d <= in_n - 1, i in [0, k)
    lo = np.maximum(0, -(first // d))            # ceil(-first / d)
    hi = np.minimum(k - 1, (in_n - 1 - first) // d)
    return np.maximum(0, hi - lo + 1)


def check_fwd_ones_count(orc):
    """x == 1 and w == 1: each output equals its number of in-bounds taps, exactly."""
    for case in CASES:
        n, ic, ih, iw, m, k, s, p, d = case
        x = np.ones((n, ic, ih, iw))
        w = np.ones((ic * m, k[0], k[1]))
        y = orc.dwconv2d_fwd(x, w, None, s, p, d)
        oh, ow = y.shape[2:]
        ch = _count(oh, ih, k[0], s[0], p[0], d[0])
        cw = _count(ow, iw, k[1], s[1], p[1], d[1])
        want = np.broadcast_to(np.outer(ch, cw), y.shape)
        assert np.array_equal(y, want), case


def check_fwd_zero_input_gives_bias(orc):
    for case in CASES:
        n, ic, ih, iw, m, k, s, p, d = case
        _, w, b = _rand_case(case, 40)
        y = orc.dwconv2d_fwd(np.zeros((n, ic, ih, iw)), w, b, s, p, d)
        assert np.array_equal(y, np.broadcast_to(b[None, :, None, None], y.shape)), case


# ---------------------------------------------------------------- grad-input
def check_bwd_input_adjoint(orc):
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        x, w, _ = _rand_case(case, 50 + ci, bias=False)
        y = orc.dwconv2d_fwd(x, w, None, s, p, d)
        dy = _rng(60 + ci).normal(0, 1, y.shape)
        dx = orc.dwconv2d_bwd_input(dy, w, x.shape, s, p, d)
        lhs, rhs = float(np.sum(dy * y)), float(np.sum(dx * x))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * y.size, (case, lhs, rhs)


def check_bwd_input_dense_transpose(orc):
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        _, w, _ = _rand_case(case, 70 + ci, bias=False)
        oh = _out_len(ih, k[0], s[0], p[0], d[0])
        ow = _out_len(iw, k[1], s[1], p[1], d[1])
        dy = _rng(80 + ci).normal(0, 1, (n, ic * m, oh, ow))
        dx = orc.dwconv2d_bwd_input(dy, w, (n, ic, ih, iw), s, p, d)
        for nn in range(n):
            for g in range(ic):
                want = np.zeros(ih * iw)
                for mm in range(m):
                    A, _, _ = dense_operator(w[g * m + mm], ih, iw, k, s, p, d)
                    want += A.T @ dy[nn, g * m + mm].reshape(-1)
                np.testing.assert_allclose(dx[nn, g].reshape(-1), want, rtol=1e-12,
                                           atol=1e-12, err_msg=str(case))


def check_bwd_input_structural_zeros(orc):
    """Stride 2, dilation 2, pad 4, 5x5: only even rows/cols are ever read, the rest of dx is exactly 0."""
    n, ic, ih, iw, m = 1, 2, 12, 10, 2
    r = _rng(90)
    w = r.normal(0, 1, (ic * m, 5, 5))
    oh, ow = _out_len(ih, 5, 2, 4, 2), _out_len(iw, 5, 2, 4, 2)
    dy = r.normal(0, 1, (n, ic * m, oh, ow))
    dx = orc.dwconv2d_bwd_input(dy, w, (n, ic, ih, iw), 2, 4, 2)
    assert np.all(dx[:, :, 1::2, :] == 0.0) and np.all(dx[:, :, :, 1::2] == 0.0)
    assert np.all(dx[:, :, 0::2, 0::2] != 0.0)


# ---------------------------------------------------------------- grad-weight
def check_bwd_weight_adjoint(orc):
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        x, w, _ = _rand_case(case, 100 + ci, bias=False)
        y = orc.dwconv2d_fwd(x, w, None, s, p, d)
        dy = _rng(110 + ci).normal(0, 1, y.shape)
        dw, db = orc.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d)
        lhs, rhs = float(np.sum(dy * y)), float(np.sum(dw * w))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * y.size, (case, lhs, rhs)
        np.testing.assert_allclose(db, dy.sum(axis=(0, 2, 3)), rtol=1e-12, atol=1e-12)


def check_backward_torch_autograd(orc):
    torch, F = _torch()
    for ci, case in enumerate(CASES):
        n, ic, ih, iw, m, k, s, p, d = case
        x, w, b = _rand_case(case, 120 + ci)
        xt = torch.from_numpy(x).requires_grad_(True)
        wt = torch.from_numpy(w).unsqueeze(1).requires_grad_(True)
        bt = torch.from_numpy(b).requires_grad_(True)
        yt = F.conv2d(xt, wt, bt, s, p, d, groups=ic)
        dy = _rng(130 + ci).normal(0, 1, tuple(yt.shape))
        yt.backward(torch.from_numpy(dy))
        dx = orc.dwconv2d_bwd_input(dy, w, x.shape, s, p, d)
        dw, db = orc.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d)
        np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11, err_msg=str(case))
        np.testing.assert_allclose(dw, wt.grad.numpy()[:, 0], rtol=1e-11, atol=1e-11,
                                   err_msg=str(case))
        np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- dynamic
DYN_CASES = [  # (n, c, h, w, k, dilations)
    (2, 3, 9, 11, 3, (1, 3, 5)),
    (1, 2, 12, 7, 5, (1, 2)),
    (1, 2, 6, 6, 3, (2,)),
    (2, 1, 4, 13, 1, (1, 3)),
]


def _dyn_inputs(case, seed):
    n, c, h, w, k, dils = case
    r = _rng(seed)
    x = r.normal(0, 1, (n, c, h, w))
    fs = [r.normal(0, 1 / 3, (n, c, k * k, h, w)) for _ in dils]
    return x, fs


def check_dyn_equals_static(orc):
    """Every pixel carrying filter w_b[c]: branch b is the stride-1 depthwise conv at pad = r*d_b, dilation d_b."""
    for ci, case in enumerate(DYN_CASES):
        n, c, h, w, k, dils = case
        r = _rng(140 + ci)
        x = r.normal(0, 1, (n, c, h, w))
        wb = [r.normal(0, 1, (c, k, k)) for _ in dils]
        fs = [np.broadcast_to(wv.reshape(1, c, k * k, 1, 1), (n, c, k * k, h, w)) for wv in wb]
        y = orc.dynconv_multidil_fwd(x, fs, dils)
        for bi, dd in enumerate(dils):
            ys = orc.dwconv2d_fwd(x, wb[bi], None, 1, (k - 1) // 2 * dd, dd)
            np.testing.assert_allclose(y[:, bi * c:(bi + 1) * c], ys, rtol=1e-12, atol=1e-12,
                                       err_msg=str(case))


def check_dyn_unfold(orc):
    """Library formulation: F.unfold windows times per-pixel filters, summed over taps."""
    torch, F = _torch()
    for ci, case in enumerate(DYN_CASES):
        n, c, h, w, k, dils = case
        x, fs = _dyn_inputs(case, 150 + ci)
        y = orc.dynconv_multidil_fwd(x, fs, dils)
        outs = []
        for bi, dd in enumerate(dils):
            cols = F.unfold(torch.from_numpy(x), k, dilation=dd, padding=(k - 1) // 2 * dd)
            cols = cols.view(n, c, k * k, h, w)
            outs.append((cols * torch.from_numpy(fs[bi])).sum(2))
        want = torch.cat(outs, 1).numpy()
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12, err_msg=str(case))


def check_dyn_one_hot_tap(orc):
    """Filter one-hot at tap t = i*k + j: branch output is x shifted by ((i-r)d, (j-r)d), exactly."""
    for case in DYN_CASES:
        n, c, h, w, k, dils = case
        x, _ = _dyn_inputs(case, 160)
        rr = (k - 1) // 2
        for t in range(k * k):
            i, j = divmod(t, k)
            fs = []
            for _ in dils:
                f = np.zeros((n, c, k * k, h, w))
                f[:, :, t] = 1.0
                fs.append(f)
            y = orc.dynconv_multidil_fwd(x, fs, dils)
            for bi, dd in enumerate(dils):
                want = np.zeros((n, c, h, w))
                dyy, dxx = (i - rr) * dd, (j - rr) * dd
                for py in range(h):
                    for px in range(w):
                        sy, sx = py + dyy, px + dxx
                        if 0 <= sy < h and 0 <= sx < w:
                            want[:, :, py, px] = x[:, :, sy, sx]
                assert np.array_equal(y[:, bi * c:(bi + 1) * c], want), (case, t, bi)


def check_dyn_ones_count(orc):
    for case in DYN_CASES:
        n, c, h, w, k, dils = case
        fs = [np.ones((n, c, k * k, h, w)) for _ in dils]
        y = orc.dynconv_multidil_fwd(np.ones((n, c, h, w)), fs, dils)
        for bi, dd in enumerate(dils):
            p = (k - 1) // 2 * dd
            want = np.outer(_count(h, h, k, 1, p, dd), _count(w, w, k, 1, p, dd))
            assert np.array_equal(y[:, bi * c:(bi + 1) * c], np.broadcast_to(want, (n, c, h, w)))


# ---------------------------------------------------------------- dynamic, backward
def _dyn_bwd_case(case, seed):
    n, c, h, w, k, dils = case
    x, fs = _dyn_inputs(case, seed)
    dy = _rng(seed + 1).normal(0, 1, (n, len(dils) * c, h, w))
    return x, fs, dy


def check_dyn_bwd_adjoint(orc):
    """y is bilinear: <dy, y> = <dx, x> = sum_b <dF_b, F_b>."""
    for ci, case in enumerate(DYN_CASES):
        x, fs, dy = _dyn_bwd_case(case, 170 + ci)
        dils = case[5]
        y = orc.dynconv_multidil_fwd(x, fs, dils)
        dx, dfs = orc.dynconv_multidil_bwd(x, fs, dy, dils)
        ref = float(np.sum(dy * y))
        lx = float(np.sum(dx * x))
        lf = float(sum(np.sum(df * f) for df, f in zip(dfs, fs)))
        tol = 1e-12 * max(1.0, abs(ref)) * y.size
        assert abs(ref - lx) <= tol and abs(ref - lf) <= tol, (case, ref, lx, lf)


def check_dyn_bwd_autograd(orc):
    """torch autograd (float64, CPU) of the F.unfold formulation."""
    torch, F = _torch()
    for ci, case in enumerate(DYN_CASES):
        n, c, h, w, k, dils = case
        x, fs, dy = _dyn_bwd_case(case, 180 + ci)
        xt = torch.from_numpy(x).requires_grad_(True)
        ft = [torch.from_numpy(f).requires_grad_(True) for f in fs]
        outs = []
        for bi, dd in enumerate(dils):
            cols = F.unfold(xt, k, dilation=dd, padding=(k - 1) // 2 * dd).view(n, c, k * k, h, w)
            outs.append((cols * ft[bi]).sum(2))
        torch.cat(outs, 1).backward(torch.from_numpy(dy))
        dx, dfs = orc.dynconv_multidil_bwd(x, fs, dy, dils)
        np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11, err_msg=str(case))
        for bi in range(len(dils)):
            np.testing.assert_allclose(dfs[bi], ft[bi].grad.numpy(), rtol=1e-11, atol=1e-11,
                                       err_msg="%s branch %d" % (case, bi))


def check_dyn_bwd_one_hot(orc):
    """Filters one-hot at tap t: dx is the sum over branches of dy_b shifted back by
    ((i-r)d_b, (j-r)d_b), and dF_b at every tap is dy_b times x shifted forward, exactly."""
    for case in DYN_CASES:
        n, c, h, w, k, dils = case
        x, _, dy = _dyn_bwd_case(case, 190)
        rr = (k - 1) // 2
        for t in range(k * k):
            i, j = divmod(t, k)
            fs = []
            for _ in dils:
                f = np.zeros((n, c, k * k, h, w))
                f[:, :, t] = 1.0
                fs.append(f)
            dx, dfs = orc.dynconv_multidil_bwd(x, fs, dy, dils)
            want = np.zeros((n, c, h, w))
            for bi, dd in enumerate(dils):
                g = dy[:, bi * c:(bi + 1) * c]
                for py in range(h):
                    for px in range(w):
                        sy, sx = py + (i - rr) * dd, px + (j - rr) * dd
                        if 0 <= sy < h and 0 <= sx < w:
                            want[:, :, sy, sx] += g[:, :, py, px]
            assert np.array_equal(dx, want), (case, t)
        x, fs, dy = _dyn_bwd_case(case, 195)
        _, dfs = orc.dynconv_multidil_bwd(x, fs, dy, dils)
        for bi, dd in enumerate(dils):
            g = dy[:, bi * c:(bi + 1) * c]
            for t in range(k * k):
                i, j = divmod(t, k)
                want = np.zeros((n, c, h, w))
                for py in range(h):
                    for px in range(w):
                        sy, sx = py + (i - rr) * dd, px + (j - rr) * dd
                        if 0 <= sy < h and 0 <= sx < w:
                            want[:, :, py, px] = g[:, :, py, px] * x[:, :, sy, sx]
                assert np.array_equal(dfs[bi][:, :, t], want), (case, bi, t)


def check_dyn_bwd_parts(orc):
    """Asking for one part gives the same values as asking for both."""
    for ci, case in enumerate(DYN_CASES):
        x, fs, dy = _dyn_bwd_case(case, 200 + ci)
        dils = case[5]
        dx, dfs = orc.dynconv_multidil_bwd(x, fs, dy, dils)
        dx1, none1 = orc.dynconv_multidil_bwd(x, fs, dy, dils, need_df=False)
        none2, dfs2 = orc.dynconv_multidil_bwd(x, fs, dy, dils, need_dx=False)
        assert none1 is None and none2 is None
        assert np.array_equal(dx, dx1)
        for a, b in zip(dfs, dfs2):
            assert np.array_equal(a, b)


ALL_CHECKS = [v for k_, v in sorted(globals().items()) if k_.startswith("check_")]
