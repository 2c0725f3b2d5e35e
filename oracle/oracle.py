"""CPU oracle for depthwise 2-D convolution and the dynamic multi-dilation filter.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The HIP product path
never imports, links or calls anything under ``oracle/``, and this module
imports nothing from the product package.

The arithmetic lives in ``dwconv_oracle.c`` (plain C, fp64 direct loops; its
header names the passages each loop follows).  This module only compiles it
with gcc when no build is present, converts arrays to contiguous float64 and
calls it through ctypes.  Inputs may be numpy arrays or CPU torch tensors of any
float dtype; they are upcast exactly to float64, so a 16-bit tensor the device
sees is the same value here.  Outputs are float64 numpy arrays, never rounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dwconv_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)
GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """gcc-compile one oracle source file into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc"] + GCC_FLAGS + ["-o", tmp, src])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile liboracle.so when missing or older than its source."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        compile_source(SRC, LIB)
    return LIB


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch CPU tensor: exact upcast through torch
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        geo = [_I64] * 13
        lib.oracle_out_size.argtypes = [_I64] * 5
        lib.oracle_out_size.restype = _I64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_dwconv_fwd.argtypes = [_DP, _DP, _DP, _DP] + geo
        lib.oracle_dwconv_fwd.restype = None
        lib.oracle_dwconv_bwd_input.argtypes = [_DP, _DP, _DP] + geo
        lib.oracle_dwconv_bwd_input.restype = None
        lib.oracle_dwconv_bwd_weight.argtypes = [_DP, _DP, _DP, _DP] + geo
        lib.oracle_dwconv_bwd_weight.restype = None
        lib.oracle_dynconv_multidil_fwd.argtypes = [
            _DP, ctypes.POINTER(_DP), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, _DP,
            _I64, _I64, _I64, _I64, _I64]
        lib.oracle_dynconv_multidil_fwd.restype = None
        lib.oracle_dynconv_multidil_bwd.argtypes = [
            _DP, ctypes.POINTER(_DP), _DP, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, _DP,
            ctypes.POINTER(_DP), _I64, _I64, _I64, _I64, _I64]
        lib.oracle_dynconv_multidil_bwd.restype = None
        self._lib = lib
        self.path = path

    # -- geometry -----------------------------------------------------------
    def out_size(self, in_size: int, k: int, stride: int, pad: int, dil: int) -> int:
        """Output length along one axis (0 when no window fits)."""
        return int(self._lib.oracle_out_size(in_size, k, stride, pad, dil))

    def num_threads(self) -> int:
        """OpenMP threads the oracle's loops run on."""
        return int(self._lib.oracle_num_threads())

    def set_threads(self, n: int) -> None:
        """Run later calls on n OpenMP threads (results do not depend on it)."""
        self._lib.oracle_set_threads(int(n))

    def geometry(self, x_shape, w_shape, stride=1, padding=0, dilation=1):
        """(13 geometry integers, oh, ow); raises ValueError on an invalid problem."""
        n, ic, ih, iw = (int(s) for s in x_shape)
        w_shape = tuple(int(s) for s in w_shape)
        oc, kh, kw = w_shape[0], w_shape[-2], w_shape[-1]
        sh, sw = _pair(stride)
        ph, pw = _pair(padding)
        dh, dw = _pair(dilation)
        if min(n, ic, ih, iw, oc, kh, kw, sh, sw, dh, dw) < 1 or min(ph, pw) < 0:
            raise ValueError("sizes, strides and dilations must be >= 1, pads >= 0")
        if oc % ic:
            raise ValueError("output channels must be a multiple of input channels")
        oh = self.out_size(ih, kh, sh, ph, dh)
        ow = self.out_size(iw, kw, sw, pw, dw)
        if oh < 1 or ow < 1:
            raise ValueError("empty output")
        return (n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw), oh, ow

    # -- static depthwise ---------------------------------------------------
    def dwconv2d_fwd(self, x, w, bias=None, stride=1, padding=0, dilation=1) -> np.ndarray:
        """y (n, oc, oh, ow) = depthwise conv of x (n, ic, ih, iw) with w (oc, [1,] kh, kw) + bias."""
        x, w = _f64(x), _f64(w)
        b = None if bias is None else _f64(bias)
        geo, oh, ow = self.geometry(x.shape, w.shape, stride, padding, dilation)
        y = np.empty((geo[0], geo[4], oh, ow), np.float64)
        self._lib.oracle_dwconv_fwd(_ptr(x), _ptr(w), _ptr(b), _ptr(y), *geo)
        return y

    def dwconv2d_bwd_input(self, dy, w, x_shape, stride=1, padding=0, dilation=1) -> np.ndarray:
        """dx (shape x_shape) of the forward above, given dy (n, oc, oh, ow)."""
        dy, w = _f64(dy), _f64(w)
        geo, oh, ow = self.geometry(x_shape, w.shape, stride, padding, dilation)
        if tuple(dy.shape) != (geo[0], geo[4], oh, ow):
            raise ValueError("dy shape %s does not match the geometry" % (dy.shape,))
        dx = np.empty(tuple(int(s) for s in x_shape), np.float64)
        self._lib.oracle_dwconv_bwd_input(_ptr(dy), _ptr(w), _ptr(dx), *geo)
        return dx

    def dwconv2d_bwd_weight(self, x, dy, w_shape, stride=1, padding=0, dilation=1,
                            with_bias=True):
        """(dw of shape w_shape, db of shape (oc,) or None) of the forward above."""
        x, dy = _f64(x), _f64(dy)
        geo, oh, ow = self.geometry(x.shape, w_shape, stride, padding, dilation)
        if tuple(dy.shape) != (geo[0], geo[4], oh, ow):
            raise ValueError("dy shape %s does not match the geometry" % (dy.shape,))
        dw = np.empty(tuple(int(s) for s in w_shape), np.float64)
        db = np.empty((geo[4],), np.float64) if with_bias else None
        self._lib.oracle_dwconv_bwd_weight(_ptr(x), _ptr(dy), _ptr(dw), _ptr(db), *geo)
        return dw, db

    # -- dynamic multi-dilation ---------------------------------------------
    def dynconv_multidil_fwd(self, x, filters, dilations=(1, 3, 5)) -> np.ndarray:
        """Branch-concatenated output (n, nb*c, h, w); filters[b] is (n, c, k*k, h, w)."""
        x = _f64(x)
        fs = [_f64(f) for f in filters]
        n, c, h, w = x.shape
        nb = len(fs)
        if nb < 1 or nb != len(dilations):
            raise ValueError("one filter tensor per dilation")
        kk = fs[0].shape[2]
        k = int(round(kk ** 0.5))
        if k * k != kk or k % 2 == 0:
            raise ValueError("filters must hold an odd k*k taps")
        for f in fs:
            if tuple(f.shape) != (n, c, kk, h, w):
                raise ValueError("filter shape %s does not match x" % (f.shape,))
        if min(int(d) for d in dilations) < 1:
            raise ValueError("dilations must be >= 1")
        y = np.empty((n, nb * c, h, w), np.float64)
        arr = (_DP * nb)(*[_ptr(f) for f in fs])
        dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
        self._lib.oracle_dynconv_multidil_fwd(_ptr(x), arr, dil, nb, _ptr(y), n, c, h, w, k)
        return y

    def dynconv_multidil_bwd(self, x, filters, dy, dilations=(1, 3, 5), need_dx=True, need_df=True):
        """(dx, [dF_b]) of the branch-concatenated dynamic filter for the output gradient dy
        (n, nb*c, h, w); dx is (n, c, h, w), dF_b like filters[b].  Either part may be
        skipped (returned as None)."""
        x = _f64(x)
        fs = [_f64(f) for f in filters]
        dy = _f64(dy)
        n, c, h, w = x.shape
        nb = len(fs)
        if nb < 1 or nb != len(dilations):
            raise ValueError("one filter tensor per dilation")
        kk = fs[0].shape[2]
        k = int(round(kk ** 0.5))
        if k * k != kk or k % 2 == 0:
            raise ValueError("filters must hold an odd k*k taps")
        for f in fs:
            if tuple(f.shape) != (n, c, kk, h, w):
                raise ValueError("filter shape %s does not match x" % (f.shape,))
        if tuple(dy.shape) != (n, nb * c, h, w):
            raise ValueError("dy shape %s does not match (n, nb*c, h, w)" % (dy.shape,))
        if min(int(d) for d in dilations) < 1:
            raise ValueError("dilations must be >= 1")
        dx = np.empty((n, c, h, w), np.float64) if need_dx else None
        dfs = [np.empty((n, c, kk, h, w), np.float64) for _ in fs] if need_df else None
        arr = (_DP * nb)(*[_ptr(f) for f in fs])
        darr = (_DP * nb)(*[_ptr(f) for f in dfs]) if need_df else None
        dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
        self._lib.oracle_dynconv_multidil_bwd(_ptr(x), arr, _ptr(dy), dil, nb, _ptr(dx), darr, n, c, h, w, k)
        return dx, dfs


_default = None


def default() -> Oracle:
    """The oracle built from dwconv_oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def load_variant(path: str) -> Oracle:
    """An Oracle bound to another build; the planted-mistake test uses this."""
    return Oracle(path)


# Module-level shortcuts to the default oracle.
def out_size(*a):
    return default().out_size(*a)


def num_threads():
    return default().num_threads()


def set_threads(n):
    default().set_threads(n)


def geometry(*a, **k):
    return default().geometry(*a, **k)


def dwconv2d_fwd(*a, **k):
    return default().dwconv2d_fwd(*a, **k)


def dwconv2d_bwd_input(*a, **k):
    return default().dwconv2d_bwd_input(*a, **k)


def dwconv2d_bwd_weight(*a, **k):
    return default().dwconv2d_bwd_weight(*a, **k)


def dynconv_multidil_fwd(*a, **k):
    return default().dynconv_multidil_fwd(*a, **k)


def dynconv_multidil_bwd(*a, **k):
    return default().dynconv_multidil_bwd(*a, **k)
