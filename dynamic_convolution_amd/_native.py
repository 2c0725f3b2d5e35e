"""ctypes binding to libdwconv.so (the C ABI in include/dwconv.h).

Argument marshalling only: tensor shapes become the ABI's integers, data
pointers and torch's current HIP stream are passed through, and a nonzero
status becomes an exception.  Every step of the computation runs in the HIP
kernels behind the ABI; there is no CPU path.  When libdwconv.so is missing
the first call raises, naming the build step.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdwconv.so")

DW_F32, DW_F16, DW_BF16 = 0, 1, 2
STATUS = {
    0: "DW_OK", -1: "DW_EPTR", -2: "DW_ESHAPE", -3: "DW_EMULT", -4: "DW_EDTYPE",
    -5: "DW_EWORKSPACE", -6: "DW_ETOOLARGE", -7: "DW_EALIAS", -8: "DW_EHIP",
    -9: "DW_EDYN", -10: "DW_EUNSUPPORTED", -11: "DW_ESCRATCH",
}
# every exported symbol the header declares
EXPORTS = (
    "dwconv2d_out_size", "dwconv2d_fwd", "dwconv2d_bwd_input",
    "dwconv2d_bwd_weight_workspace_bytes", "dwconv2d_bwd_weight",
    "dynconv_multidil_fwd", "dynconv_multidil_bwd", "dynconv_multidil_fwd_into",
    "dynconv_multidil_bwd_from", "dwconv2d_algo", "dw_status_str",
    "dwconv2d_algo_candidates", "dwconv2d_set_algo", "dwconv2d_tune_fwd", "dwconv2d_tune_bwd_input",
    "dwconv2d_tune_bwd_weight", "dwconv2d_bwd_weight_noalloc",
)

# size of the device array dwconv2d_bwd_weight_noalloc keeps its partial sums in
NOALLOC_SCRATCH_BYTES = 32 << 20

_I64 = ctypes.c_int64
_VP = ctypes.c_void_p
_GEO = [_I64] * 13
_lib = None


class DwconvError(RuntimeError):
    """A nonzero status returned by libdwconv."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), status_str(status)))


def lib() -> ctypes.CDLL:
    """The loaded libdwconv.so with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libdwconv.so is not built (%s); run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python dynamic_convolution_amd/build.py`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.dwconv2d_out_size.argtypes = _GEO + [ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
    L.dwconv2d_out_size.restype = ctypes.c_int
    L.dwconv2d_fwd.argtypes = [_VP, _VP, _VP, _VP] + _GEO + [ctypes.c_int, _VP]
    L.dwconv2d_fwd.restype = ctypes.c_int
    L.dwconv2d_bwd_input.argtypes = [_VP, _VP, _VP] + _GEO + [ctypes.c_int, _VP]
    L.dwconv2d_bwd_input.restype = ctypes.c_int
    L.dwconv2d_bwd_weight_workspace_bytes.argtypes = _GEO + [ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.dwconv2d_bwd_weight_workspace_bytes.restype = ctypes.c_int
    L.dwconv2d_bwd_weight.argtypes = [_VP, _VP, _VP, _VP, _VP, ctypes.c_size_t] + _GEO + [ctypes.c_int, _VP]
    L.dwconv2d_bwd_weight.restype = ctypes.c_int
    L.dwconv2d_bwd_weight_noalloc.argtypes = [_VP, _VP, _VP, _VP] + _GEO + [ctypes.c_int, _VP]
    L.dwconv2d_bwd_weight_noalloc.restype = ctypes.c_int
    L.dynconv_multidil_fwd.argtypes = [_VP, ctypes.POINTER(_VP), ctypes.POINTER(ctypes.c_int32),
                                       ctypes.c_int32, _VP, _I64, _I64, _I64, _I64, _I64,
                                       ctypes.c_int, _VP]
    L.dynconv_multidil_fwd.restype = ctypes.c_int
    L.dynconv_multidil_bwd.argtypes = [_VP, ctypes.POINTER(_VP), _VP, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.c_int32, _VP, ctypes.POINTER(_VP), _I64, _I64, _I64, _I64, _I64,
                                       ctypes.c_int, _VP]
    L.dynconv_multidil_bwd.restype = ctypes.c_int
    L.dynconv_multidil_fwd_into.argtypes = [_VP, ctypes.POINTER(_VP), ctypes.POINTER(ctypes.c_int32),
                                            ctypes.c_int32, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                            ctypes.c_int, _VP]
    L.dynconv_multidil_fwd_into.restype = ctypes.c_int
    L.dynconv_multidil_bwd_from.argtypes = [_VP, ctypes.POINTER(_VP), _VP, _I64, _I64, ctypes.POINTER(ctypes.c_int32),
                                            ctypes.c_int32, _VP, ctypes.POINTER(_VP), _I64, _I64, _I64, _I64, _I64,
                                            ctypes.c_int, _VP]
    L.dynconv_multidil_bwd_from.restype = ctypes.c_int
    L.dwconv2d_algo.argtypes = [ctypes.c_int] + _GEO + [ctypes.c_int]
    L.dwconv2d_algo.restype = ctypes.c_char_p
    _CP = ctypes.c_char_p
    L.dwconv2d_algo_candidates.argtypes = [ctypes.c_int] + _GEO + [ctypes.c_int, ctypes.POINTER(_CP), ctypes.c_int]
    L.dwconv2d_algo_candidates.restype = ctypes.c_int
    L.dwconv2d_set_algo.argtypes = [ctypes.c_int] + _GEO + [ctypes.c_int, _CP]
    L.dwconv2d_set_algo.restype = ctypes.c_int
    L.dwconv2d_tune_fwd.argtypes = [_VP, _VP, _VP, _VP] + _GEO + [ctypes.c_int, ctypes.c_int, _VP,
                                                                  ctypes.POINTER(_CP)]
    L.dwconv2d_tune_fwd.restype = ctypes.c_int
    L.dwconv2d_tune_bwd_input.argtypes = [_VP, _VP, _VP] + _GEO + [ctypes.c_int, ctypes.c_int, _VP,
                                                                   ctypes.POINTER(_CP)]
    L.dwconv2d_tune_bwd_input.restype = ctypes.c_int
    L.dwconv2d_tune_bwd_weight.argtypes = [_VP, _VP, _VP, _VP, _VP, ctypes.c_size_t] + _GEO + [
        ctypes.c_int, ctypes.c_int, _VP, ctypes.POINTER(_CP)]
    L.dwconv2d_tune_bwd_weight.restype = ctypes.c_int
    L.dw_status_str.argtypes = [ctypes.c_int]
    L.dw_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().dw_status_str(int(status)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise DwconvError(rc, where)


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: DW_F32, torch.float16: DW_F16, torch.bfloat16: DW_BF16}
    if t.dtype not in codes:
        raise TypeError("unsupported dtype %s (float32, float16, bfloat16)" % t.dtype)
    return codes[t.dtype]


def _dev(t, name: str):
    """Device pointer of a contiguous GPU tensor (raises for CPU or strided tensors)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor: there is no CPU path" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (NCHW)" % name)
    return t.data_ptr()


def _match(t, name: str, shape, ref):
    """Raises unless tensor t has exactly `shape`, ref's dtype and ref's device (the
    library writes or reads that many elements of that type through t's pointer)."""
    if tuple(int(v) for v in t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != ref.dtype:
        raise TypeError("%s dtype %s != %s" % (name, t.dtype, ref.dtype))
    if t.device != ref.device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, ref.device))


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _geo(x_shape, w_shape, stride, padding, dilation):
    n, ic, ih, iw = (int(s) for s in x_shape)
    w_shape = tuple(int(s) for s in w_shape)
    if len(w_shape) == 4 and w_shape[1] != 1:
        raise ValueError("depthwise filters have shape (oc, kh, kw) or (oc, 1, kh, kw)")
    oc, kh, kw = w_shape[0], w_shape[-2], w_shape[-1]
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    return (n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw)


def dwconv2d_out_size(x_shape, w_shape, stride=1, padding=0, dilation=1):
    """(oh, ow) for the geometry, computed by the library."""
    oh, ow = _I64(), _I64()
    _check(lib().dwconv2d_out_size(*_geo(x_shape, w_shape, stride, padding, dilation),
                                   ctypes.byref(oh), ctypes.byref(ow)), "dwconv2d_out_size")
    return oh.value, ow.value


def dwconv2d_algo(pass_, x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=None):
    """Kernel family pass_ (0 fwd, 1 grad-input, 2 grad-weight) launches for this geometry."""
    import torch
    code = _dtype_code(torch.empty(0, dtype=dtype or torch.float32))
    r = lib().dwconv2d_algo(int(pass_), *_geo(x_shape, w_shape, stride, padding, dilation), code)
    if r is None:
        raise ValueError("invalid pass, dtype or geometry")
    return r.decode()


def dwconv2d_bwd_weight_workspace_bytes(x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=None):
    import torch
    code = _dtype_code(torch.empty(0, dtype=dtype or torch.float32))
    nbytes = ctypes.c_size_t()
    _check(lib().dwconv2d_bwd_weight_workspace_bytes(*_geo(x_shape, w_shape, stride, padding, dilation),
                                                     code, ctypes.byref(nbytes)),
           "dwconv2d_bwd_weight_workspace_bytes")
    return nbytes.value


def dwconv2d_fwd(x, w, bias=None, stride=1, padding=0, dilation=1, out=None):
    """y = depthwise conv2d of x (n, ic, ih, iw) with w (oc, [1,] kh, kw) plus bias (oc)."""
    import torch
    geo = _geo(x.shape, w.shape, stride, padding, dilation)
    oh, ow = dwconv2d_out_size(x.shape, w.shape, stride, padding, dilation)
    if out is None:
        out = torch.empty((geo[0], geo[4], oh, ow), dtype=x.dtype, device=x.device)
    code = _dtype_code(x)
    _match(w, "w", w.shape, x)
    if bias is not None:
        _match(bias, "bias", (geo[4],), x)
    _match(out, "out", (geo[0], geo[4], oh, ow), x)
    _check(lib().dwconv2d_fwd(_dev(x, "x"), _dev(w, "w"), _dev(bias, "bias"), _dev(out, "out"), *geo,
                              code, _stream(x)), "dwconv2d_fwd")
    return out


def dwconv2d_bwd_input(dy, w, x_shape, stride=1, padding=0, dilation=1, out=None):
    """dx (shape x_shape) of the forward above, given dy (n, oc, oh, ow)."""
    import torch
    geo = _geo(x_shape, w.shape, stride, padding, dilation)
    if out is None:
        out = torch.empty(tuple(int(s) for s in x_shape), dtype=dy.dtype, device=dy.device)
    code = _dtype_code(dy)
    oh, ow = dwconv2d_out_size(x_shape, w.shape, stride, padding, dilation)
    _match(dy, "dy", (geo[0], geo[4], oh, ow), dy)
    _match(w, "w", w.shape, dy)
    _match(out, "out", geo[:4], dy)
    _check(lib().dwconv2d_bwd_input(_dev(dy, "dy"), _dev(w, "w"), _dev(out, "out"), *geo, code,
                                    _stream(dy)), "dwconv2d_bwd_input")
    return out


def dwconv2d_bwd_weight(x, dy, w_shape, stride=1, padding=0, dilation=1, with_bias=True,
                        out=None, out_bias=None, workspace=None):
    """(dw of shape w_shape, db of shape (oc,) or None) of the forward above.

    The workspace (uint8 GPU tensor) is allocated here when not given.
    """
    import torch
    geo = _geo(x.shape, w_shape, stride, padding, dilation)
    code = _dtype_code(x)
    oh, ow = dwconv2d_out_size(x.shape, w_shape, stride, padding, dilation)
    _match(dy, "dy", (geo[0], geo[4], oh, ow), x)
    if out is None:
        out = torch.empty(tuple(int(s) for s in w_shape), dtype=x.dtype, device=x.device)
    _match(out, "out", w_shape, x)
    if with_bias:
        if out_bias is None:
            out_bias = torch.empty((geo[4],), dtype=x.dtype, device=x.device)
        _match(out_bias, "out_bias", (geo[4],), x)
    nbytes = dwconv2d_bwd_weight_workspace_bytes(x.shape, w_shape, stride, padding, dilation, x.dtype)
    if workspace is None:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    if workspace.device != x.device:
        raise ValueError("workspace is on %s, expected %s" % (workspace.device, x.device))
    _check(lib().dwconv2d_bwd_weight(_dev(x, "x"), _dev(dy, "dy"), _dev(out, "out"),
                                     _dev(out_bias, "out_bias") if with_bias else None,
                                     _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                     *geo, code, _stream(x)), "dwconv2d_bwd_weight")
    return out, (out_bias if with_bias else None)


def dwconv2d_bwd_weight_noalloc(x, dy, w_shape, stride=1, padding=0, dilation=1, with_bias=True,
                                out=None, out_bias=None):
    """dwconv2d_bwd_weight with the partial sums in the library's fixed device scratch.

    The library allocates nothing; pass `out` (and `out_bias`) to allocate nothing here either.
    """
    import torch
    geo = _geo(x.shape, w_shape, stride, padding, dilation)
    code = _dtype_code(x)
    oh, ow = dwconv2d_out_size(x.shape, w_shape, stride, padding, dilation)
    _match(dy, "dy", (geo[0], geo[4], oh, ow), x)
    if out is None:
        out = torch.empty(tuple(int(s) for s in w_shape), dtype=x.dtype, device=x.device)
    _match(out, "out", w_shape, x)
    if with_bias:
        if out_bias is None:
            out_bias = torch.empty((geo[4],), dtype=x.dtype, device=x.device)
        _match(out_bias, "out_bias", (geo[4],), x)
    with torch.cuda.device(x.device):  # the library resolves the scratch of the current device
        _check(lib().dwconv2d_bwd_weight_noalloc(_dev(x, "x"), _dev(dy, "dy"), _dev(out, "out"),
                                                 _dev(out_bias, "out_bias") if with_bias else None,
                                                 *geo, code, _stream(x)), "dwconv2d_bwd_weight_noalloc")
    return out, (out_bias if with_bias else None)


def dynconv_multidil_fwd(x, filters, dilations=(1, 3, 5), out=None):
    """Branch-concatenated dynamic-filter output (n, nb*c, h, w); filters[b] is (n, c, k*k, h, w)."""
    import torch
    n, c, h, w = (int(s) for s in x.shape)
    nb = len(filters)
    if nb != len(dilations):
        raise ValueError("one filter tensor per dilation")
    kk = int(filters[0].shape[2])
    k = int(round(kk ** 0.5))
    if k * k != kk:
        raise ValueError("filters must hold k*k taps")
    for f in filters:
        if tuple(f.shape) != (n, c, kk, h, w) or f.dtype != x.dtype:
            raise ValueError("filter %s %s does not match x" % (tuple(f.shape), f.dtype))
        _match(f, "filter", (n, c, kk, h, w), x)
    if out is None:
        out = torch.empty((n, nb * c, h, w), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (n, nb * c, h, w) or out.dtype != x.dtype:
        raise ValueError("out %s %s does not match" % (tuple(out.shape), out.dtype))
    _match(out, "out", (n, nb * c, h, w), x)
    fptrs = (_VP * nb)(*[_dev(f, "filter") for f in filters])
    dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
    _check(lib().dynconv_multidil_fwd(_dev(x, "x"), fptrs, dil, nb, _dev(out, "out"), n, c, h, w, k,
                                      _dtype_code(x), _stream(x)), "dynconv_multidil_fwd")
    return out


def dynconv_multidil_bwd(x, filters, dy, dilations=(1, 3, 5), need_dx=True, need_dfilters=True,
                         out_dx=None, out_dfilters=None):
    """(dx, [dF_b]) of dynconv_multidil_fwd for the output gradient dy (n, nb*c, h, w).

    dx has x's shape and dF_b filters[b]'s; a part not needed is returned as None.
    """
    import torch
    n, c, h, w = (int(s) for s in x.shape)
    nb = len(filters)
    if nb != len(dilations):
        raise ValueError("one filter tensor per dilation")
    kk = int(filters[0].shape[2])
    k = int(round(kk ** 0.5))
    if k * k != kk:
        raise ValueError("filters must hold k*k taps")
    for f in filters:
        if tuple(f.shape) != (n, c, kk, h, w) or f.dtype != x.dtype:
            raise ValueError("filter %s %s does not match x" % (tuple(f.shape), f.dtype))
        _match(f, "filter", (n, c, kk, h, w), x)
    if tuple(dy.shape) != (n, nb * c, h, w) or dy.dtype != x.dtype:
        raise ValueError("dy %s %s does not match (n, nb*c, h, w)" % (tuple(dy.shape), dy.dtype))
    _match(dy, "dy", (n, nb * c, h, w), x)
    dx = None
    if need_dx:
        dx = out_dx if out_dx is not None else torch.empty_like(x)
        if tuple(dx.shape) != tuple(x.shape) or dx.dtype != x.dtype:
            raise ValueError("out_dx %s %s does not match x" % (tuple(dx.shape), dx.dtype))
        _match(dx, "out_dx", x.shape, x)
    dfs = None
    if need_dfilters:
        dfs = list(out_dfilters) if out_dfilters is not None else [torch.empty_like(f) for f in filters]
        if len(dfs) != nb:
            raise ValueError("one filter gradient per branch")
        for g, f in zip(dfs, filters):
            if g is not None and (tuple(g.shape) != tuple(f.shape) or g.dtype != f.dtype):
                raise ValueError("filter gradient %s %s does not match" % (tuple(g.shape), g.dtype))
            if g is not None:
                _match(g, "filter gradient", f.shape, x)
    fptrs = (_VP * nb)(*[_dev(f, "filter") for f in filters])
    dptrs = (_VP * nb)(*[_dev(g, "filter gradient") for g in dfs]) if dfs is not None else None
    dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
    _check(lib().dynconv_multidil_bwd(_dev(x, "x"), fptrs, _dev(dy, "dy"), dil, nb, _dev(dx, "dx"), dptrs,
                                      n, c, h, w, k, _dtype_code(x), _stream(x)), "dynconv_multidil_bwd")
    return dx, dfs


def _dyn_shapes(x, filters, dilations):
    n, c, h, w = (int(s) for s in x.shape)
    nb = len(filters)
    if nb != len(dilations):
        raise ValueError("one filter tensor per dilation")
    kk = int(filters[0].shape[2])
    k = int(round(kk ** 0.5))
    if k * k != kk:
        raise ValueError("filters must hold k*k taps")
    for f in filters:
        if tuple(f.shape) != (n, c, kk, h, w) or f.dtype != x.dtype:
            raise ValueError("filter %s %s does not match x" % (tuple(f.shape), f.dtype))
        _match(f, "filter", (n, c, kk, h, w), x)
    return n, c, h, w, nb, k


def dynconv_multidil_fwd_into(x, filters, y, channel_offset, dilations=(1, 3, 5)):
    """Write the branch outputs into channels [channel_offset, channel_offset + nb*c) of
    the caller's (n, C_total, h, w) tensor y; returns y."""
    n, c, h, w, nb, k = _dyn_shapes(x, filters, dilations)
    if y.dim() != 4 or (int(y.shape[0]), int(y.shape[2]), int(y.shape[3])) != (n, h, w) or y.dtype != x.dtype:
        raise ValueError("y %s %s does not match x" % (tuple(y.shape), y.dtype))
    _match(y, "y", y.shape, x)
    fptrs = (_VP * nb)(*[_dev(f, "filter") for f in filters])
    dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
    _check(lib().dynconv_multidil_fwd_into(_dev(x, "x"), fptrs, dil, nb, _dev(y, "y"), int(y.shape[1]),
                                           int(channel_offset), n, c, h, w, k, _dtype_code(x), _stream(x)),
           "dynconv_multidil_fwd_into")
    return y


def dynconv_multidil_bwd_from(x, filters, dy, channel_offset, dilations=(1, 3, 5), need_dx=True,
                              need_dfilters=True):
    """(dx, [dF_b]) with the branch gradients read from channels
    [channel_offset, channel_offset + nb*c) of the caller's (n, C_total, h, w) tensor dy."""
    import torch
    n, c, h, w, nb, k = _dyn_shapes(x, filters, dilations)
    if dy.dim() != 4 or (int(dy.shape[0]), int(dy.shape[2]), int(dy.shape[3])) != (n, h, w) or dy.dtype != x.dtype:
        raise ValueError("dy %s %s does not match x" % (tuple(dy.shape), dy.dtype))
    _match(dy, "dy", dy.shape, x)
    dx = torch.empty_like(x) if need_dx else None
    dfs = [torch.empty_like(f) for f in filters] if need_dfilters else None
    fptrs = (_VP * nb)(*[_dev(f, "filter") for f in filters])
    dptrs = (_VP * nb)(*[_dev(g, "filter gradient") for g in dfs]) if dfs is not None else None
    dil = (ctypes.c_int32 * nb)(*[int(d) for d in dilations])
    _check(lib().dynconv_multidil_bwd_from(_dev(x, "x"), fptrs, _dev(dy, "dy"), int(dy.shape[1]),
                                           int(channel_offset), dil, nb, _dev(dx, "dx"), dptrs, n, c, h, w, k,
                                           _dtype_code(x), _stream(x)), "dynconv_multidil_bwd_from")
    return dx, dfs


# ---------------------------------------------------------------- kernel selection
def dwconv2d_algo_candidates(pass_, x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=None):
    """Names of the kernel families that can run pass_ (0 fwd, 1 grad-input, 2 grad-weight)."""
    import torch
    code = _dtype_code(torch.empty(0, dtype=dtype or torch.float32))
    geo = _geo(x_shape, w_shape, stride, padding, dilation)
    names = (ctypes.c_char_p * 16)()
    cnt = lib().dwconv2d_algo_candidates(int(pass_), *geo, code, names, 16)
    if cnt < 0:
        _check(cnt, "dwconv2d_algo_candidates")
    return [names[i].decode() for i in range(min(cnt, 16))]


def dwconv2d_set_algo(pass_, x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=None, algo=None):
    """Record family `algo` for this geometry (None: back to the built-in choice)."""
    import torch
    code = _dtype_code(torch.empty(0, dtype=dtype or torch.float32))
    geo = _geo(x_shape, w_shape, stride, padding, dilation)
    _check(lib().dwconv2d_set_algo(int(pass_), *geo, code, algo.encode() if algo else None), "dwconv2d_set_algo")


def dwconv2d_tune_fwd(x, w, bias=None, stride=1, padding=0, dilation=1, out=None, reps=10):
    """Time every forward family on these tensors, record the fastest; returns its name."""
    import torch
    geo = _geo(x.shape, w.shape, stride, padding, dilation)
    oh, ow = dwconv2d_out_size(x.shape, w.shape, stride, padding, dilation)
    if out is None:
        out = torch.empty((geo[0], geo[4], oh, ow), dtype=x.dtype, device=x.device)
    _match(w, "w", w.shape, x)
    if bias is not None:
        _match(bias, "bias", (geo[4],), x)
    _match(out, "out", (geo[0], geo[4], oh, ow), x)
    chosen = ctypes.c_char_p()
    _check(lib().dwconv2d_tune_fwd(_dev(x, "x"), _dev(w, "w"), _dev(bias, "bias"), _dev(out, "out"), *geo,
                                   _dtype_code(x), int(reps), _stream(x), ctypes.byref(chosen)), "dwconv2d_tune_fwd")
    return chosen.value.decode()


def dwconv2d_tune_bwd_input(dy, w, x_shape, stride=1, padding=0, dilation=1, out=None, reps=10):
    """Time every grad-input family on these tensors, record the fastest; returns its name."""
    import torch
    geo = _geo(x_shape, w.shape, stride, padding, dilation)
    if out is None:
        out = torch.empty(tuple(int(s) for s in x_shape), dtype=dy.dtype, device=dy.device)
    oh, ow = dwconv2d_out_size(x_shape, w.shape, stride, padding, dilation)
    _match(dy, "dy", (geo[0], geo[4], oh, ow), dy)
    _match(w, "w", w.shape, dy)
    _match(out, "out", geo[:4], dy)
    chosen = ctypes.c_char_p()
    _check(lib().dwconv2d_tune_bwd_input(_dev(dy, "dy"), _dev(w, "w"), _dev(out, "out"), *geo, _dtype_code(dy),
                                         int(reps), _stream(dy), ctypes.byref(chosen)), "dwconv2d_tune_bwd_input")
    return chosen.value.decode()


def dwconv2d_tune_bwd_weight(x, dy, w_shape, stride=1, padding=0, dilation=1, with_bias=True, reps=10):
    """Time every grad-weight family on these tensors, record the fastest; returns its name."""
    import torch
    geo = _geo(x.shape, w_shape, stride, padding, dilation)
    oh, ow = dwconv2d_out_size(x.shape, w_shape, stride, padding, dilation)
    _match(dy, "dy", (geo[0], geo[4], oh, ow), x)
    out = torch.empty(tuple(int(s) for s in w_shape), dtype=x.dtype, device=x.device)
    ob = torch.empty((geo[4],), dtype=x.dtype, device=x.device) if with_bias else None
    nbytes = dwconv2d_bwd_weight_workspace_bytes(x.shape, w_shape, stride, padding, dilation, x.dtype)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    chosen = ctypes.c_char_p()
    _check(lib().dwconv2d_tune_bwd_weight(_dev(x, "x"), _dev(dy, "dy"), _dev(out, "out"), _dev(ob, "out_bias"),
                                          _dev(ws, "workspace"), nbytes, *geo, _dtype_code(x), int(reps), _stream(x),
                                          ctypes.byref(chosen)), "dwconv2d_tune_bwd_weight")
    return chosen.value.decode()
