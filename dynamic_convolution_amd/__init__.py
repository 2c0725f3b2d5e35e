"""MI355X (gfx950) depthwise and dynamic-filter convolution.

The computation runs in hand-written HIP kernels behind the C ABI of
include/dwconv.h (libdwconv.so, built in-tree by ``build.build()``); this
package only marshals torch tensors into that ABI.  The functions carry the
ABI's names:

    dwconv2d_fwd(x, w, bias=None, stride=1, padding=0, dilation=1)
    dwconv2d_bwd_input(dy, w, x_shape, stride=1, padding=0, dilation=1)
    dwconv2d_bwd_weight(x, dy, w_shape, stride=1, padding=0, dilation=1, with_bias=True)
    dwconv2d_bwd_weight_noalloc(x, dy, w_shape, stride=1, padding=0, dilation=1, with_bias=True)
        (same result; partial sums in the library's fixed device scratch, no allocation)
    dynconv_multidil_fwd(x, filters, dilations=(1, 3, 5))
    dynconv_multidil_bwd(x, filters, dy, dilations=(1, 3, 5), need_dx=True, need_dfilters=True)
    dynconv_multidil_fwd_into(x, filters, y, channel_offset, dilations=(1, 3, 5))
    dynconv_multidil_bwd_from(x, filters, dy, channel_offset, dilations=(1, 3, 5))
    dwconv2d_out_size(x_shape, w_shape, stride=1, padding=0, dilation=1)
    dwconv2d_bwd_weight_workspace_bytes(x_shape, w_shape, stride, padding, dilation, dtype)
    dwconv2d_algo_candidates / dwconv2d_set_algo / dwconv2d_tune_{fwd,bwd_input,bwd_weight}
        (per-geometry kernel selection, measured on the device)
"""
from ._native import (  # noqa: F401
    DwconvError,
    dwconv2d_algo,
    dwconv2d_algo_candidates,
    dwconv2d_bwd_input,
    dwconv2d_bwd_weight,
    dwconv2d_bwd_weight_noalloc,
    dwconv2d_bwd_weight_workspace_bytes,
    dwconv2d_fwd,
    dwconv2d_out_size,
    dwconv2d_set_algo,
    dwconv2d_tune_bwd_input,
    dwconv2d_tune_bwd_weight,
    dwconv2d_tune_fwd,
    dynconv_multidil_bwd,
    dynconv_multidil_bwd_from,
    dynconv_multidil_fwd,
    dynconv_multidil_fwd_into,
    lib,
    status_str,
)
