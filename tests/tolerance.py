"""Parity bar between the HIP path and the fp64 oracle.

Elementwise |gpu - oracle| <= atol + rtol * |oracle| with
  fp32:        rtol = 1e-5
  fp16, bf16:  rtol = 1e-2
  atol = 1e-4 * sqrt(L) for every dtype, L = number of products summed into
  the element: kh*kw (forward), M*kh*kw (grad-input), n*oh*ow (grad-weight and
  grad-bias), k*k (dynamic filter).
The 16-bit outputs are rounded once to the I/O type (relative error <= 2^-9)
on top of fp32 accumulation, so rtol 1e-2 covers them; the absolute floor
covers fp32 accumulation error at outputs near zero.
"""
import math

import numpy as np
import torch


def rtol_for(dtype) -> float:
    return 1e-5 if dtype == torch.float32 else 1e-2


def assert_close(got_t, want, L, dtype, what=""):
    got = got_t.detach().float().cpu().double().numpy() if hasattr(got_t, "detach") else np.asarray(got_t)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    atol = 1e-4 * math.sqrt(max(L, 1))
    lim = atol + rtol_for(dtype) * np.abs(want)
    err = np.abs(got - want)
    bad = ~(err <= lim)  # NaN counts as bad
    if bad.any():
        ratio = np.where(np.isfinite(err), err / lim, np.inf)
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: got %r want %r (err/tol %.3g)"
                             % (what, int(bad.sum()), bad.size, i, got[i], want[i], ratio[i]))
    return float(np.max(err / lim)) if err.size else 0.0
