"""Seeded synthetic inputs shaped like the workloads the pages measure.

This module holds no convolution arithmetic: it only draws random tensors.
Both the HIP path (tests, bench) and the CPU oracle consume the very same
tensors it returns, so it is the one module the two sides share.

Every tensor is drawn in fp32 by a torch generator seeded with
``seed * 16 + OFFSET[name]`` and then rounded to the requested dtype (round to
nearest even), so the dtype variants of one case round the same draws.
Distributions are written ``("U", a, b)`` (uniform on [a, b)) or
``("N", mean, variance)``.
"""
from __future__ import annotations

import math

import torch

OFFSET = {"x": 0, "w": 1, "b": 2, "dy": 3, "f0": 4, "f1": 5, "f2": 6, "f3": 7}


def draw(shape, dist, seed: int, name: str, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """A seeded random tensor of `shape` from distribution `dist`, rounded to `dtype`."""
    g = torch.Generator(device=device).manual_seed(int(seed) * 16 + OFFSET[name])
    kind, p, q = dist
    shape = tuple(int(s) for s in shape)
    if kind == "U":
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (q - p) + p
    elif kind == "N":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * math.sqrt(q) + p
    else:
        raise ValueError("unknown distribution %r" % (kind,))
    return t.to(dtype)


# The five workload families (shapes and value distributions), as data.
TINY = dict(n=1, c=8, h=16, k=3, stride=1, pad=1, dil=1, mult=1, dtype="f32",
            x=("U", -1.0, 1.0), w=("N", 0.0, 1.0 / 9), b=("U", -0.1, 0.1), dy=("N", 0.0, 1.0))

MOBILENET_LAYERS = [(32, 112), (64, 112), (128, 56), (256, 28), (512, 14), (1024, 7)]
MOBILENET = dict(batches=(1, 64, 128), layers=MOBILENET_LAYERS, strides=(1, 2), k=3, pad=1, dil=1,
                 dtype="f32", x=("U", 0.0, 1.0), w=("N", 0.0, 2.0 / 9), dy=("N", 0.0, 1.0))

MULT_DIL = dict(n=128, c=256, mult=2, h=56, k=5, stride=2, pad=4, dil=2, dtype="bf16",
                x=("N", 0.0, 1.0), w=("N", 0.0, 1.0 / 25), dy=("N", 0.0, 1.0))

LARGE_K = dict(n=64, c=384, hs=(32, 48, 64), ks=(7, 13, 31), dtypes=("f32", "f16"),
               x=("N", 0.0, 1.0), dy=("N", 0.0, 1.0))  # w ~ N(0, 1/k^2), pad k//2

DYNAMIC = dict(batches=(1, 2), c=64, hs=(128, 256), k=3, dilations=(1, 3, 5),
               dtypes=("f32", "f16", "bf16"), x=("N", 0.0, 1.0), f=("N", 0.0, 1.0 / 9),
               dy=("N", 0.0, 1.0))  # dy: the output gradient of the backward

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
