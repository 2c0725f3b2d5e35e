"""Benchmark of the depthwise / dynamic-filter hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload all|largek|mobilenet|multdil|dynamic|tiny]

Prints ONE JSON line.  The headline is the large-kernel workload (the largest
configuration: N=64, C=384, H in {32,48,64}, k in {7,13,31}, fp32 and fp16,
forward + grad-input + grad-weight; valid-tap GFLOP/s).  With the default
``--workload all`` the same line carries the other workloads as sub-records
under ``workloads`` (each with its own roofline, per-case table and CPU
baseline):

  largek     N=64, C=384, H in {32,48,64}, k in {7,13,31}, pad k//2, fp32 and fp16
  mobilenet  3x3 depthwise layers of MobileNet, N in {1, 64, 128}, (C, H) in
             {(32,112), (64,112), (128,56), (256,28), (512,14), (1024,7)}, stride 1
             and 2, pad 1, fp32 (36 cases x 3 passes)
  multdil    multiplier 2, dilation 2, stride 2, 5x5, pad 4, N=128, C=256->512,
             56x56, bf16
  dynamic    per-pixel 3x3 filters at dilations 1/3/5, N in {1,2}, C=64,
             H in {128,256}, fp32/fp16/bf16, forward and backward
  tiny       N=1, C=8, 16x16, 3x3, fp32: latency of each pass

A step is one pass of every entry point the workload uses over every case,
pass-major (every forward, then every grad-input, then every grad-weight), with
inputs resident in HBM.  The whole step is captured once into one HIP graph
and replayed (--eager: call by call).  A workload whose step moves less than
2 GiB gets identical copies of its tensors and step i uses copy i % copies, so
no launch finds its inputs in the 256 MB last-level cache.

value        algorithmic work of one step per second: valid-tap flops (2 per
             in-bounds multiply-add) for largek, compulsory bytes (each input
             element the result depends on once, each output once) for the
             bandwidth-bound workloads; the K timed steps after W warmup steps
step_timing  the K-step timing repeated --repeats times (median, mean, std, min;
             the first is the one `value` reports)
roofline     the dominant kernel tag (most event time): algorithmic bytes or flops
             per launch over its average launch duration (HIP events on the
             launch stream around a graph of back-to-back rounds of its calls,
             >= 1 GiB of traffic per replay), repeated --repeats times (median
             reported) against the MI355X peak for that tag's arithmetic
             (HBM 8 TB/s; fp32 157.3 TFLOP/s; fp16/bf16 matrix cores 2.5 PFLOP/s).
             step_frac: the whole step's rate against the same peak.
             ceiling: the same launch against what this GPU was measured to
             reach in the same run (libdwprobe.so): 16-byte nontemporal
             copy / read / write streams for bandwidth-bound tags (mixed by the
             tag's read share of its bytes), the fp32 or fp16 matrix-instruction
             rate, or the fp32 vector FMA rate for the tag's arithmetic.
per_case     each call alone and cold (after a 512 MiB fill that evicts the last-level
             cache): HIP events around one eager call, median of --repeats, its
             rate and fraction of roofline, and the oracle's time for the same call
             (scaled from the CPU sample) over it.  Calls whose roofline time is
             under 5 us are flagged as latency-bound (their figure is a latency);
             their kernel tags carry a ".lat" suffix, so per_kernel and the
             dominant-tag roofline keep them apart from the batched launches.
cpu_baseline the fp64 CPU oracle on a bounded sample of the same host tensors,
             on all host threads and on one thread (channel subset), with the
             host CPU model
input_sha256 SHA-256 of every input tensor (first 16 hex digits) and of their list
gpu_clocks   shader / memory clock read from sysfs before and after the timed region
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import gc
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
FP32_PEAK_TFLOPS = 157.3        # MI355X published fp32 peak (vector and matrix)
F16_MATRIX_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix-core peak
LATENCY_US = 5.0                # calls whose roofline time is below this are latency-bound
WORKLOADS = ["largek", "mobilenet", "multdil", "dynamic", "tiny"]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all"] + WORKLOADS)
    ap.add_argument("--repeats", type=int, default=5, help="repeats of each timed measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target oracle time (all threads) for the headline's CPU baseline; sub-records use half")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
    ap.add_argument("--no-hash", action="store_true", help="skip the SHA-256 of the inputs")
    ap.add_argument("--eager", action="store_true", help="launch call by call instead of replaying HIP graphs")
    ap.add_argument("--tune", action="store_true",
                    help="before timing, let the library time every kernel family that can run each call's "
                         "geometry and keep the fastest (its selection table)")
    ap.add_argument("--only-tag", default=None, help="run only the calls of this kernel tag (for counter runs)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/traffic_<--only-tag>.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--launches", type=int, default=0,
                    help="calls of the tag in the counter runs (0: the largest dispatch count of one of "
                         "its kernels, right when every call launches each kernel once; give it when the "
                         "tag's cases launch different instantiations)")
    ap.add_argument("--cmd", default="", help="command recorded with the traffic figures")
    return ap.parse_args(argv)


# ---------------------------------------------------------------- accounting
def read_extent(in_n, out_n, k, s, p, d):
    """How many input rows (or cols) some tap of some output position reads."""
    seen = set()
    for o in range(out_n):
        for i in range(k):
            h = o * s - p + i * d
            if 0 <= h < in_n:
                seen.add(h)
    return len(seen)


def valid_taps(in_n, out_n, k, s, p, d):
    """Sum over output positions of the in-bounds tap count along one axis."""
    tot = 0
    for o in range(out_n):
        for i in range(k):
            h = o * s - p + i * d
            tot += 0 <= h < in_n
    return tot


# kernel families that run 16-bit I/O on the matrix cores (tag infixes)
MATRIX16_FAMILIES = (".largek_mfma.", ".largek_mfma_h16.", ".largek_roll16.")
MATRIX32_FAMILIES = (".largek_mfma_f32.", ".largek_mfma_t16.", ".largek_roll_f32.")


def tag_peak(tag, kind):
    """(bound, peak, unit) of a kernel tag: HBM for bandwidth-bound workloads; for
    flop-counted ones the matrix-core peak of 16-bit I/O on the matrix cores, the
    fp32 matrix peak of fp32 matrix families, else the fp32 vector peak (the two
    fp32 peaks are the same figure)."""
    if kind == "bytes":
        return "hbm", HBM_PEAK_GBS, "GB/s"
    if any(f in tag for f in MATRIX16_FAMILIES) and not tag.endswith("_f32"):
        return "mfma", F16_MATRIX_PEAK_TFLOPS, "TFLOP/s"
    if any(f in tag for f in MATRIX32_FAMILIES):
        return "mfma", FP32_PEAK_TFLOPS, "TFLOP/s"
    return "alu", FP32_PEAK_TFLOPS, "TFLOP/s"


class Call:
    """One entry-point call of the step: its tag (pass.family.geometry), algorithmic
    bytes and flops, the case it belongs to, and (static passes) a tuner."""

    def __init__(self, tag, fn, nbytes, flops, case, pass_, tune=None, rbytes=None):
        self.tag, self.fn, self.nbytes, self.flops, self.tune = tag, fn, nbytes, flops, tune
        self.case, self.pass_ = case, pass_
        self.rbytes = nbytes if rbytes is None else rbytes  # bytes read (the rest are written)


def static_calls(dc, case, dev, seed, passes=("fwd", "bwd_in", "bwd_w")):
    import torch
    from dynamic_convolution_amd import synth
    n, c, h, M, k, s, p, d, dtype, dists, label, with_bias = case
    e = torch.empty(0, dtype=dtype).element_size()
    x = synth.draw((n, c, h, h), dists["x"], seed, "x", dtype, device=dev)
    w = synth.draw((c * M, k, k), dists["w"], seed, "w", dtype, device=dev)
    b = synth.draw((c * M,), ("U", -0.1, 0.1), seed, "b", dtype, device=dev) if with_bias else None
    oh, ow = dc.dwconv2d_out_size(x.shape, w.shape, s, p, d)
    dy = synth.draw((n, c * M, oh, ow), dists["dy"], seed, "dy", dtype, device=dev)
    y = torch.empty((n, c * M, oh, ow), dtype=dtype, device=dev)
    dx = torch.empty_like(x)
    gw = torch.empty_like(w)
    gb = torch.empty((c * M,), dtype=dtype, device=dev) if with_bias else None
    ws = torch.empty((dc.dwconv2d_bwd_weight_workspace_bytes(x.shape, w.shape, s, p, d, dtype),),
                     dtype=torch.uint8, device=dev)
    rows = read_extent(h, oh, k, s, p, d)
    sx = n * c * rows * rows * e
    X, W, B, Y = x.numel() * e, w.numel() * e, (c * M * e if with_bias else 0), y.numel() * e
    macs = n * c * M * valid_taps(h, oh, k, s, p, d) ** 2
    calls = []
    dts = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[dtype]

    def tag(pi, name, nbytes=None):
        # one tag = one kernel instantiation: the library's algorithm for this geometry,
        # plus the template parameters it is specialised on; calls whose HBM time at
        # the peak is under LATENCY_US get their own ".lat" tag (a latency, not a rate)
        algo = dc.dwconv2d_algo(pi, x.shape, w.shape, s, p, d, dtype)
        t = "%s.%s.k%d_s%d_m%d_%s" % (name, algo, k, s, M, dts)
        if nbytes is not None and nbytes / (HBM_PEAK_GBS * 1e9) * 1e6 < LATENCY_US and 2 * macs < 1e9:
            t += ".lat"
        return t

    if "fwd" in passes:
        calls.append(Call(tag(0, "fwd", sx + W + B + Y), lambda: dc.dwconv2d_fwd(x, w, b, s, p, d, out=y),
                          sx + W + B + Y, 2 * macs,
                          label, "fwd", lambda: dc.dwconv2d_tune_fwd(x, w, b, s, p, d, out=y, reps=5),
                          rbytes=sx + W + B))
    if "bwd_in" in passes:
        calls.append(Call(tag(1, "bwd_input", Y + W + X),
                          lambda: dc.dwconv2d_bwd_input(dy, w, x.shape, s, p, d, out=dx),
                          Y + W + X, 2 * macs, label, "bwd_input",
                          lambda: dc.dwconv2d_tune_bwd_input(dy, w, x.shape, s, p, d, out=dx, reps=5),
                          rbytes=Y + W))
    if "bwd_w" in passes:
        calls.append(Call(tag(2, "bwd_weight", sx + Y + W + B),
                          lambda: dc.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d, with_bias=with_bias, out=gw,
                                                         out_bias=gb, workspace=ws),
                          sx + Y + W + B, 2 * macs, label, "bwd_weight",
                          lambda: dc.dwconv2d_tune_bwd_weight(x, dy, w.shape, s, p, d, with_bias=with_bias, reps=5),
                          rbytes=sx + Y))
    tensors = dict(x=x, w=w, b=b, dy=dy, y=y, dx=dx, gw=gw, gb=gb)
    inputs = {"x": x, "w": w, "dy": dy}
    if b is not None:
        inputs["b"] = b
    return calls, tensors, inputs


def build_workload(name, dc, dev):
    """dict(cases, per_case=[(calls, tensors, inputs)], calls (pass-major), desc, dtype, kind, cfg)."""
    import torch
    from dynamic_convolution_amd import synth
    cases = []
    if name == "mobilenet":
        m = synth.MOBILENET
        dists = dict(x=m["x"], w=m["w"], dy=m["dy"])
        seed = 100
        for n in m["batches"]:
            for c, h in m["layers"]:
                for s in m["strides"]:
                    cases.append(((n, c, h, 1, 3, s, 1, 1, torch.float32, dists,
                                   "N%d_C%d_H%d_3x3_s%d_f32" % (n, c, h, s), False), seed))
                    seed += 1
        desc = "mobilenet_dw3x3_sweep"
        dt, kind = "f32", "bytes"
        cfg = {"batches": list(m["batches"]), "layers_c_h": [list(l) for l in m["layers"]],
               "strides": list(m["strides"]), "kernel": 3, "pad": 1, "passes": ["fwd", "bwd_input", "bwd_weight"]}
    elif name == "multdil":
        m = synth.MULT_DIL
        dists = dict(x=m["x"], w=m["w"], dy=m["dy"])
        cases.append(((m["n"], m["c"], m["h"], m["mult"], m["k"], m["stride"], m["pad"], m["dil"],
                       torch.bfloat16, dists, "N128_C256x2_H56_5x5_s2_d2_bf16", False), 200))
        desc, dt, kind = "mult2_dil2_stride2_5x5", "bf16", "bytes"
        cfg = {"n": m["n"], "c_in": m["c"], "c_out": m["c"] * m["mult"], "hw": m["h"], "kernel": 5, "stride": 2,
               "pad": 4, "dilation": 2, "passes": ["fwd", "bwd_input", "bwd_weight"]}
    elif name == "largek":
        L = synth.LARGE_K
        seed = 300
        for h in L["hs"]:
            for k in L["ks"]:
                for dts in L["dtypes"]:
                    dists = dict(x=L["x"], w=("N", 0.0, 1.0 / k ** 2), dy=L["dy"])
                    cases.append(((L["n"], L["c"], h, 1, k, 1, k // 2, 1, synth.DTYPES[dts], dists,
                                   "N64_C384_H%d_k%d_%s" % (h, k, dts), False), seed))
                    seed += 1
        desc, dt, kind = "large_kernel_dw_n64_c384", "f32+f16", "flops"
        cfg = {"n": L["n"], "c": L["c"], "hw": list(L["hs"]), "kernels": list(L["ks"]), "dtypes": list(L["dtypes"]),
               "passes": ["fwd", "bwd_input", "bwd_weight"]}
    elif name == "tiny":
        t = synth.TINY
        cases.append(((t["n"], t["c"], t["h"], 1, t["k"], t["stride"], t["pad"], t["dil"], torch.float32,
                       dict(x=t["x"], w=t["w"], dy=t["dy"]), "N1_C8_H16_3x3_s1_f32", True), 1))
        desc, dt, kind = "tiny_dw3x3_n1_c8_16x16", "f32", "bytes"
        cfg = {"n": 1, "c": 8, "hw": 16, "kernel": 3, "pad": 1, "passes": ["fwd", "bwd_input", "bwd_weight"]}
    else:
        return build_dynamic(dc, dev)
    per_case = [static_calls(dc, cs, dev, seed) for cs, seed in cases]
    # pass-major; within a pass, calls of one kernel geometry (tag) are adjacent
    calls = []
    for pi in range(3):
        tags = {}
        for cls, _t, _i in per_case:
            for cl in cls[pi:pi + 1]:
                tags.setdefault(cl.tag, []).append(cl)
        for cl_list in tags.values():
            calls.extend(cl_list)
    return dict(cases=cases, per_case=per_case, calls=calls, desc=desc, dtype=dt, kind=kind, cfg=cfg)


def build_dynamic(dc, dev):
    """Forward and backward of the fused dynamic filter over the workload's cases.

    Compulsory bytes per call (each input element the result depends on once,
    each output element once): forward |x| + in-bounds filter taps + |y|;
    backward |x| + |dy| + in-bounds filter taps (read for dx) + |dx| + every
    filter-gradient element (written, zero for taps outside the image).
    """
    import torch
    from dynamic_convolution_amd import synth
    D = synth.DYNAMIC
    fwd, bwd, per_case, cases = [], [], [], []
    seed = 400
    for n in D["batches"]:
        for h in D["hs"]:
            for dts in D["dtypes"]:
                dtype = synth.DTYPES[dts]
                e = torch.empty(0, dtype=dtype).element_size()
                c = D["c"]
                x = synth.draw((n, c, h, h), D["x"], seed, "x", dtype, device=dev)
                fs = [synth.draw((n, c, 9, h, h), D["f"], seed, "f%d" % i, dtype, device=dev) for i in range(3)]
                dy = synth.draw((n, 3 * c, h, h), D["dy"], seed, "dy", dtype, device=dev)
                y = torch.empty((n, 3 * c, h, h), dtype=dtype, device=dev)
                dx = torch.empty_like(x)
                dfs = [torch.empty_like(f) for f in fs]
                taps = sum(valid_taps(h, h, 3, 1, dd, dd) ** 2 for dd in D["dilations"])
                X, Y, TF = x.numel() * e, y.numel() * e, n * c * taps * e
                FF = sum(f.numel() for f in fs) * e
                label = "N%d_C%d_H%d_%s" % (n, c, h, dts)
                cf_ = Call("dyn.fused.k3_%s" % dts,
                           (lambda x=x, fs=fs, y=y: dc.dynconv_multidil_fwd(x, fs, D["dilations"], out=y)),
                           X + TF + Y, 2 * n * c * taps, label, "fwd", rbytes=X + TF)
                cb = Call("dyn_bwd.fused.k3_%s" % dts,
                          (lambda x=x, fs=fs, dy=dy, dx=dx, dfs=dfs:
                           dc.dynconv_multidil_bwd(x, fs, dy, D["dilations"], out_dx=dx, out_dfilters=dfs)),
                          X + Y + TF + X + FF, 3 * n * c * taps, label, "bwd", rbytes=X + Y + TF)
                fwd.append(cf_)
                bwd.append(cb)
                inputs = {"x": x, "dy": dy}
                inputs.update({"f%d" % i: f for i, f in enumerate(fs)})
                per_case.append(([cf_, cb], dict(x=x, fs=fs, y=y, dy=dy, dx=dx, dfs=dfs), inputs))
                cases.append(((n, c, h, dts), seed))
                seed += 1
    cfg = {"batches": list(D["batches"]), "c": D["c"], "hw": list(D["hs"]), "k": 3, "dilations": list(D["dilations"]),
           "dtypes": list(D["dtypes"]), "passes": ["fwd", "bwd (dx and filter gradients)"]}
    return dict(cases=cases, per_case=per_case, calls=fwd + bwd, desc="dynamic_multidil_3x3_d135", dtype="f32+f16+bf16",
                kind="bytes", cfg=cfg)


def device_ceilings(dev, nbytes=1 << 30, reps=5):
    """What this GPU reaches in this run, measured with libdwprobe.so: GB/s of
    16-byte nontemporal copy (read + write bytes), read-only and write-only
    streams over `nbytes` buffers, and TFLOP/s of fp32 and fp16 matrix
    instructions and fp32 vector FMAs; median of `reps` launches each.
    None when the probe library is not built."""
    import ctypes
    import torch
    from dynamic_convolution_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    L = ctypes.CDLL(B.PROBE_LIB)
    L.dw_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.dw_probe_stream.restype = ctypes.c_int
    L.dw_probe_compute.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.dw_probe_compute.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    word = torch.zeros(4, dtype=torch.int32, device=dev)

    def timed(launch):
        launch()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return statistics.median(ts)

    out = {}
    for name, kind, moved in (("copy_gbs", 0, 2 * nbytes), ("read_gbs", 1, nbytes), ("write_gbs", 2, nbytes)):
        def launch(kind=kind):
            rc = L.dw_probe_stream(kind, src.data_ptr(), dst.data_ptr(), nbytes, word.data_ptr(), sp)
            if rc != 0:
                raise RuntimeError("dw_probe_stream failed: %d" % rc)
        out[name] = round(moved / timed(launch) / 1e9, 1)
    del src, dst
    blocks, iters = 4096, 512
    buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for name, kind, it in (("mfma_f32_tflops", 0, iters), ("mfma_f16_tflops", 1, iters),
                           ("valu_fma_f32_tflops", 2, 8 * iters)):
        fl = ctypes.c_double()

        def launch(kind=kind, it=it):
            rc = L.dw_probe_compute(kind, buf.data_ptr(), blocks, it, ctypes.byref(fl), sp)
            if rc != 0:
                raise RuntimeError("dw_probe_compute failed: %d" % rc)
        sec = timed(launch)
        out[name] = round(fl.value / sec / 1e12, 1)
    return out


def ceiling_of(tag, kind, rfrac, ceil):
    """(value, unit, basis) of the measured ceiling for a tag: bandwidth-bound
    tags interpolate linearly in their read share between the write-only
    (0), copy (1/2) and read-only (1) stream rates; flop-counted tags take the
    matrix or vector rate of their arithmetic."""
    if not ceil:
        return None
    if kind == "bytes":
        if rfrac >= 0.5:
            v = ceil["copy_gbs"] + (ceil["read_gbs"] - ceil["copy_gbs"]) * (rfrac - 0.5) / 0.5
        else:
            v = ceil["write_gbs"] + (ceil["copy_gbs"] - ceil["write_gbs"]) * rfrac / 0.5
        return v, "GB/s", "stream (read share %.2f)" % rfrac
    if any(f in tag for f in MATRIX16_FAMILIES) and not tag.endswith("_f32"):
        return ceil["mfma_f16_tflops"], "TFLOP/s", "fp16 matrix instructions"
    if any(f in tag for f in MATRIX32_FAMILIES):
        return ceil["mfma_f32_tflops"], "TFLOP/s", "fp32 matrix instructions"
    return ceil["valu_fma_f32_tflops"], "TFLOP/s", "fp32 vector FMA"


def tag_ceiling(tag, r, kind, ceil):
    """The measured ceiling of one tag's rate in the step and the fraction reached."""
    cv = ceiling_of(tag, kind, r["rbytes"] / max(1, r["bytes"]), ceil)
    if cv is None:
        return {}
    rate = (r["bytes"] / (r["ms"] / 1e3) / 1e9) if kind == "bytes" else (r["flops"] / (r["ms"] / 1e3) / 1e12)
    return {"ceiling": round(cv[0], 1), "frac_of_ceiling": round(rate / cv[0], 4)}


# ---------------------------------------------------------------- host facts
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_clocks():
    """Current shader and memory clocks (MHz) from the amdgpu sysfs DPM tables, or None."""
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for key, fname in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
            try:
                with open(os.path.join(dev, fname)) as f:
                    for line in f:
                        if line.strip().endswith("*"):
                            out.setdefault(key, []).append(int(line.split(":")[1].strip().lower()
                                                               .split("mhz")[0]))
            except (OSError, ValueError, IndexError):
                continue
    return out or None


def input_digests(wl):
    """SHA-256 of every input tensor of the workload (host copy of its bytes), computed on a
    thread pool; (list of [case, tensor, first 16 hex digits], digest of the list)."""
    import torch
    items = []
    for (_calls, _t, inputs), (cs, _seed) in zip(wl["per_case"], wl["cases"]):
        label = _calls[0].case
        for nm, t in inputs.items():
            items.append((label, nm, t))

    def digest(t):
        a = t.detach().contiguous().view(torch.uint8).cpu().numpy()
        return hashlib.sha256(memoryview(a)).hexdigest()

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        hexes = list(ex.map(lambda it: digest(it[2]), items))
    rows = [[lab, nm, hx[:16]] for (lab, nm, _t), hx in zip(items, hexes)]
    total = hashlib.sha256("".join(hexes).encode()).hexdigest()
    return {"per_tensor": rows, "all": total[:32], "count": len(rows)}


# ---------------------------------------------------------------- CPU baseline
def oracle_inputs(wl, case_idx, nimg, chans):
    """fp64 host copies of a case's inputs restricted to images [0, nimg) and the given
    channels (None: all); returns (arrays, fraction of the case's work they cover)."""
    import numpy as np
    import torch
    _calls, t, _inputs = wl["per_case"][case_idx]
    cs = wl["cases"][case_idx][0]

    def f64(a):
        return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())

    n, c = t["x"].shape[:2]
    sl = min(nimg, n)
    ch = chans if chans is not None else list(range(c))
    frac = sl / n * len(ch) / c
    if "fs" in t:  # dynamic (channels independent)
        nb = len(t["fs"])
        dy = t["dy"][:sl].reshape(sl, nb, c, *t["dy"].shape[2:])[:, :, ch]
        return dict(x=f64(t["x"][:sl][:, ch]), fs=[f64(f[:sl][:, ch]) for f in t["fs"]],
                    dy=f64(dy.reshape(sl, nb * len(ch), *t["dy"].shape[2:]))), frac
    M = cs[3]
    och = [g * M + m for g in ch for m in range(M)]
    return dict(x=f64(t["x"][:sl][:, ch]), w=f64(t["w"][och]), dy=f64(t["dy"][:sl][:, och])), frac


def oracle_call(O, wl, case_idx, cl, arrs):
    """Seconds the oracle takes for one call on the given inputs."""
    if "fs" in arrs:
        t0 = time.perf_counter()
        if cl.pass_ == "fwd":
            O.dynconv_multidil_fwd(arrs["x"], arrs["fs"], (1, 3, 5))
        else:
            O.dynconv_multidil_bwd(arrs["x"], arrs["fs"], arrs["dy"], (1, 3, 5))
        return time.perf_counter() - t0
    n, c, h, M, k, s, p, d = wl["cases"][case_idx][0][:8]
    x, w, dy = arrs["x"], arrs["w"], arrs["dy"]
    t0 = time.perf_counter()
    if cl.pass_ == "fwd":
        O.dwconv2d_fwd(x, w, None, s, p, d)
    elif cl.pass_ == "bwd_input":
        O.dwconv2d_bwd_input(dy, w, x.shape, s, p, d)
    else:
        O.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d, with_bias=False)
    return time.perf_counter() - t0


def cpu_baseline(wl, target_s):
    """The oracle as it stands, timed on this host: (record, per-call full-batch time estimates).

    All threads: every call on a batch slice (the whole batch when it fits target_s,
    repeated passes when the whole workload takes under half of it).  One thread: every
    call on one image and a channel subset that holds channels 0 and C-1 (work is linear
    in images and channels, so rates compare directly)."""
    from oracle import oracle as O
    kind = wl["kind"]
    idx = [(ci, cl) for ci, (calls, _t, _i) in enumerate(wl["per_case"]) for cl in calls]
    threads = O.num_threads()

    def units(cl):
        return cl.nbytes if kind == "bytes" else cl.flops

    def run(nimg, chans_of=None):
        """Every call once on the sample; a call under 1 s is run three times and its
        fastest run kept (the first run of a call also pays for first-touching the
        oracle's freshly allocated outputs)."""
        tot_u = tot_t = spent = 0.0
        per = {}
        cached = (None, None, None)
        for ci, cl in idx:
            if cached[0] != ci:  # one case's host copies at a time
                cached = (None, None, None)
                arrs, frac = oracle_inputs(wl, ci, nimg, chans_of(ci) if chans_of else None)
                cached = (ci, arrs, frac)
            _ci, arrs, frac = cached
            sec = oracle_call(O, wl, ci, cl, arrs)
            spent += sec
            if sec < 1.0:
                for _ in range(2):
                    s2 = oracle_call(O, wl, ci, cl, arrs)
                    spent += s2
                    sec = min(sec, s2)
            tot_t += sec
            tot_u += units(cl) * frac
            per[id(cl)] = sec / frac  # seconds for the whole call
        return tot_u, tot_t, per, spent

    u1, t1, per, spent = run(1)
    ns = 1
    if 0 < spent < target_s:
        ns = max(1, min(128, int(target_s / spent)))
        if ns > 1:
            u1, t1, per, spent = run(ns)
    whole = all(ns >= t["x"].shape[0] for _c, t, _i in wl["per_case"])
    est = per
    used = max(min(ns, t["x"].shape[0]) for _c, t, _i in wl["per_case"])
    what = "every case's whole batch" if whole else "first %d image(s) of every case's batch" % used
    unit = "GB/s" if kind == "bytes" else "GFLOP/s"
    rec = {"value": round(u1 / t1 / 1e9, 4), "unit": unit, "cores": threads, "kind": "oracle",
           "sample": "%s, every pass (a call under 1 s: fastest of 3), same host tensors; %.1f s of oracle "
                     "time counted, %.1f s spent" % (what, t1, spent),
           "cpu_model": cpu_model()}
    # one thread: one image, a channel subset holding 0 and C-1
    try:
        O.set_threads(1)

        def subset(ci):
            c = wl["per_case"][ci][1]["x"].shape[1]
            step = max(1, c // 16)
            return sorted(set(list(range(0, c, step)) + [c - 1]))
        u, t_, _, _sp = run(1, subset)
        rec["one_thread"] = {"value": round(u / t_ / 1e9, 4), "unit": unit, "cores": 1,
                             "sample": "first image, every 1/16th channel (and the last) of every case, every pass "
                                       "(a call under 1 s: fastest of 3); %.1f s of oracle time" % t_}
    finally:
        O.set_threads(threads)
    return rec, est


# ---------------------------------------------------------------- traffic from committed counters
COPY_REF_BYTES = 256 << 20  # bytes read (and written) by one reference copy


def kernel_sources_sha256():
    """Hash of every kernel source: counters are valid only for the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_convolution_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(tag):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % tag.replace("/", "_"))


def committed_traffic(tag):
    """HBM bytes per launch from profiles/traffic_<tag>.json when the kernel sources are unchanged."""
    path = traffic_path(tag)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_sources_sha256():
        return None
    return rec.get("bytes_per_launch")


def read_counter_csv(path, counter):
    """Per-dispatch (kernel name, value) of one counter from a rocprofv3 counter_collection.csv,
    in dispatch order."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((int(r.get("Dispatch_Id") or 0), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort(key=lambda t: t[0])
    return [(name, v) for _d, name, v in rows]


def traffic_from(fetch_csv, write_csv, tag, launches, cmd):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of this library's kernels by the
    reference copy's reading and write profiles/traffic_<tag>.json."""
    out = {"tag": tag, "source_sha256": kernel_sources_sha256(), "command": cmd}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = read_counter_csv(path, counter)
        mine = [v for name, v in rows if "dw::" in name]
        # the reference copies are the first three copy dispatches after this library's
        # last kernel (--copy-ref runs them after everything else; earlier copies are the
        # inputs' dtype conversions)
        last = max((i for i, (name, _v) in enumerate(rows) if "dw::" in name), default=-1)
        refs = [v for name, v in rows[last + 1:] if "dw::" not in name and "copy" in name.lower()][:3]
        if not mine or not refs:
            raise SystemExit("no %s rows for this library or the reference copy in %s" % (counter, path))
        if launches <= 0:
            # each call of a tag launches each of its kernels once: the number of
            # calls is the dispatch count of any of this library's kernels
            counts = {}
            for name, _v in rows:
                if "dw::" in name:
                    counts[name] = counts.get(name, 0) + 1
            launches = max(counts.values())
        ref_kib = sum(refs) / len(refs)
        scale = (COPY_REF_BYTES / 1024.0) / ref_kib
        out[key + "_kib_raw"] = sum(mine)
        out[key + "_ref_copy_kib"] = ref_kib
        out[key + "_scale"] = scale
        out[key + "_bytes_per_launch"] = sum(mine) * 1024.0 * scale / launches
    out["launches"] = launches
    out["bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(traffic_path(tag), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


# ---------------------------------------------------------------- one workload
def stats(vals, nd=4):
    return {"median": round(statistics.median(vals), nd), "mean": round(statistics.fmean(vals), nd),
            "std": round(statistics.pstdev(vals), nd), "min": round(min(vals), nd), "n": len(vals)}


def run_workload(name, args, dc, dev, cpu_target, ceil=None):
    import torch
    wl = build_workload(name, dc, dev)
    if args.tune:
        # the library times the families each call's geometry allows and keeps the
        # fastest; the workload is then rebuilt so its tags name the chosen families
        for cl in wl["calls"]:
            if cl.tune is not None:
                cl.tune()
        torch.cuda.synchronize()
        del wl
        torch.cuda.empty_cache()
        wl = build_workload(name, dc, dev)
    kind = wl["kind"]
    digests = None if args.no_hash else input_digests(wl)
    # rotating copies: a step whose traffic is under 2 GiB would find part of its
    # inputs still in the 256 MB last-level cache when it runs again
    ncopy = int(min(8, max(1, math.ceil((2 << 30) / max(1, sum(cl.nbytes for cl in wl["calls"]))))))
    copies = [wl] + [build_workload(name, dc, dev) for _ in range(ncopy - 1)]
    calls_by_copy = [w_["calls"] for w_ in copies]
    if args.only_tag:
        calls_by_copy = [[cl for cl in cc if cl.tag == args.only_tag] for cc in calls_by_copy]
        if not calls_by_copy[0]:
            raise SystemExit("no call has tag %r; tags: %s" % (args.only_tag, sorted({c.tag for c in wl["calls"]})))
    calls = calls_by_copy[0]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def tag_groups(cc):
        gs = []
        for cl in cc:
            if gs and gs[-1][0] == cl.tag:
                gs[-1][1].append(cl)
            else:
                gs.append((cl.tag, [cl]))
        return gs

    groups_by_copy = [tag_groups(cc) for cc in calls_by_copy]
    groups = groups_by_copy[0]
    for cc in calls_by_copy:
        for cl in cc:
            cl.fn()
    torch.cuda.synchronize()
    graphs = []

    def runner(fns):
        """A callable launching fns in order: replay of one HIP graph holding them (--eager: direct calls)."""
        if args.eager:
            return lambda: [f() for f in fns]
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for f in fns:
                f()
        graphs.append(gr)
        return gr.replay

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    step_runs = [runner([cl.fn for cl in cc]) for cc in calls_by_copy]
    torch.cuda.synchronize()
    for w_ in range(args.warmup):
        step_runs[w_ % ncopy]()
    torch.cuda.synchronize()
    clocks_before = gpu_clocks()
    step_secs = []
    for _r in range(max(1, args.repeats)):
        t0 = time.perf_counter()
        for st in range(args.steps):
            step_runs[st % ncopy]()
        torch.cuda.synchronize()
        step_secs.append(time.perf_counter() - t0)
    clocks_after = gpu_clocks()
    elapsed = step_secs[0]

    # per-tag event times: each tag's calls replayed from a graph of their own,
    # tags in step order (each figure includes one graph-launch gap)
    tag_runs = [[runner([c.fn for c in cls]) for _tag, cls in gs] for gs in groups_by_copy]
    torch.cuda.synchronize()
    ev = [[event_pair() for _ in groups] for _ in range(args.steps)]
    for st in range(args.steps):
        for gi, run in enumerate(tag_runs[st % ncopy]):
            ev[st][gi][0].record(stream)
            run()
            ev[st][gi][1].record(stream)
    torch.cuda.synchronize()
    per_tag = {}
    for st in range(args.steps):
        for gi, (tag, cls) in enumerate(groups):
            ms = ev[st][gi][0].elapsed_time(ev[st][gi][1])
            r = per_tag.setdefault(tag, {"ms": 0.0, "launches": 0, "bytes": 0, "rbytes": 0, "flops": 0})
            r["ms"] += ms
            r["launches"] += len(cls)
            r["bytes"] += sum(c.nbytes for c in cls)
            r["rbytes"] += sum(c.rbytes for c in cls)
            r["flops"] += sum(c.flops for c in cls)
    dom_tag = max(per_tag, key=lambda t: per_tag[t]["ms"])

    # the dominant tag's launch duration: HIP events around one graph of REP
    # back-to-back rounds of its calls (>= 1 GiB of traffic per replay), three
    # replays per measurement, the measurement repeated
    dom_calls = [cl for cl in calls if cl.tag == dom_tag]
    dom_bytes = sum(cl.nbytes for cl in dom_calls)
    rep = int(min(64, max(4, math.ceil((1 << 30) / max(dom_bytes, 1)))))
    dom_run = runner([cl.fn for r in range(rep) for cl in calls_by_copy[r % ncopy] if cl.tag == dom_tag])
    dom_run()
    torch.cuda.synchronize()
    dom_launches = 3 * rep * len(dom_calls)
    avg_list = []
    for _r in range(max(1, args.repeats)):
        e0, e1 = event_pair()
        e0.record(stream)
        for _ in range(3):
            dom_run()
        e1.record(stream)
        torch.cuda.synchronize()
        avg_list.append(e0.elapsed_time(e1) / 1e3 / dom_launches)
    avg_s = statistics.median(avg_list)
    executed = (len(calls) * (ncopy + args.warmup + args.steps * (max(1, args.repeats) + 1))
                + len(dom_calls) * rep * (1 + 3 * max(1, args.repeats)))
    if args.copy_ref:
        src = torch.empty(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del graphs[:]

    # per call, cold: a 512 MiB fill (outside the timed window) evicts the last-level
    # cache and keeps the GPU busy while the host enqueues the events and the call, so
    # the window holds the call alone; median of the repeats
    per_case = []
    if not args.only_tag:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for ci, (ccalls, _t, _i) in enumerate(wl["per_case"]):
            for cl in ccalls:
                ts = []
                for r_ in range(max(1, args.repeats)):
                    scratch.fill_(r_ & 0xff)
                    e0, e1 = event_pair()
                    e0.record(stream)
                    cl.fn()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) / 1e3)
                per_case.append((ci, cl, statistics.median(ts)))
        del scratch

    step_bytes = sum(cl.nbytes for cl in calls)
    step_flops = sum(cl.flops for cl in calls)
    ms_step = elapsed / args.steps * 1e3
    dom_nbytes = dom_bytes / len(dom_calls)
    dom_nflops = sum(cl.flops for cl in dom_calls) / len(dom_calls)
    bound, peak, unit_r = tag_peak(dom_tag, kind)
    if kind == "bytes":
        value = step_bytes / (elapsed / args.steps) / 1e9
        unit = "GB/s"
        achieved = dom_nbytes / avg_s / 1e9
        step_peak = HBM_PEAK_GBS
    else:
        value = step_flops / (elapsed / args.steps) / 1e9
        unit = "GFLOP/s"
        achieved = dom_nflops / avg_s / 1e12
        step_peak = FP32_PEAK_TFLOPS * 1e3
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit_r,
            "frac": round(achieved / peak, 4), "traffic": committed_traffic(dom_tag),
            "kernel": dom_tag, "avg_launch_us": round(avg_s * 1e6, 2), "timed_launches": dom_launches,
            "avg_launch_us_repeats": stats([a * 1e6 for a in avg_list], 2),
            "step_frac": round(value / step_peak, 4),
            "frac_is": "the dominant kernel tag's average launch against its peak; step_frac is the whole "
                       "step's rate against %s" % ("8 TB/s" if kind == "bytes" else "the fp32 peak (157.3 TFLOP/s)")}
    dom_rfrac = sum(cl.rbytes for cl in dom_calls) / max(1, dom_bytes)
    cv = ceiling_of(dom_tag, kind, dom_rfrac, ceil)
    if cv is not None:
        roof["ceiling"] = {"value": round(cv[0], 1), "unit": cv[1], "basis": cv[2],
                           "frac": round(achieved / cv[0], 4)}
    rec = {
        "workload": wl["desc"], "value": round(value, 2), "unit": unit, "ms_per_step": round(ms_step, 4),
        "dtype": wl["dtype"], "config": dict({"workload": wl["desc"],
                                              "launch": "eager" if args.eager else "hip_graph_per_step",
                                              "kernel_selection": "tuned on this device" if args.tune
                                              else "built-in rules"}, **wl["cfg"]),
        "step_gbytes": round(step_bytes / 1e9, 4), "step_gflop": round(step_flops / 1e9, 4),
        "gbs": round(step_bytes / (elapsed / args.steps) / 1e9, 2),
        "gflops": round(step_flops / (elapsed / args.steps) / 1e9, 2),
        "step_timing_ms": stats([s_ / args.steps * 1e3 for s_ in step_secs]),
        "roofline": roof, "launches_executed": executed, "tensor_copies": ncopy,
        "gpu_clocks": {"before": clocks_before, "after": clocks_after},
        "per_kernel": {t: dict({"avg_us": round(r["ms"] / r["launches"] * 1e3, 2),
                                "share": round(r["ms"] / sum(v["ms"] for v in per_tag.values()), 4),
                                "gbs": round(r["bytes"] / (r["ms"] / 1e3) / 1e9, 1),
                                "gflops": round(r["flops"] / (r["ms"] / 1e3) / 1e9, 1)},
                               **tag_ceiling(t, r, kind, ceil))
                       for t, r in sorted(per_tag.items())},
    }
    if digests is not None:
        rec["input_sha256"] = digests
    cpu_est = {}
    if not args.no_cpu and not args.only_tag:
        rec["cpu_baseline"], cpu_est = cpu_baseline(wl, cpu_target)
    rows = []
    for ci, cl, sec in per_case:
        b_, pk, _u = tag_peak(cl.tag, kind)
        rate = (cl.nbytes / sec / 1e9) if kind == "bytes" else (cl.flops / sec / 1e12)
        t_roof = max(cl.nbytes / (HBM_PEAK_GBS * 1e9), cl.flops / (pk * 1e12 if b_ != "hbm" else FP32_PEAK_TFLOPS * 1e12))
        row = [cl.case, cl.pass_, round(sec * 1e6, 2), round(rate, 2 if kind == "bytes" else 3),
               round(rate / pk, 4), t_roof * 1e6 < LATENCY_US]
        est = cpu_est.get(id(cl))
        row.append(round(est / sec, 1) if est else None)
        cv = ceiling_of(cl.tag, kind, cl.rbytes / max(1, cl.nbytes), ceil)
        row.append(round(rate / cv[0], 4) if cv else None)
        rows.append(row)
    rec["per_case"] = {"columns": ["case", "pass", "us", "GB/s" if kind == "bytes" else "TFLOP/s", "frac",
                                   "latency_bound", "speedup_vs_oracle_all_threads", "frac_of_ceiling"], "rows": rows,
                       "timing": "HIP events around one eager call after a 512 MiB fill (cold), median of %d"
                                 % max(1, args.repeats)}
    del copies, wl, calls_by_copy, calls
    gc.collect()
    torch.cuda.empty_cache()
    return rec


def main(argv=None):
    args = parse(argv)
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.only_tag, args.launches, args.cmd)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.only_tag and args.workload == "all":
        raise SystemExit("--only-tag needs one --workload")
    import torch
    import dynamic_convolution_amd as dc

    if not os.path.exists(dc._native.LIB_PATH):
        from dynamic_convolution_amd import build as hb
        hb.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = WORKLOADS if args.workload == "all" else [args.workload]
    print("[bench] device ceilings", file=sys.stderr, flush=True)
    ceil = device_ceilings(dev)
    recs = {}
    for i, nm in enumerate(names):
        print("[bench] %s" % nm, file=sys.stderr, flush=True)
        recs[nm] = run_workload(nm, args, dc, dev, args.cpu_seconds if i == 0 else args.cpu_seconds / 2, ceil)
    head = recs[names[0]]
    out = {
        "metric": "dwconv fwd+bwd GFLOP/s and HBM GB/s at 1 GPU, % of roofline, vs CPU oracle",
        "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": head["config"],
        "device_ceilings": ceil,
    }
    for k_ in ("step_gbytes", "step_gflop", "gbs", "gflops", "step_timing_ms", "roofline", "launches_executed",
               "tensor_copies", "gpu_clocks", "per_kernel", "per_case", "input_sha256", "cpu_baseline"):
        if k_ in head:
            out[k_] = head[k_]
    if len(names) > 1:
        out["workloads"] = {nm: recs[nm] for nm in names[1:]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
