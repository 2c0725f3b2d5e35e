"""Benchmark of the depthwise / dynamic-filter hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mobilenet|multdil|largek|dynamic]

Prints ONE JSON line.  A step is one pass of every entry point the workload
uses over every case of the workload, with inputs resident in HBM:

  mobilenet (default)  3x3 depthwise layers of MobileNet, N in {1, 64, 128},
                       (C, H) in {(32,112), (64,112), (128,56), (256,28), (512,14),
                       (1024,7)}, stride 1 and 2, pad 1, fp32; forward, grad-input,
                       grad-weight (36 cases x 3 passes)
  multdil              multiplier 2, dilation 2, stride 2, 5x5, pad 4,
                       N=128, C=256->512, 56x56, bf16; the three passes
  largek               N=64, C=384, H in {32,48,64}, k in {7,13,31}, pad k//2,
                       fp32 and fp16; the three passes
  dynamic              per-pixel 3x3 filters at dilations 1/3/5, N in {1,2}, C=64,
                       H in {128,256}, fp32/fp16/bf16; output concatenated;
                       forward, then backward (dx and the filter gradients)

Passes run in pass-major order (every case's forward, then every grad-input,
then every grad-weight) so a tensor is re-read only after gigabytes of other
traffic, i.e. from HBM, not from the 256 MB last-level cache.

value      whole-step algorithmic throughput: compulsory bytes (each input element
           the result depends on once, each output once) per second for the
           bandwidth-bound workloads; valid-tap flops (2 per in-bounds multiply-add)
           per second for largek
launches   the whole step is captured once into a HIP graph and the timed steps
           replay it (--eager launches call by call instead).  A workload whose
           step moves less than 2 GiB gets identical copies of all its tensors
           (one graph per copy) and step i uses copy i % copies, so no launch
           finds its inputs still in the 256 MB last-level cache
per_kernel per kernel geometry (a "tag"): HIP events on the launch stream around
           a replay of a graph holding that tag's calls of one step, tags in step
           order, as many rounds as timed steps (each figure includes one
           graph-launch gap)
roofline   the dominant tag (most event time): its algorithmic bytes or flops per
           launch over its average launch duration, measured with HIP events on
           the launch stream around a graph of back-to-back rounds of its calls
           (at least 1 GiB of traffic per replay), against the MI355X peak;
           roofline.secondary relates it to what this machine reaches on a plain
           device-to-device copy measured in the same run (bandwidth-bound
           workloads) or to the unpacked v_fma_f32 rate (vector-bound ones)
cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
           (a batch slice of the same host tensors), on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak
FP32_UNPACKED_FMA_TFLOPS = 78.6  # one v_fma_f32 per lane and clock: 256 CUs x 64 lanes x 2.4 GHz x 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mobilenet", choices=["mobilenet", "multdil", "largek", "dynamic"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline leg")
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
                    help="calls of the tag in the counter runs (0: the dispatch count of its kernels)")
    ap.add_argument("--cmd", default="", help="command recorded with the traffic figures")
    return ap.parse_args()


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


class Call:
    """One entry-point call of the step with its algorithmic bytes and flops; tune, when
    given, times the kernel families that can run the call's geometry and records the
    fastest in the library's selection table."""

    def __init__(self, tag, fn, nbytes, flops, tune=None):
        self.tag, self.fn, self.nbytes, self.flops, self.tune = tag, fn, nbytes, flops, tune


def static_calls(dc, case, dev, seed, passes=("fwd", "bwd_in", "bwd_w")):
    import torch
    from dynamic_convolution_amd import synth
    n, c, h, M, k, s, p, d, dtype, dists, _label, with_bias = case
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

    def tag(pi, name):
        # one tag = one kernel instantiation: the library's algorithm for this geometry,
        # plus the template parameters it is specialised on
        algo = dc.dwconv2d_algo(pi, x.shape, w.shape, s, p, d, dtype)
        return "%s.%s.k%d_s%d_m%d_%s" % (name, algo, k, s, M, dts)

    if "fwd" in passes:
        calls.append(Call(tag(0, "fwd"), lambda: dc.dwconv2d_fwd(x, w, b, s, p, d, out=y), sx + W + B + Y, 2 * macs,
                          lambda: dc.dwconv2d_tune_fwd(x, w, b, s, p, d, out=y, reps=5)))
    if "bwd_in" in passes:
        calls.append(Call(tag(1, "bwd_input"), lambda: dc.dwconv2d_bwd_input(dy, w, x.shape, s, p, d, out=dx),
                          Y + W + X, 2 * macs,
                          lambda: dc.dwconv2d_tune_bwd_input(dy, w, x.shape, s, p, d, out=dx, reps=5)))
    if "bwd_w" in passes:
        calls.append(Call(tag(2, "bwd_weight"),
                          lambda: dc.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d, with_bias=with_bias, out=gw,
                                                         out_bias=gb, workspace=ws),
                          sx + Y + W + B, 2 * macs,
                          lambda: dc.dwconv2d_tune_bwd_weight(x, dy, w.shape, s, p, d, with_bias=with_bias, reps=5)))
    tensors = dict(x=x, w=w, b=b, dy=dy, y=y, dx=dx, gw=gw, gb=gb)
    return calls, tensors


def build_workload(name, dc, dev):
    """(cases, pass-major list of calls, description, dtype string, value kind)."""
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
                    cases.append(((n, c, h, 1, 3, s, 1, 1, torch.float32, dists, "3x3_s%d_" % s, False), seed))
                    seed += 1
        desc = "mobilenet_dw3x3_sweep"
        dt, kind = "f32", "bytes"
        cfg = {"batches": list(m["batches"]), "layers_c_h": [list(l) for l in m["layers"]],
               "strides": list(m["strides"]), "kernel": 3, "pad": 1, "passes": ["fwd", "bwd_input", "bwd_weight"]}
    elif name == "multdil":
        m = synth.MULT_DIL
        dists = dict(x=m["x"], w=m["w"], dy=m["dy"])
        cases.append(((m["n"], m["c"], m["h"], m["mult"], m["k"], m["stride"], m["pad"], m["dil"],
                       torch.bfloat16, dists, "5x5_m2_d2_s2_", False), 200))
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
                                   "k%d_%s_" % (k, dts), False), seed))
                    seed += 1
        desc, dt, kind = "large_kernel_dw_n64_c384", "f32+f16", "flops"
        cfg = {"n": L["n"], "c": L["c"], "hw": list(L["hs"]), "kernels": list(L["ks"]), "dtypes": list(L["dtypes"]),
               "passes": ["fwd", "bwd_input", "bwd_weight"]}
    else:
        return build_dynamic(dc, dev)
    per_case = [static_calls(dc, cs, dev, seed) for cs, seed in cases]
    # pass-major; within a pass, calls of one kernel geometry (tag) are adjacent
    calls = []
    for pi in range(3):
        tags = {}
        for cls, _t in per_case:
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
                cf = Call("dyn.fused.k3_%s" % dts,
                          (lambda x=x, fs=fs, y=y: dc.dynconv_multidil_fwd(x, fs, D["dilations"], out=y)),
                          X + TF + Y, 2 * n * c * taps)
                cb = Call("dyn_bwd.fused.k3_%s" % dts,
                          (lambda x=x, fs=fs, dy=dy, dx=dx, dfs=dfs:
                           dc.dynconv_multidil_bwd(x, fs, dy, D["dilations"], out_dx=dx, out_dfilters=dfs)),
                          X + Y + TF + X + FF, 3 * n * c * taps)
                fwd.append(cf)
                bwd.append(cb)
                per_case.append(([cf, cb], dict(x=x, fs=fs, y=y, dy=dy, dx=dx, dfs=dfs)))
                cases.append(((n, h, dts), seed))
                seed += 1
    cfg = {"batches": list(D["batches"]), "c": D["c"], "hw": list(D["hs"]), "k": 3, "dilations": list(D["dilations"]),
           "dtypes": list(D["dtypes"]), "passes": ["fwd", "bwd (dx and filter gradients)"]}
    return dict(cases=cases, per_case=per_case, calls=fwd + bwd, desc="dynamic_multidil_3x3_d135", dtype="f32+f16+bf16",
                kind="bytes", cfg=cfg)


def device_copy_gbs(dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate (read + write bytes per second, GB/s) of torch's
    copy kernel over two buffers of `nbytes`, timed with HIP events."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return 2 * nbytes / sec / 1e9


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, target_s):
    """Time the oracle on a batch slice of the workload's own tensors."""
    import numpy as np
    import torch
    from oracle import oracle as O

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    kind = wl["kind"]

    def run_sample(ns):
        tot_units, tot_t = 0.0, 0.0
        for (cs, _seed), (calls, t) in zip(wl["cases"], wl["per_case"]):
            if "fs" in t:  # dynamic
                n = t["x"].shape[0]
                sl = min(ns, n)
                x = f64(t["x"][:sl])
                fs = [f64(f[:sl]) for f in t["fs"]]
                dy = f64(t["dy"][:sl])
                t0 = time.perf_counter()
                O.dynconv_multidil_fwd(x, fs, (1, 3, 5))
                O.dynconv_multidil_bwd(x, fs, dy, (1, 3, 5))
                tot_t += time.perf_counter() - t0
                tot_units += sum(cl.nbytes if kind == "bytes" else cl.flops for cl in calls) * sl / n
                continue
            n, c, h, M, k, s, p, d = cs[:8]
            sl = min(ns, n)
            x, w, dy = f64(t["x"][:sl]), f64(t["w"]), f64(t["dy"][:sl])
            for cl in calls:
                t0 = time.perf_counter()
                if cl.tag.startswith("fwd."):
                    O.dwconv2d_fwd(x, w, None, s, p, d)
                elif cl.tag.startswith("bwd_input."):
                    O.dwconv2d_bwd_input(dy, w, x.shape, s, p, d)
                else:
                    O.dwconv2d_bwd_weight(x, dy, w.shape, s, p, d, with_bias=False)
                tot_t += time.perf_counter() - t0
                tot_units += (cl.nbytes if kind == "bytes" else cl.flops) * sl / n
        return tot_units, tot_t

    u1, t1 = run_sample(1)
    ns = 1
    if t1 > 0 and t1 < target_s:
        ns = max(1, min(128, int(target_s / t1)))
        if ns > 1:
            u1, t1 = run_sample(ns)
    used = max(min(ns, t["x"].shape[0]) for _c, t in wl["per_case"])
    whole = all(min(ns, t["x"].shape[0]) == t["x"].shape[0] for _c, t in wl["per_case"])
    # a whole workload that the oracle finishes well inside the target is run
    # again, so the rate comes from about target_s of oracle time
    reps = 1
    if whole and 0 < t1 < target_s / 2:
        reps = min(20, max(1, int(target_s / t1)))
        for _ in range(reps - 1):
            u, t_ = run_sample(ns)
            u1, t1 = u1 + u, t1 + t_
    if kind == "bytes":
        val, unit = u1 / t1 / 1e9, "GB/s"
    else:
        val, unit = u1 / t1 / 1e9, "GFLOP/s"
    what = "every case's whole batch" if whole else "first %d image(s) of every case's batch" % used
    if reps > 1:
        what += " (%d passes over it)" % reps
    return {"value": round(val, 4), "unit": unit, "cores": O.num_threads(), "kind": "oracle",
            "sample": "%s, every pass, same host tensors; %.1f s of oracle time" % (what, t1)}


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


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.only_tag, args.launches, args.cmd)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dynamic_convolution_amd as dc

    if not os.path.exists(dc._native.LIB_PATH):
        from dynamic_convolution_amd import build as hb
        hb.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = build_workload(args.workload, dc, dev)
    if args.tune:
        # the library times the families each call's geometry allows and keeps the
        # fastest; the workload is then rebuilt so its tags name the chosen families
        for cl in wl["calls"]:
            if cl.tune is not None:
                cl.tune()
        torch.cuda.synchronize()
        del wl
        torch.cuda.empty_cache()
        wl = build_workload(args.workload, dc, dev)
    # rotating copies: a step whose traffic is under 2 GiB would find part of its
    # inputs still in the 256 MB last-level cache when it runs again, so such
    # workloads get identical copies of every tensor and step i uses copy i % ncopy
    ncopy = int(min(8, max(1, math.ceil((2 << 30) / max(1, sum(cl.nbytes for cl in wl["calls"]))))))
    copies = [wl] + [build_workload(args.workload, dc, dev) for _ in range(ncopy - 1)]
    calls_by_copy = [w_["calls"] for w_ in copies]
    if args.only_tag:
        calls_by_copy = [[cl for cl in cc if cl.tag == args.only_tag] for cc in calls_by_copy]
        if not calls_by_copy[0]:
            raise SystemExit("no call has tag %r; tags: %s" % (args.only_tag, sorted({c.tag for c in wl["calls"]})))
    calls = calls_by_copy[0]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # one group of consecutive calls per tag (= one kernel geometry); every copy
    # has the same calls in the same order
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

    # the whole step is captured once into one HIP graph, so the step's launches
    # cost no host time and no gap between graph launches, as a fixed training
    # step would run
    graphs = []
    step_runs = [runner([cl.fn for cl in cc]) for cc in calls_by_copy]
    torch.cuda.synchronize()
    for w_ in range(args.warmup):
        step_runs[w_ % ncopy]()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for st in range(args.steps):
        step_runs[st % ncopy]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-tag event times: each tag's calls replayed from a graph of their own,
    # tags in step order, HIP events recorded on the launch stream around each
    # replay (each figure includes one graph-launch gap)
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
            r = per_tag.setdefault(tag, {"ms": 0.0, "launches": 0, "bytes": 0, "flops": 0})
            r["ms"] += ms
            r["launches"] += len(cls)
            r["bytes"] += sum(c.nbytes for c in cls)
            r["flops"] += sum(c.flops for c in cls)
    dom_tag = max(per_tag, key=lambda t: per_tag[t]["ms"])

    # the dominant tag's launch duration: HIP events around one graph of REP
    # back-to-back rounds of its calls (at least 1 GiB of traffic per replay,
    # so every round reads its inputs from HBM again), three replays
    dom_calls = [cl for cl in calls if cl.tag == dom_tag]
    dom_bytes = sum(cl.nbytes for cl in dom_calls)
    rep = int(min(64, max(4, math.ceil((1 << 30) / max(dom_bytes, 1)))))
    dom_run = runner([cl.fn for r in range(rep) for cl in calls_by_copy[r % ncopy] if cl.tag == dom_tag])
    dom_run()
    torch.cuda.synchronize()
    e0, e1 = event_pair()
    e0.record(stream)
    for _ in range(3):
        dom_run()
    e1.record(stream)
    torch.cuda.synchronize()
    dom_launches = 3 * rep * len(dom_calls)
    avg_s = e0.elapsed_time(e1) / 1e3 / dom_launches
    executed = len(calls) * (ncopy + args.warmup + 2 * args.steps) + len(dom_calls) * rep * 4
    if args.copy_ref:
        src = torch.empty(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del graphs

    step_bytes = sum(cl.nbytes for cl in calls)
    step_flops = sum(cl.flops for cl in calls)
    ms_step = elapsed / args.steps * 1e3
    dom_nbytes = dom_bytes / len(dom_calls)
    dom_nflops = sum(cl.flops for cl in dom_calls) / len(dom_calls)
    if wl["kind"] == "bytes":
        value = step_bytes / (elapsed / args.steps) / 1e9
        unit = "GB/s"
        achieved = dom_nbytes / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        value = step_flops / (elapsed / args.steps) / 1e9
        unit = "GFLOP/s"
        achieved = dom_nflops / avg_s / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 2), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP32_VALU_PEAK_TFLOPS, 4)}
    roof["traffic"] = committed_traffic(dom_tag)
    # secondary ratios: the on-box device-to-device copy rate (bytes read plus
    # bytes written, over buffers four times the last-level cache) measured in
    # this run, and for vector-bound kernels the unpacked v_fma_f32 rate
    if wl["kind"] == "bytes":
        if args.copy_ref:  # counter runs: their own reference copy must stay the last copy
            roof["secondary"] = None
        else:
            copy_gbs = device_copy_gbs(dev)
            roof["secondary"] = {"copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)}
    else:
        roof["secondary"] = {"unpacked_fma_tflops": FP32_UNPACKED_FMA_TFLOPS,
                             "frac_of_unpacked": round(achieved / FP32_UNPACKED_FMA_TFLOPS, 4)}
    roof["kernel"] = dom_tag
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)
    roof["timed_launches"] = dom_launches

    out = {
        "metric": "dwconv fwd+bwd GFLOP/s and HBM GB/s at 1 GPU, % of roofline, vs CPU oracle",
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl["dtype"], "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": dict({"workload": wl["desc"], "launch": "eager" if args.eager else "hip_graph_per_step",
                        "kernel_selection": "tuned on this device" if args.tune else "built-in rules"},
                       **wl["cfg"]),
        "step_gbytes": round(step_bytes / 1e9, 4), "step_gflop": round(step_flops / 1e9, 4),
        "gbs": round(step_bytes / (elapsed / args.steps) / 1e9, 2),
        "gflops": round(step_flops / (elapsed / args.steps) / 1e9, 2),
        "roofline": roof,
        "launches_executed": executed,
        "tensor_copies": ncopy,
        "per_kernel": {t: {"avg_us": round(r["ms"] / r["launches"] * 1e3, 2),
                                       "share": round(r["ms"] / sum(v["ms"] for v in per_tag.values()), 4),
                                       "gbs": round(r["bytes"] / (r["ms"] / 1e3) / 1e9, 1),
                                       "gflops": round(r["flops"] / (r["ms"] / 1e3) / 1e9, 1)}
                       for t, r in sorted(per_tag.items())},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
