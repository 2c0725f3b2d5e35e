"""Streams and host threads: every entry point enqueues on the caller's current
stream, and concurrent calls from several host threads on their own streams,
with disjoint outputs, give bitwise the results of the same calls made one at
a time (every kernel family is deterministic), also while another thread
edits the kernel-selection table."""
import threading

import pytest
import torch

import dynamic_convolution_amd as dc
from dynamic_convolution_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print("[case] " + msg, flush=True)


def make_jobs():
    """(name, closure writing into preallocated outputs, outputs) for a spread of kernel families."""
    jobs = []
    g = [0]

    def draw(shape, dt, dist=("N", 0.0, 1.0)):
        g[0] += 1
        return synth.draw(shape, dist, 900 + g[0], "x", dt, device=DEV)

    # 3x3 row-walk forward and grad-weight, fp32
    x = draw((4, 8, 64, 64), torch.float32)
    w = draw((8, 3, 3), torch.float32)
    y = torch.empty_like(x)
    dy = draw((4, 8, 64, 64), torch.float32)
    gw, gb = torch.empty_like(w), torch.empty((8,), device=DEV)
    jobs.append(("rowwalk fwd", lambda x=x, w=w, y=y: dc.dwconv2d_fwd(x, w, None, 1, 1, 1, out=y), [y]))
    jobs.append(("rowwalk bwd_weight",
                 lambda x=x, dy=dy, gw=gw, gb=gb: dc.dwconv2d_bwd_weight(x, dy, gw.shape, 1, 1, 1, out=gw,
                                                                         out_bias=gb),
                 [gw, gb]))
    # 31x31 forward on the matrix cores (fp16) and the vector path (fp32)
    for dt in (torch.float16, torch.float32):
        x = draw((2, 4, 40, 40), dt)
        w = (draw((4, 31, 31), torch.float32) / 31).to(dt)
        y = torch.empty_like(x)
        jobs.append(("largek fwd %s" % dt, lambda x=x, w=w, y=y: dc.dwconv2d_fwd(x, w, None, 1, 15, 1, out=y), [y]))
    # multiplier 2 / dilation 2 / stride 2 grad-input, bf16
    x = draw((2, 6, 40, 40), torch.bfloat16)
    w = draw((12, 5, 5), torch.bfloat16, ("N", 0.0, 0.2))
    oh, ow = dc.dwconv2d_out_size(x.shape, w.shape, 2, 4, 2)
    dy = draw((2, 12, oh, ow), torch.bfloat16)
    dx = torch.empty_like(x)
    jobs.append(("even-grid bwd_input",
                 lambda dy=dy, w=w, dx=dx, xs=x.shape: dc.dwconv2d_bwd_input(dy, w, xs, 2, 4, 2, out=dx), [dx]))
    # fused dynamic filter forward and backward, fp32
    x = draw((1, 8, 48, 48), torch.float32)
    fs = [draw((1, 8, 9, 48, 48), torch.float32, ("N", 0.0, 1.0 / 3)) for _ in range(3)]
    y = torch.empty((1, 24, 48, 48), device=DEV)
    dy = draw((1, 24, 48, 48), torch.float32)
    dx = torch.empty_like(x)
    dfs = [torch.empty_like(f) for f in fs]
    jobs.append(("dynamic fwd", lambda x=x, fs=fs, y=y: dc.dynconv_multidil_fwd(x, fs, (1, 3, 5), out=y), [y]))
    jobs.append(("dynamic bwd",
                 lambda x=x, fs=fs, dy=dy, dx=dx, dfs=dfs: dc.dynconv_multidil_bwd(x, fs, dy, (1, 3, 5), out_dx=dx,
                                                                                   out_dfilters=dfs),
                 [dx] + dfs))
    torch.cuda.synchronize()
    return jobs


def snapshot(outs):
    return [o.detach().clone() for o in outs]


def test_calls_follow_the_current_stream():
    jobs = make_jobs()
    ref = []
    for name, fn, outs in jobs:
        note("default stream: " + name)
        fn()
        torch.cuda.synchronize()
        ref.append(snapshot(outs))
        for o in outs:
            o.fill_(float("nan"))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        for name, fn, _outs in jobs:
            note("side stream: " + name)
            fn()
    s.synchronize()
    for (name, _fn, outs), r in zip(jobs, ref):
        for o, ro in zip(outs, r):
            assert torch.equal(o, ro), name


def test_concurrent_threads_on_own_streams():
    jobs = make_jobs()
    ref = []
    for name, fn, outs in jobs:
        fn()
        torch.cuda.synchronize()
        ref.append(snapshot(outs))
        for o in outs:
            o.zero_()
    torch.cuda.synchronize()
    errors = []

    def worker(idx):
        name, fn, outs = jobs[idx]
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    fn()
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((name, repr(e)))

    def table_editor():
        # record and remove a selection for a geometry no job uses, repeatedly
        geo = ((2, 3, 20, 20), (3, 3, 3), 1, 1, 1)
        try:
            for _ in range(50):
                cands = dc.dwconv2d_algo_candidates(0, *geo, dtype=torch.float32)
                dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo=cands[0])
                dc.dwconv2d_set_algo(0, *geo, dtype=torch.float32, algo=None)
        except Exception as e:
            errors.append(("table", repr(e)))

    note("threads: %d jobs + a selection-table editor" % len(jobs))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    threads.append(threading.Thread(target=table_editor))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for (name, _fn, outs), r in zip(jobs, ref):
        for o, ro in zip(outs, r):
            assert torch.equal(o, ro), name
