"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs under tests/sanitize/ are built with the sanitizers on host code
only (device code is compiled but never launched) and run:

* host_check: every host path of the C ABI -- argument validation, output
  sizes, kernel-family selection for thousands of seeded geometries, the
  selection table, workspace sizing and status strings -- linked against the
  library's own sources;
* oracle_check: every function of the C oracle on small seeded geometries with
  exactly sized heap arrays, plus the adjoint identities between its passes.

Objects are cached under _build/sanitize keyed by the hash of their source and
flags, so only the first run after a change pays for the compile.
"""
import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_convolution_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
# sanitizers on the host pass only; the device pass is built unoptimised since it never runs
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Xarch_device", "-O0", "-Xarch_device", "-g0",
             "-I" + INCLUDE, "-I" + CSRC]
for _f in SAN:
    HIP_FLAGS += ["-Xarch_host", _f]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="3")

needs_tools = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and shutil.which("gcc")),
                                 reason="hipcc, clang++ and gcc are needed")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=ENV)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stdout[-4000:])
    return r.stdout


def _object(src, compiler, flags):
    text = open(src, "rb").read()
    deps = b"".join(open(h, "rb").read() for h in sorted(glob.glob(os.path.join(CSRC, "*.hpp")) +
                                                          glob.glob(os.path.join(INCLUDE, "*.h"))))
    key = hashlib.sha256(text + deps + " ".join([compiler] + flags).encode()).hexdigest()[:16]
    obj = os.path.join(OUT, "%s.%s.o" % (os.path.basename(src), key))
    if not os.path.exists(obj):
        tmp = obj + ".tmp%d" % os.getpid()
        _run([compiler] + flags + ["-c", src, "-o", tmp])
        os.replace(tmp, obj)
    return obj


@needs_tools
def test_host_abi_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _object(s, HIPCC, HIP_FLAGS), srcs))
    drv = _object(os.path.join(HERE, "host_check.cpp"), CLANGXX,
                  ["-std=c++17", "-O1", "-g", "-I" + INCLUDE] + SAN)
    exe = os.path.join(OUT, "host_check")
    _run([CLANGXX] + SAN + [drv] + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                                           "-o", exe])
    out = _run([exe])
    assert "host checks ok" in out, out


@needs_tools
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_check")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-Wall", "-Wextra"] + SAN +
         [os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "dwconv_oracle.c"), "-lm", "-o", exe])
    out = _run([exe])
    assert "oracle checks ok" in out, out
