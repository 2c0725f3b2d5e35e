"""The CPU oracle against its pins, and the pins against planted mistakes.

Every ``check_*`` in oracle_pins.py runs against the oracle built from
oracle/dwconv_oracle.c.  Then each mutation below is planted in a copy of that
source (on the CPU, in a temporary directory), the copy is compiled, and the
whole battery must reject it: a dropped term, a wrong sign or index, a
transposed operand or a wrong channel mapping in any entry point fails at
least one pin.
"""
import os
import re
import shutil
import tempfile

import pytest

import oracle_pins as P
from oracle import oracle as O


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


# (name, regex to find, replacement, which occurrence: 0-based index or None = all)
MUTATIONS = [
    ("fwd_pad_sign", r"oh \* sh - ph", "oh * sh + ph", 0),
    ("fwd_kernel_transposed", r"wp\[i \* kw \+ j\] \* xp", "wp[j * kh + i] * xp", 0),
    ("fwd_bias_dropped", r"b \? b\[o\] : 0\.0", "0.0", 0),
    ("fwd_channel_map", r"g = o / mult;", "g = o % ic;", 0),
    ("fwd_col_bound", r"c < iw\)", "c <= iw)", 0),
    ("fwd_dilation_col", r"ow \* sw - pw \+ j \* dw", "ow * sw - pw + j", 0),
    ("fwd_stride_row", r"oh \* sh - ph \+ i \* dh", "oh - ph + i * dh", 0),
    ("outsize_off_by_one", r"<= in - 1 \+ p\) o\+\+", "< in - 1 + p) o++", 0),
    ("bwdin_mult_loop", r"for \(int64_t m = 0; m < mult; m\+\+\)", "for (int64_t m = 0; m < 1; m++)", 0),
    ("bwdin_pad_sign", r"oh \* sh - ph", "oh * sh + ph", 1),
    ("bwdin_kernel_transposed", r"wp\[i \* kw \+ j\] \* dyp", "wp[j * kh + i] * dyp", 0),
    ("bwdw_bias_sum_dropped", r"bsum \+= gy;", "", 0),
    ("bwdw_dilation", r"oh \* sh - ph \+ i \* dh", "oh * sh - ph + i", 2),
    ("bwdw_channel_map", r"g = o / mult;", "g = o % ic;", 1),
    ("dyn_tap_flip", r"py \+ \(i - r\) \* d", "py + (r - i) * d", 0),
    ("dyn_concat_interleaved", r"nn \* nb \* c \+ br \* c \+ ch", "nn * nb * c + ch * nb + br", 0),
    ("dyn_filter_spatial_transposed", r"h \* w \+ py \* w \+ px\]", "h * w + px * h + py]", 0),
    ("dyn_tap_order", r"\(i \* k \+ j\) \* h \* w", "(j * k + i) * h * w", 0),
    ("dyn_dilation_ignored", r"sx = px \+ \(j - r\) \* d", "sx = px + (j - r)", 0),
    ("dynbwd_tap_flip", r"py \+ \(i - r\) \* d", "py + (r - i) * d", 1),
    ("dynbwd_branch_offset", r"nn \* nb \* c \+ br \* c \+ ch", "nn * nb * c + ch * nb + br", 1),
    ("dynbwd_df_reads_filter", r"g \* xp\[sy \* w \+ sx\]", "g * fp[t]", 0),
    ("dynbwd_dx_drops_dy", r"\+= fp\[t\] \* g;", "+= fp[t];", 0),
    ("dynbwd_dilation_ignored", r"sx = px \+ \(j - r\) \* d", "sx = px + (j - r)", 1),
]


def _mutate(src, pattern, repl, occ):
    hits = list(re.finditer(pattern, src))
    assert hits, "mutation pattern not found: " + pattern
    if occ is None:
        return re.sub(pattern, repl, src)
    m = hits[occ]
    return src[:m.start()] + repl + src[m.end():]


@pytest.fixture(scope="module")
def mutants():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    src = open(O.SRC).read()
    libs = {}
    for name, pat, repl, occ in MUTATIONS:
        path = os.path.join(tmp, name + ".c")
        with open(path, "w") as f:
            f.write(_mutate(src, pat, repl, occ))
        libs[name] = O.compile_source(path, os.path.join(tmp, "lib%s.so" % name))
    yield libs
    shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(mutants, name):
    variant = O.load_variant(mutants[name])
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(variant)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    assert caught, "planted mistake %s passed every pin" % name
