"""Host-side exhaustive check of the division inside the library's fp8
quantisation (tests/quotient_exactness.c; no GPU).

The kernels quantise x / s ("PR #55356 完整报告", 关键源码片段: scaled_convert
with the layer's kv_scales entry; "PR #51772 完整报告", 实现拆解 item 1: codes
bit-identical to torch's e4m3fn cast of the quotient) without a divide:
r = RN(1/s) once, q0 = RN(x r), one fused-multiply-add remainder and one
correction.  The C program runs that sequence in binary32 on the host and
compares it with the IEEE quotient:
  - every bf16 significand x every fp32 significand of s: identical;
  - every fp16 significand x every fp32 significand of s: identical;
  - every finite bf16 pattern (subnormals, zeros) x scales of every binary32
    exponent: wherever the difference could reach an e4m3fn or e5m2 code, the
    two agree for 2^-85 <= |s| < 2^126 -- the range of scales the library
    states as exact -- and disagree outside it, so the stated bounds are the
    true ones;
  - the same sweep without the correction step (a planted mistake) fails.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quotient_exactness.c")


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_exactness")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-Wall", "-o", exe, SRC, "-lm"], check=True)
    return exe


def run(prog, sweep):
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = dict(os.environ, OMP_NUM_THREADS=str(max(1, min(16, n))))
    return subprocess.run([prog, sweep], capture_output=True, text=True, check=True,
                          env=env).stdout


def test_every_bf16_significand_against_every_scale_significand(prog):
    assert "sig16 7 mismatches 0" in run(prog, "bf16")


def test_every_fp16_significand_against_every_scale_significand(prog):
    assert "sig16 10 mismatches 0" in run(prog, "fp16")


def test_scale_exponent_range_is_exact_and_tight(prog):
    out = run(prog, "edges")
    bad = {int(e): int(n) for e, n in re.findall(r"edges exp (-?\d+) mismatches (\d+)", out)}
    inside = {e: n for e, n in bad.items() if -85 <= e < 126}
    assert not inside, f"quotient differs for scales inside [2^-85, 2^126): {inside}"
    assert -86 in bad and 126 in bad, "the stated bounds are not the tight ones"


def test_sweep_catches_a_missing_correction(prog):
    out = run(prog, "bf16-uncorrected")
    n = int(re.search(r"uncorrected mismatches (\d+)", out).group(1))
    assert n > 0
