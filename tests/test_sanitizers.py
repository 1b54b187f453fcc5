"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The planner's work split (plan.cpp with tests/plan_split_check.cpp, the
  driver test_plan_host.py runs) built with -fsanitize=address,undefined:
  every range, bound and brute-force comparison of the driver runs with
  bounds, overflow and alignment checks on.
- The oracle (oracle/mdcn_oracle.c) built the same way and loaded in place of
  its default build (MDCN_ORACLE_LIBRARY) by a child pytest that runs the
  pin suites of the forward, the FP8 mode and the backward: every oracle
  call of those pins runs checked.  Any report aborts the child.
Only host compilers are used; no code for the GPU is built here.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "modulated_deformable_convolution_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


needs_gcc = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                               reason="no host compiler")


@needs_gcc
def test_plan_split_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_split_check_san"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g"] + SAN +
                   ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "plan_split_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=600)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.startswith("ok"), out.stdout


@needs_gcc
@pytest.mark.skipif(runtime("libasan.so") is None or runtime("libubsan.so") is None,
                    reason="no sanitizer runtimes")
def test_oracle_pins_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import oracle
    lib = oracle.compile_library(output=str(tmp_path / "libmdcn_oracle_san.so"),
                                 extra_flags=SAN + ["-g"])
    env = dict(os.environ)
    env.update(MDCN_ORACLE_LIBRARY=lib,
               LD_PRELOAD="%s:%s" % (runtime("libasan.so"), runtime("libubsan.so")),
               # the interpreter itself is not instrumented: only the oracle's
               # accesses are checked, and its leaks are not the oracle's
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "not planted_mistake",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_fp8_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_backward_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
