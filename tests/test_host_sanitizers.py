"""Host code under the sanitizers: the planner (csrc/plan.cpp) driven through
the C ABI by a plain C99 program on many pseudo-random matrix sets, options
and tuned entries (tests/plan_sanitize_check.c), and the grouped launches'
block -> tile maps (tests/tile_map_check.cpp), each built with g++/gcc and
-fsanitize=address,undefined with no recovery, so that any out-of-bounds
access, leak, signed overflow or misaligned access fails the test.  Host
compilers only: no GPU code is built here."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_optimizer_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _have_sanitizer_runtime() -> bool:
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        return False
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "t.c")
        with open(src, "w") as f:
            f.write("int main(void){return 0;}\n")
        r = subprocess.run(["gcc", *SAN, src, "-o", os.path.join(td, "t")], capture_output=True, text=True)
        return r.returncode == 0


needs_san = pytest.mark.skipif(not _have_sanitizer_runtime(), reason="no host sanitizer runtime")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[0], r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    return r


@needs_san
def test_planner_under_sanitizers():
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    with tempfile.TemporaryDirectory() as td:
        plan_o = os.path.join(td, "plan.o")
        drv_o = os.path.join(td, "drv.o")
        exe = os.path.join(td, "plan_check")
        _run(["g++", *SAN, "-std=c++17", "-Wall", "-Werror", f"-I{INCLUDE}", "-c", os.path.join(CSRC, "plan.cpp"),
              "-o", plan_o])
        _run(["gcc", *SAN, "-std=c99", "-Wall", "-Werror", f"-I{INCLUDE}", "-c",
              os.path.join(ROOT, "tests", "plan_sanitize_check.c"), "-o", drv_o])
        _run(["g++", *SAN, drv_o, plan_o, "-o", exe])
        r = _run([exe], env=env, timeout=300)
        assert r.stdout.strip().endswith("OK"), r.stdout


@needs_san
def test_tile_maps_under_sanitizers():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "tile_map_check")
        _run(["g++", *SAN, "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}",
              os.path.join(ROOT, "tests", "tile_map_check.cpp"), "-o", exe])
        r = _run([exe], timeout=600)
        assert r.stdout.strip().endswith("OK"), r.stdout
