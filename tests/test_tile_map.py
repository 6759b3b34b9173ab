"""The grouped launches' block -> tile maps, checked on the host: bijective,
in range, contiguous and balanced per XCD (tests/tile_map_check.cpp compiled
with g++ against the library's own tile_map.h)."""

import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_maps_are_bijections():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "tile_map_check")
        r = subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror",
                            "-I" + os.path.join(ROOT, "matrix_optimizer_02_amd", "csrc"),
                            os.path.join(ROOT, "tests", "tile_map_check.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
