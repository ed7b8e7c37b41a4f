"""The workgroup-to-tile mapping of the matrix-core launches (tile_order in
fa_device.h) is a bijection onto (head, tile rank) and keeps a head's tiles on
one XCD when the heads split evenly over the eight XCDs.  The device header is
compiled for the host with hipcc and run on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "tile_order_check.hip")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.fail("hipcc is required to build the host check")


def test_tile_order_is_a_bijection(tmp_path):
    exe = tmp_path / "tile_order_check"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", SRC, "-o",
                        str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
