"""LDS carve-ups and workspace plans, checked on the host (no GPU).

tests/cpp/check_layouts.cpp includes the plan headers the kernels use and
checks, for every tile shape, dtype and level count, that each region fits,
that regions which are live at the same time do not overlap, that the
overlays (dS over V, the lambda row sums over Q, the level shares over K and
dS) fit the tile they reuse, and
that the backward workspace regions are ordered, aligned and sized, and, for
the Gated DeltaNet kernels, that every LDS region holds the tiles placed in it,
the workspace regions are ordered and sized, and every tree node a query chunk
reads lies inside its level.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_layouts_and_workspace_plans(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = tmp_path / "check_layouts"
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", os.path.join(HERE, "cpp", "check_layouts.cpp"),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.strip().startswith("ok")
