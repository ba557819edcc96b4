"""Host logic of the library, checked on the host (no GPU).

tests/cpp/check_layouts.cpp includes the plan headers the kernels use and
checks, for every tile shape, dtype and level count, that each region fits,
that regions which are live at the same time do not overlap, that the
overlays (dS over V, the lambda row sums over Q, the level shares over K and
dS) fit the tile they reuse, and
that the backward workspace regions are ordered, aligned and sized, and, for
the Gated DeltaNet kernels, that every LDS region holds the tiles placed in it,
the workspace regions are ordered and sized, and every tree node a query chunk
reads lies inside its level.

tests/cpp/check_host_logic.cpp checks the bucket enumeration of the forward's
output kernel against the closed-form Fenwick level 1 + msb(t xor s) for
every chunk and group size (each earlier chunk covered exactly once, at that
level), and the argument checks of every C entry point (null pointers,
alignment, workspace size, decode capacity) with addresses that are never
dereferenced.

Both programs are built with g++ under the address and undefined-behaviour
sanitizers, so an out-of-range shift or an overflow in the plan arithmetic
fails the test as well.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_and_run(name, tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = tmp_path / name
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", *SANITIZE, "-I", os.path.join(ROOT, "include"),
                        os.path.join(HERE, "cpp", name + ".cpp"), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert r.stdout.strip().startswith("ok"), r.stdout[-2000:]


def test_layouts_and_workspace_plans(tmp_path):
    _build_and_run("check_layouts", tmp_path)


def test_bucket_enumeration_and_argument_checks(tmp_path):
    _build_and_run("check_host_logic", tmp_path)
