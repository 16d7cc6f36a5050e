"""Host checks of the grouped GEMM's index arithmetic (no GPU needed):
tests/tile_plan_check.hip walks the launched grid through the same
split_rows / find_tile_2d / find_tail functions the kernel runs, for
edge-case and random group sizes; tests/kmajor_layout_check.hip runs the
k-major operand loads and transposing reads of the backward GEMMs;
tests/router_split_check.hip checks that the router's three bf16 parts of an
fp32 weight sum to it exactly."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _build_and_run(tmp_path, name):
    exe = str(tmp_path / name)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "sparse_mixture_experts_42_amd", "csrc"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", exe, os.path.join(ROOT, "tests", name + ".hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert re.search(r"(^|\s)0 failures", r.stdout)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_tile_plan_covers_every_row_once(tmp_path):
    _build_and_run(tmp_path, "tile_plan_check")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_kmajor_operand_layout(tmp_path):
    _build_and_run(tmp_path, "kmajor_layout_check")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_router_weight_split_is_exact(tmp_path):
    _build_and_run(tmp_path, "router_split_check")
