"""The workgroup orders of the causal and masked query-tile passes
(`wg_coords_grouped` in csrc/miattn_device.h), checked on the CPU by a host
program built from the same header: a bijection for every shape, and equal
causal work on every XCD whenever an XCD's range holds whole heads (a group
of heads narrower than four when the range holds fewer); and the packed-
sequence order (`wg_coords_unit_major`): a bijection giving every XCD the
same heads of every sequence, so equal work whatever the lengths."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_09_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "abi_host", "wg_order.hip")
OUT = os.path.join(ROOT, "_build", "wg_order")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_query_tile_order_is_a_balanced_bijection():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", DRIVER, "-o", OUT]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = subprocess.run([OUT], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "order checks passed" in run.stdout
