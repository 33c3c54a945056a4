"""The C-ABI layer (csrc/api.hip) built for the host with AddressSanitizer and
driven by tests/abi_host/abi_asan.hip: the kernel launchers are stubs, so every
entry point's validation, workspace carving and planning runs on the CPU, on
host buffers of exactly the documented sizes.  Any out-of-bounds access or
dereference of a "device" pointer by the host layer is an ASan error; the
driver also checks return codes and where the workspace is carved.  CPU only.
Only host code is instrumented (the sanitizer flag is given to the host
compilation alone)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_09_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "abi_host", "abi_asan.hip")
OUT = os.path.join(ROOT, "_build", "abi_asan")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_abi_layer_under_host_asan():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "api.hip"), DRIVER, "-o", OUT]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    run = subprocess.run([OUT], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "AddressSanitizer" not in run.stderr
    assert "abi host checks passed" in run.stdout
