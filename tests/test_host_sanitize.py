"""The C ABI's host-side validation layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds ``rssm_api.hip`` (the ABI's host code: configuration checks, buffer sizing, ring
offsets, argument validation) with host-only sanitizers, links launchers that record calls
instead of launching (tests/sanitize/stub_launch.hip), and runs tests/sanitize/harness.cpp on
the CPU: a grid of valid and invalid configurations, every entry point with rejected
arguments (nothing may be launched), an empty batch, and valid arguments that reach the
launcher.  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_validation_layer_under_asan_and_ubsan():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "harness")
    # the sanitizers apply to host code only: each -fsanitize= follows -Xarch_host
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "attention_decode_mamba_amd", "csrc", "rssm_api.hip"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launch.hip"),
           os.path.join(ROOT, "tests", "sanitize", "harness.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    assert run.stdout.strip() == "ok"
    assert "Sanitizer" not in run.stderr and "runtime error" not in run.stderr
