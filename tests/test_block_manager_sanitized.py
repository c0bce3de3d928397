"""The block manager's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/native/bm_stress.cpp drives random operations against a plain model
of the page mapping and checks the manager's invariants after every call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "bm_stress")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "exact_tiled_attention_pa_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "bm_stress.cpp"),
           os.path.join(ROOT, "exact_tiled_attention_pa_amd", "csrc", "block_manager.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0, (run.returncode, run.stdout[-2000:], run.stderr[-3000:])
    assert "ok" in run.stdout
