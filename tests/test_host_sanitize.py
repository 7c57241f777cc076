"""Host code of the C-ABI layer (geometry, buffer sizing, argument checks)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
only, then fuzzed with seeded problem shapes up to the int32 limits of the
index tensors (tests/sanitize/host_fuzz.cpp): no sanitizer report, every
status documented, and the work-list, slot and partial-row arithmetic in
bounds for the heaviest selections each shape allows.  Needs no GPU: nothing
is launched."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_sel_amd", "csrc")


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        pytest.skip("hipcc not available")
    return path


@pytest.mark.slow
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_fuzz")
    cmd = [
        hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=all",
        "-Xarch_host", "-fno-omit-frame-pointer",
        f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
        os.path.join(CSRC, "fsa_api.hip"),
        os.path.join(ROOT, "tests", "sanitize", "host_fuzz.cpp"),
        os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp"),
        "-o", exe,
    ]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=600)
    print(run.stdout)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
    assert run.stdout.startswith("iterations 3000 valid")
