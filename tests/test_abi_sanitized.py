"""The entry points' host code (argument validation, dispatch, error text)
built with AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel
launchers replaced by host-only stand-ins (tests/sanitize/), and driven through
invalid, extreme (INT_MAX sizes), empty and valid arguments. Runs on the host;
no GPU code is built or run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
API = os.path.join(ROOT, "online_softmax_attention_cascaded_amd", "csrc", "rf_api.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

# The sanitizers apply to the host compilation only (each flag after -Xarch_host).
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
         *HOST_SAN]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_entry_points_under_sanitizers(tmp_path):
    objs = []
    for src, extra in ((API, ['-DRF_BUILD_ID="sanitized"']),
                       (os.path.join(HERE, "stub_launchers.cpp"), []),
                       (os.path.join(HERE, "driver.cpp"), [])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        objs.append(obj)
    exe = str(tmp_path / "driver")
    res = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
                          "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0 and "passed: 0 failure(s)" in res.stdout, res.stdout + res.stderr
