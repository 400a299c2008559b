"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): every source is built with the sanitizers on its host side only
(device code as usual, at -O1 to keep the build short), linked with the C driver
tests/host/host_checks.c, and run.  The driver walks the host-side paths
(layouts, workspace sizes, status strings, each entry point's argument checks);
the test fails on any sanitizer report or any unexpected return code."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a16_grouped_expert_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
# each sanitizer flag right after -Xarch_host: host code only, never the GPU objects
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"


@pytest.mark.timeout(900)
def test_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC] + SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC] + flags + ["-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_checks.o")
    _run([HIPCC, "-x", "c", "-O1", "-g", "-I", INCLUDE, "-c", os.path.join(ROOT, "tests", "host", "host_checks.c"),
          "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", "-fno-gpu-rdc"] + SAN + ["-o", exe, drv] + objs)
    env = dict(os.environ)
    # the HIP runtime's own allocations live until exit: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failures" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
