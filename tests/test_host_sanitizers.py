"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the C-ABI host code (hylra_api.cpp: validation, workspace layout,
split plans, the policy loops and the policy DP) and the C oracle with
``-fsanitize=address,undefined`` using g++/gcc, links them with host stand-ins
for the device side (tests/sanitize/device_stubs.cpp: every launch touches its
whole device-memory footprint on host buffers of the documented sizes), and
runs tests/sanitize/host_driver.c.  Any sanitizer report aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_host_code_under_asan_ubsan(tmp_path):
    inc = os.path.join(ROOT, "include")
    api = os.path.join(ROOT, "sparse_layer_reuse_amd", "csrc", "hylra_api.cpp")
    stubs = os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp")
    driver = os.path.join(ROOT, "tests", "sanitize", "host_driver.c")
    orc = os.path.join(ROOT, "oracle", "hylra_oracle.c")
    objs = []
    for src, cc, std in ((api, "g++", "-std=c++17"), (stubs, "g++", "-std=c++17"),
                         (driver, "gcc", "-std=c11"), (orc, "gcc", "-std=c99")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [cc, std, "-I", inc, "-Wall", "-Wno-unused-function", "-c", src, "-o", obj] + SAN
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    r = subprocess.run(["g++", "-o", exe] + objs + SAN + ["-lm"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
