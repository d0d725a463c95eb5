"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

capi.hip (argument validation, launch planning, workspace sizing, error strings)
is compiled host-only with both sanitizers and linked against stub launchers
(tests/sanitize/capi_driver.cpp) that check each launch plan against the shapes
the kernels assume.  The driver sweeps pseudo-random valid and invalid arguments
through every entry point; any sanitizer report or failed check fails the test.
No GPU is involved: the stubs replace every kernel launch.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "token_tree_verification_02_amd")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_capi_host_layer_under_sanitizers(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    # sanitizers on the host side only (the sanitizer binary holds no device code)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", *inc, *san]
    objs = []
    for src, obj in ((os.path.join(PKG, "csrc", "capi.hip"), "capi.o"),
                     (os.path.join(ROOT, "tests", "sanitize", "capi_driver.cpp"), "driver.o")):
        out = str(tmp_path / obj)
        r = subprocess.run([cc, *common, "-c", src, "-o", out], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(out)
    exe = str(tmp_path / "capi_driver")
    r = subprocess.run([cc, *san[:4], *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout[-2000:] + r.stderr[-4000:])
