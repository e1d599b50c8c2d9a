"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled as for the library (gfx950 device code
included), with both sanitizers on the host compilation only, and linked with
tests/host_abi_driver.c, which calls every entry point with arguments that fail
validation, the workspace-size queries over the whole accepted shape range and the
diagnostic hooks.  The sanitizers abort on their first report; the driver exits
non-zero on any unexpected status."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tv_loss_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["capi.hip", "verify.hip", "tv_loss.hip"]
HIPCC = "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
# each sanitizer flag applies to the host compilation only (-Xarch_host before it)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_abi_under_sanitizers(tmp_path):
    def compile_(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               *SAN, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_, SOURCES))
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([HIPCC, "-x", "c", "-O1", "-g", "-I", INCLUDE, *SAN, "-c",
                        os.path.join(ROOT, "tests", "host_abi_driver.c"), "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", *SAN, drv, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
