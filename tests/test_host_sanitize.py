"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds libfdllm's sources with the host half instrumented (hipcc
-Xarch_host -fsanitize=address / undefined; the gfx950 device code is built
as usual and never runs) together with tests/sanitize/reject_paths.cpp, a
driver that calls every C-ABI entry point with arguments it must reject and
runs the workspace planners over valid geometries up to the header's
limits, and checks that the driver exits cleanly with no sanitizer report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_wise_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "reject_paths.cpp")
SOURCES = ["fdllm_api.cpp", "block_attn.hip", "unmask.hip", "kv_refresh.hip", "lmhead.hip", "validate.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def test_c_abi_rejection_paths_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    objs = []
    jobs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        jobs.append([hipcc, *COMMON, *DEVICE, *SAN, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj])
    drv = str(tmp_path / "driver.o")
    jobs.append([hipcc, *COMMON, *SAN, "-c", DRIVER, "-o", drv])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(_run, jobs))
    exe = str(tmp_path / "reject_paths")
    _run([hipcc, "--offload-arch=gfx950", *SAN, *objs, drv, "-o", exe])
    env = dict(os.environ)
    # the HIP runtime's own allocations are not this library's to account for
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    print(out)
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0, out
    assert " 0 failures" in r.stdout
