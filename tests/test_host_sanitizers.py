"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources with the sanitizers applied to the host pass only (the gfx950
device code is compiled as usual and never launched), links tests/hostcheck/host_checks.cpp
against them and runs it: workspace-size queries over a grid of shapes, extreme ones
included, and calls that fail their host-side checks before anything is enqueued. No GPU
is needed or touched. Any sanitizer report ends the run with a nonzero status.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "verify_step_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_code_under_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    assert srcs
    objs = []
    jobs = []
    for s in srcs:
        o = str(tmp_path / (os.path.splitext(os.path.basename(s))[0] + ".o"))
        objs.append(o)
        jobs.append([HIPCC] + COMMON + SAN + ["-c", s, "-o", o])
    drv = str(tmp_path / "host_checks.o")
    jobs.append([HIPCC] + COMMON + SAN + ["-x", "hip", "-c",
                                          os.path.join(ROOT, "tests", "hostcheck",
                                                       "host_checks.cpp"), "-o", drv])
    workers = max(1, min(len(jobs), (os.cpu_count() or 2)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, str(tmp_path)), jobs))
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-arch=gfx950"] + SAN[:4] + [drv] + objs + ["-o", exe],
         str(tmp_path))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], cwd=str(tmp_path), capture_output=True, text=True, env=env,
                       timeout=300)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    shutil.rmtree(str(tmp_path), ignore_errors=True)
