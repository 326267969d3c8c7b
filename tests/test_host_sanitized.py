"""The C-ABI's host code (csrc/abi.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp is compiled with the host compiler and both sanitizers, together with
tests/sanitize/abi_host_checks.cpp, whose stub kernel launchers count launches instead of
touching a GPU. The program checks validation (every rejection launches nothing), the launch
sequence of a block and of the cached loop, the loop statistics, the mapping of a failed launch
to DIT_ERR_DEVICE (nothing launched after it) and the per-thread error state; it prints every
cache schedule it computed, which must equal the oracle's. Any sanitizer report fails the test.
"""

import os
import shutil
import subprocess

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


def _build(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "abi_host_checks")
    cmd = [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g", "-O1", "-Wall", "-Werror",
           os.path.join(ROOT, "audio_video_diffusion_dit_amd", "csrc", "abi.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_host_checks.cpp"),
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitized build failed:\n{r.stderr}"
    return exe


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = [l for l in r.stderr.splitlines() if "Sanitizer" in l or "runtime error" in l]
    assert not report, "\n".join(report[:20])
    fails = [l for l in r.stdout.splitlines() if l.startswith("FAIL")]
    assert not fails, "\n".join(fails[:20])
    assert r.returncode == 0, r.stderr[-2000:]
    done = [l for l in r.stdout.splitlines() if l.startswith("DONE")]
    assert done and done[0].split()[2] == "0"
    names = {0: "off", 1: "velocity", 2: "extrapolate"}
    n_sched = 0
    for line in r.stdout.splitlines():
        if not line.startswith("S "):
            continue
        parts = line.split()
        mode, s, e, rr, c, n = int(parts[1]), float(parts[2]), float(parts[3]), int(parts[4]), \
            int(parts[5]), int(parts[6])
        flags = parts[7] if len(parts) > 7 else ""
        want = O.cache_schedule(O.CachePolicy(names[mode], s, e, rr, c), n)
        assert flags == "".join("1" if h else "0" for h in want), line
        n_sched += 1
    assert n_sched > 8000
