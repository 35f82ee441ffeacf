"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): libgdn's sources are compiled as for the library, with the
sanitizers on the host side alone (device code is built without them), and
linked with a driver
(tests/abi_sanitize/check_abi.cpp) that exercises argument validation,
workspace sizing and planning through the C ABI, including a deterministic
fuzz of the problem fields.  Every call fails, sizes or plans before any HIP
call, so no GPU is needed."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_frame_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
HIP_SOURCES = ["gdn_chunked.hip", "gdn_recurrent.hip", "gdn_prologue.hip", "gdn_noalloc.hip"]
HOST_SOURCES = ["gdn_api.cpp", "gdn_profile.cpp", os.path.join(ROOT, "tests", "abi_sanitize", "check_abi.cpp")]


def _compile(cmd):
    return subprocess.run(cmd, capture_output=True, text=True)


@pytest.mark.slow
def test_abi_host_layer_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    # sanitizers on the host side only (each -fsanitize= right after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *san]
    device = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    jobs, objs = [], []
    for src in HIP_SOURCES + HOST_SOURCES:
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        jobs.append([HIPCC, *common, *(device if src in HIP_SOURCES else []), "-c", path, "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=4) as ex:
        for r in ex.map(_compile, jobs):
            assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "check_abi")
    r = _compile([HIPCC, "--offload-arch=gfx950", *san, "-o", exe, *objs])
    assert r.returncode == 0, r.stdout + r.stderr
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "driver was not instrumented"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi host checks passed" in r.stdout, r.stdout + r.stderr
