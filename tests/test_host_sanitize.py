"""Host code under sanitizers (no GPU): the C-ABI front end and the scheduler
(api.cpp, schedule.cpp) built with g++ -fsanitize=address,undefined, with the
HIP launchers replaced by host stubs (tests/host_sanitize/stubs.cpp), then the
whole ABI test file (argument validation of every entry point, the scheduler
and key-structure sweeps against the oracle) run against that build in a
child process.  Any sanitizer report fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_31_amd", "csrc")


def _runtime(name):
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if _runtime("libasan.so") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ with AddressSanitizer and the ROCm headers are needed")
    out = str(tmp_path_factory.mktemp("host_sanitize") / "libvdn_local_attn_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "schedule.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "stubs.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


RUNNER = """
import sys
sys.path.insert(0, {root!r})
from block_sparse_attention_31_amd import binding
binding.LIB_PATH = {lib!r}
import pytest
rc = pytest.main([{abi!r}, "-q", "-x", "-p", "no:cacheprovider"])
print("loaded:", binding.lib()._name, flush=True)
sys.exit(int(rc))
"""


def test_abi_suite_under_asan_and_ubsan(asan_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = RUNNER.format(root=ROOT, lib=asan_lib, abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=600)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert f"loaded: {asan_lib}" in r.stdout
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
