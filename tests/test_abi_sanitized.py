"""The C ABI's validation and planning under the address and undefined-behaviour sanitizers (CPU only).

api.cpp and plan.cpp hold all host logic of the library (argument checks,
chunk and workspace planning, the backward's buffer plan); they include only
host headers, so a host compiler builds them. Linked with stub launchers
(tests/host_shim/launch_stubs.cpp) into a shared object with
-fsanitize=address,undefined, they are driven by test_abi_host.py in a child
interpreter that preloads the ASan runtime; any sanitizer report aborts the
child and fails this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "retnet_retention_msr_amd", "csrc")


def _asan_runtime():
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP runtime headers")
def test_abi_host_checks_pass_under_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("no ASan runtime for g++")
    lib = tmp_path / "libretention_host.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "host_shim", "launch_stubs.cpp"), "-o", str(lib)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env.update(RETENTION_ABI_TEST_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in r.stdout and "skipped" not in r.stdout.splitlines()[-1], report
