"""Build the retention C-ABI library (libretention.so) for gfx950 with hipcc.

Run ``python -m retnet_retention_msr_amd.build`` (or call ``build()``). The
library is written next to this file so it travels with the source tree.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libretention.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Keep the compiler from forming packed-fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: avoids copying state tiles between VGPRs and AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]

# Extra flags for single sources. The output kernel schedules better with the
# iterative ILP strategy; the state walk measured slower with it, so it keeps
# the default.
FILE_FLAGS = {
    "mfma_out.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the retention library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object, then link the shared library."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        cmd = [hipcc, *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError(f"link failed:\n{out.stdout}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _wait(item):
    src, proc = item
    out, _ = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    # The host pass does not know the packed-fp32 feature flag; that note is harmless.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if any(ln.strip() for ln in lines):
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
