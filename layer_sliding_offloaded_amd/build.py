"""Build libsf.so in-tree: HIP kernels for gfx950 with hipcc, host code with g++.

Usage: python -m layer_sliding_offloaded_amd.build   (or build() from Python)
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsf.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["gemm.hip", "attention.hip", "attn_direct.hip", "rowops.hip"]
HOST_SOURCES = ["api.cpp", "layout.cpp", "engine.cpp", "adam.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# attention: MFMA accumulators in VGPRs (the softmax arithmetic reads them;
# in AGPRs every tile paid a copy per accumulator register)
HIP_EXTRA = {"attn_direct.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
# -ffp-contract=off: host Adam rounds every operation exactly like the device kernel
HOST_EXTRA = {"adam.cpp": ["-mavx2", "-mfma", "-mf16c", "-fno-math-errno", "-ffp-contract=off"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=None):
    """Compile every source and link libsf.so; always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([hipcc, *HIPCC_FLAGS, *HIP_EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([cxx, *CXX_FLAGS, *HOST_EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
