"""Build librecurrent_nn_amd.so for gfx950 (MI355X) in-tree.

Every HIP source is compiled by hipcc for --offload-arch=gfx950 with
-ffp-contract=off (the gate arithmetic must not fuse multiplies into adds)
and with the packed-fp32 instructions disabled; the host-only plan code is
plain C++17.  Objects go to _build/ (not versioned), the library next to this
file, where the Python binding loads it.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "recurrent_nn_amd")
LIB = os.path.join(HERE, "librecurrent_nn_amd.so")

ARCH = os.environ.get("RNN_AMD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]

# every .hip file of csrc (the step-loop instantiations are split over several
# translation units so that they compile in parallel) and the HIP host code
HIP_SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")) + ["run.cpp"]
CXX_SOURCES = ["plan.cpp"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    if src in CXX_SOURCES:
        cmd = ["g++", *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), HIP_SOURCES + CXX_SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    t = build(verbose="-v" in sys.argv)
    print(t)
