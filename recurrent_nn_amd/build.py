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
             # the flag and counter atomics are issued by one lane already:
             # no lane-count reduction code in the step loops
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-Wno-unused-command-line-argument"]

# The instantiation tables of the step loop: one source compiled once per
# kernel family and activation set (recurrence_inst.hip), so that they
# compile in parallel.
INST = "recurrence_inst.hip"
INST_UNITS = [(fam, act) for fam in range(5) for act in range(5)]

# Device flags of single kernel families.  The streamed step loops (families
# 1 and 2) keep the matrix accumulators in ordinary vector registers: in the
# default form the register allocator moved part of them between
# accumulation registers at every back edge of the k loop (60 extra vector
# instructions per 192 MFMAs with all row tiles of a 128-row block active).
FAMILY_FLAGS = {1: ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                2: ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# (source, extra flags, object name) of every translation unit: the .hip
# files of csrc, the instantiation units, the HIP host code
HIP_UNITS = ([(f, [], f + ".o") for f in sorted(os.listdir(CSRC))
              if f.endswith(".hip") and f != INST] +
             [(INST, [f"-DRNN_FAMILY={fam}", f"-DRNN_ACT={act}", *FAMILY_FLAGS.get(fam, [])],
               f"recurrence_inst_f{fam}_a{act}.o") for fam, act in INST_UNITS] +
             [("run.cpp", [], "run.cpp.o")])
CXX_UNITS = [("plan.cpp", [], "plan.cpp.o")]


def _compile(unit, verbose, build_dir=BUILD, defs=()):
    src, extra, oname = unit
    obj = os.path.join(build_dir, oname)
    path = os.path.join(CSRC, src)
    if unit in CXX_UNITS:
        cmd = ["g++", *COMMON, *defs, *extra, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *HIP_FLAGS, *defs, *extra, "-x", "hip", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


# The instrumented build (cycle stamps of one workgroup's steps, read back by
# `bench.py --stamps`): the same sources with -DRNN_STAMPS, its own objects
# and library file.  Never loaded unless RNN_AMD_LIB names it.
STAMPS_BUILD = os.path.join(ROOT, "_build", "recurrent_nn_amd_stamps")
STAMPS_LIB = os.path.join(HERE, "librecurrent_nn_amd_stamps.so")


def build(verbose: bool = False, jobs: int = 8, stamps: bool = False) -> str:
    build_dir, lib, defs = (STAMPS_BUILD, STAMPS_LIB, ["-DRNN_STAMPS"]) if stamps else (BUILD, LIB, [])
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose, build_dir, defs), HIP_UNITS + CXX_UNITS))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    t = build(verbose="-v" in sys.argv, stamps="--stamps" in sys.argv)
    print(t)
