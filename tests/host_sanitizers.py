"""Run the CPU test suite against host builds instrumented with AddressSanitizer
and UndefinedBehaviorSanitizer.  CPU only: nothing here runs on a GPU.

Instrumented (host code only, clang's runtime):
  - the oracle, oracle/rnn_oracle.c (without OpenMP: one thread, so that the
    sanitizers see every access in one thread);
  - the library's host code: plan.cpp (attribute parsing, checks, tiling,
    workspace layout) and run.cpp (the argument checks of rnn_run and
    rnn_cell_run, the launch sequence); the kernels' translation units are
    linked unchanged from the normal build.
Both go to _build/hostsan/, and the suite runs with the sanitizer runtime
preloaded and RNN_ORACLE_LIB / RNN_AMD_LIB pointing at those builds.  The
mutation test (which builds its own oracle copies) is left out.

    python tests/host_sanitizers.py [extra pytest arguments]
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from recurrent_nn_amd import build as libbuild  # noqa: E402

OUT = os.path.join(ROOT, "_build", "hostsan")
LLVM = "/opt/rocm/llvm"
CLANG, CLANGXX = os.path.join(LLVM, "bin", "clang"), os.path.join(LLVM, "bin", "clang++")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]
# for hipcc, every sanitizer option applies to the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-g"]


def run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def runtime():
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(out):
        import glob
        found = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so"))
        if not found:
            raise SystemExit("clang's AddressSanitizer runtime is not installed")
        out = found[0]
    return out


def build():
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = os.path.join(OUT, "librnn_oracle.so")
    run([CLANG, "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-Wno-unknown-pragmas", *SAN, "-o", oracle_lib,
         os.path.join(ROOT, "oracle", "rnn_oracle.c"), "-lm"])
    # the normal build provides the kernels' objects
    libbuild.build()
    inc = ["-I", os.path.join(ROOT, "include")]
    csrc = libbuild.CSRC
    plan_o, run_o = os.path.join(OUT, "plan.o"), os.path.join(OUT, "run.o")
    run([CLANGXX, "-std=c++17", "-fPIC", *SAN, *inc, "-c", os.path.join(csrc, "plan.cpp"),
         "-o", plan_o])
    run([libbuild.HIPCC, "-std=c++17", "-fPIC", "-O1", *inc, *libbuild.HIP_FLAGS, *HOST_SAN,
         "-x", "hip", "-c", os.path.join(csrc, "run.cpp"), "-o", run_o])
    objs = [os.path.join(libbuild.BUILD, o) for _, _, o in libbuild.HIP_UNITS
            if o != "run.cpp.o"]
    lib = os.path.join(OUT, "librecurrent_nn_amd.so")
    run([libbuild.HIPCC, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", "-o", lib,
         plan_o, run_o, *objs])
    return oracle_lib, lib


def main(argv):
    oracle_lib, lib = build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime(), RNN_ORACLE_LIB=oracle_lib, RNN_AMD_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x",
           "-m", "not gpu", "-k", "not mutation", *argv]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
