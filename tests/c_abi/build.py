"""Build tests/c_abi/step_from_c, the plain C program that drives the library
through its C ABI (test infrastructure: it links the oracle as its checker).

gcc compiles it against include/mps_adamw.h and the HIP runtime's C API and
links the built libmps_adamw.so and liboracle.so, found at run time next to
the repository through an $ORIGIN-relative search path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "step_from_c.c")
EXE = os.path.join(HERE, "step_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    rpath = ":".join(["$ORIGIN/../../mixed_precision_sharded_amd", "$ORIGIN/../../oracle",
                      os.path.join(ROCM, "lib")])
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           "-o", tmp, SRC,
           "-L" + os.path.join(ROOT, "mixed_precision_sharded_amd"), "-lmps_adamw",
           "-L" + os.path.join(ROOT, "oracle"), "-loracle",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + rpath]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*(sys.argv[1:2] or [])))
