"""Compile the gfx950 library libmps_adamw.so in-tree with hipcc.

Flags that matter for the arithmetic:
  -ffp-contract=off      no fused multiply-add: each fp32 operation of the
                         update rounds once, in source order;
  (defaults kept)        correctly rounded fp32 division and sqrt, IEEE
                         denormals, no fast-math.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed fp32 instructions in the generated code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmps_adamw.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "kernels_q8.hip"),
           os.path.join(CSRC, "api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(out: str = LIB, extra=()) -> str:
    """Compile every source into `out` (atomically replaced) and return it."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def isa(out_dir: str) -> list:
    """Write the gfx950 assembly of kernels.hip under out_dir (for reading)."""
    os.makedirs(out_dir, exist_ok=True)
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", "-o", os.path.join(out_dir, "kernels.s"),
           SOURCES[0]]
    subprocess.run(cmd, check=True)
    return [os.path.join(out_dir, "kernels.s")]


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--isa":
        print(isa(sys.argv[2]))
    else:
        print(build())
