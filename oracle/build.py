"""Build the scalar CPU oracle (test infrastructure) into oracle/liboracle.so.

Built with plain gcc at -O2 with floating-point contraction off and no
fast-math, so that every fp32 operation in oracle.c rounds once, in source
order.  Nothing here is shared with the GPU library's build.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-semantic-interposition", "-ffp-contract=off",
          "-fno-fast-math", "-fno-math-errno", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile `src` into the shared library `out` and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*(sys.argv[1:2] or [])))
