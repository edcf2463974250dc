"""Build the CPU oracle (test infrastructure only) with gcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
