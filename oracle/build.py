"""Compile the CPU oracle (qgemv_oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qgemv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# IEEE division, no contraction into FMA, subnormals kept (no -ffast-math).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra=(), out=LIB, defines=()):
    cmd = ["gcc", *CFLAGS, *extra, *[f"-D{d}" for d in defines], SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
