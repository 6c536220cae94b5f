"""Compile the C oracle into ``oracle/liboracle.so`` (test infrastructure)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-std=c11", "-O2", "-Wall", "-Wextra", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-fPIC", "-shared"]


def build(force=True):
    """Build the oracle library (always rebuilds unless force is False)."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc"] + FLAGS + [os.path.join(HERE, "oracle.c"), "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
