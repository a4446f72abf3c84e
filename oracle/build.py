"""Builds the fp64 oracle library (test infrastructure; see oracle/__init__.py)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build():
    """gcc -O2 without fast-math: IEEE fp64, no reassociation of the sums."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
