"""Compile the plain C oracle into ``oracle/libnano_oracle.so`` (test
infrastructure: building the checker is not using it)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libnano_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "nano_oracle.c")
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", src, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
