"""Build the CPU oracle (test infrastructure only) with the host C compiler.

The oracle is plain C11, single-threaded, compiled without floating-point
contraction or fast-math so that every fp32 step is one correctly rounded
operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "polestar_oracle.c")
LIB = os.path.join(HERE, "libpolestar_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
           "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
