"""Build the fp64 CPU oracle (test infrastructure only) into oracle/liboracle.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zl_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile zl_oracle.c with gcc (-O2, OpenMP, strict IEEE) and return the path."""
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
