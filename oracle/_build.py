"""Build the CPU oracle (plain C, IEEE binary32 arithmetic, no contraction)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", SO, os.path.join(HERE, "oracle.c")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
