"""Compile the oracle's plain-C helpers into oracle/liboracle_p8f.so (gcc).

Test infrastructure: the library is the oracle's own, never the product's."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_p8f.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           os.path.join(HERE, "viterbi_ref.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
