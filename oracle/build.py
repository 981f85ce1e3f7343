"""Build the oracle's C part (test infrastructure; never linked by the HIP library).

    python -m oracle.build      -> oracle/libjm_oracle.so  (gcc, -O2, OpenMP)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libjm_oracle.so")
SRC = [os.path.join(HERE, "scan_ref.c")]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-o", LIB + ".tmp", *SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
