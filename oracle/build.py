"""Build the CPU oracle (test infrastructure only).

Compiles ``gpt2_oracle.c`` twice with gcc and OpenMP: once with REAL=float
(``_build/liboracle_f32.so``, the fp32 oracle) and once with REAL=double
(``_build/liboracle_f64.so``, used for finite-difference checks).  Plain -O3
for generic x86-64, no fast-math, so the library runs on any x86-64 host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")
SRC = os.path.join(HERE, "gpt2_oracle.c")


def lib_path(precision: str) -> str:
    return os.path.join(BUILD, f"liboracle_{precision}.so")


def build(verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    for prec, real in (("f32", "float"), ("f64", "double")):
        out = lib_path(prec)
        tmp = out + ".tmp"
        cmd = ["gcc", "-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", f"-DREAL={real}",
               SRC, "-o", tmp, "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
