"""Build step for the C oracle (test infrastructure): gcc + OpenMP, fp64, -O2.

Plain compiler optimisation only; the source is the untuned loop nest.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build_c_oracle(verbose: bool = False) -> str:
    src = os.path.join(HERE, "gdn_oracle.c")
    out = os.path.join(HERE, "libgdn_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_c_oracle(verbose=True))
