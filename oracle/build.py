"""Compile the C oracle (oracle/libkda_ref.so) with gcc. Test infrastructure only."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    src = os.path.join(HERE, "kda_ref.c")
    out = os.path.join(HERE, "libkda_ref.so")
    tmp = out + ".tmp"
    # portable x86-64 code: the library is built here and also runs on other hosts
    cmd = ["gcc", "-O3", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
