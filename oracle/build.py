"""Compile the fp64 CPU oracle (test infrastructure) with gcc.

The oracle is plain C with OpenMP over independent (batch, channel) pairs;
no fast-math or other value-changing flags are used.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mamba_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmamba_oracle.so")
SSD_SRC = os.path.join(HERE, "mamba2_oracle.c")
SSD_LIB = os.path.join(OUT_DIR, "libmamba2_oracle.so")


def build_all():
    """Compile every oracle library (Mamba-1 scan and Mamba-2 SSD)."""
    return [build(), build(SSD_SRC, SSD_LIB)]


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out` and return its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-Wall", "-Wextra", *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_all())
