"""Build the generator's shared libraries in-tree.

libk3gen_host.so: plain C (gcc, OpenMP), needed by the oracle side and by any
host-side input.  libk3gen_dev.so: the HIP fill kernels for gfx950 (hipcc),
used only where a whole expert bank is written straight into HBM.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HOST_LIB = os.path.join(HERE, "libk3gen_host.so")
DEV_LIB = os.path.join(HERE, "libk3gen_dev.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_host():
    tmp = HOST_LIB + ".tmp"
    _run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
          "-o", tmp, os.path.join(CSRC, "k3gen_host.c"), "-lm"])
    os.replace(tmp, HOST_LIB)


def build_dev():
    tmp = DEV_LIB + ".tmp"
    _run(["hipcc", *HIP_FLAGS, "-I", CSRC, "-o", tmp, os.path.join(CSRC, "k3gen_dev.hip")])
    os.replace(tmp, DEV_LIB)


def build():
    build_host()
    build_dev()


if __name__ == "__main__":
    build()
