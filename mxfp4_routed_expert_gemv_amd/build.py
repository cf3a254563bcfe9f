"""Compile libk3moe.so (every HIP kernel + the C-ABI host code) for gfx950,
in-tree, with hipcc.  Objects are compiled in parallel, then linked."""
import concurrent.futures
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libk3moe.so")

SOURCES = ["abi.cpp", "route.hip", "permute.hip", "gemv.hip", "mfma.hip", "mxscale.hip", "combine.hip",
           "noalloc.hip", "rvq.hip", "cache.hip", "shared_gemm.hip"]

# -ffp-contract=off: every fused multiply-add is written out, so each template
# variant rounds identically.  -packed-fp32-ops off: packed fp32 add/mul/fma
# stay out of every kernel.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
               "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(src, obj):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ["hipcc", *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    warnings = [ln for ln in r.stderr.splitlines()
                if "warning" in ln and "packed-fp32-ops" not in ln]
    return warnings


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="k3moe_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            futs = [ex.submit(_compile, s, o) for s, o in zip(SOURCES, objs)]
            for f in futs:
                for w in f.result():
                    if verbose:
                        print(w)
        out_tmp = LIB + ".tmp"
        cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
