"""Build ``libsgemm.so`` (the gfx950 kernels and the C interface) in-tree.

Every source is compiled with hipcc for gfx950 only.  Packed FP32 VALU
instructions are disabled (``-packed-fp32-ops``): the kernels use scalar
FP32 FMA on the vector path and FP32 MFMA on the matrix path.

``build(lds_poison=True)`` makes the race-check variant
``libsgemm_ldspoison.so`` (SGEMM_LDS_POISON=1): before each direct-to-LDS
refill of a pipeline stage, every wave first writes NaN into exactly the LDS
bytes its loads will fill.  A read of a stage after the barrier that freed
it, or of a refill before its loads have landed, then sees NaN instead of
stale but plausible data, and the parity tests fail.  Load it with
SGEMM_LIBRARY=<path> to run the test suite against it.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsgemm.so")
LIB_POISON = os.path.join(HERE, "libsgemm_ldspoison.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["api.cpp", "mfma.hip", "valu.hip", "skinny.hip", "simple.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def _compile(src: str, extra=(), bdir=BUILD) -> str:
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    lines = [ln for ln in r.stderr.splitlines() if noise not in ln and "(ignoring feature)" not in ln]
    if any(ln.strip() for ln in lines):
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = False, jobs: int = 8, lds_poison: bool = False) -> str:
    bdir = BUILD + ("_ldspoison" if lds_poison else "")
    lib = LIB_POISON if lds_poison else LIB
    extra = ["-DSGEMM_LDS_POISON=1"] if lds_poison else []
    os.makedirs(bdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, bdir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def asm(src: str, out: str, lds_poison: bool = False) -> None:
    """Write the gfx950 assembly of one source (for register and schedule inspection)."""
    extra = ["-DSGEMM_LDS_POISON=1"] if lds_poison else []
    cmd = [HIPCC, *COMMON, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)


if __name__ == "__main__":
    print(build(verbose=True, lds_poison="--lds-poison" in sys.argv[1:]))
