"""Build the gfx950 HIP library libssmscan.so in-tree with hipcc.

All HIP code is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the kernels only issue scalar fp32 VALU
operations, transcendentals through the hardware exp2/log2/rcp instructions,
and bf16 conversions through v_cvt_pk_bf16_f32.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libssmscan.so")
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", os.path.join(HERE, "csrc")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    """Compile every csrc/*.hip to an object (in parallel) and link libssmscan.so."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = hipcc_path()
    jobs = jobs or max(1, min(len(sources), os.cpu_count() or 1))
    objs = [os.path.join(objdir, os.path.basename(src)[:-4] + ".o") for src in sources]
    cmds = [[hipcc, *compile_flags(), *extra, "-c", "-o", obj, src] for src, obj in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
