"""Build the gfx950 HIP library libssmscan.so in-tree with hipcc.

All HIP code is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the kernels only issue scalar fp32 VALU
operations, transcendentals through the hardware exp2/log2/rcp instructions,
and bf16 conversions through v_cvt_pk_bf16_f32.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libssmscan.so")
SRC = os.path.join(HERE, "csrc", "ssm_scan.hip")
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


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc_path(), *compile_flags(), *extra, "-shared", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
