"""Build the gfx950 HIP library libssmscan.so in-tree with hipcc.

All HIP code is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the kernels only issue scalar fp32 VALU
operations, transcendentals through the hardware exp2/log2/rcp instructions,
and bf16 conversions through v_cvt_pk_bf16_f32.  The device assembly of every
build is checked for DPP hazards (dpp_hazards) before the library is linked.
"""
import glob
import os
import re
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


# gfx9 DPP hazards (wait states a DPP instruction needs after a VALU write):
# 2 after a VALU write of its DPP source VGPR, 5 after a VALU write of EXEC.
# The compiler inserts these for the DPP instructions it emits itself; the
# kernels' inline-asm DPP FMA (common.hpp, fmac_row_bcast) relies on its source
# being written by loads only, so every build checks the generated assembly.
_DPP_SRC_WAIT, _DPP_EXEC_WAIT = 2, 5


def _vgprs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm: str) -> list:
    """DPP reads too close after a VALU write of their source VGPR (or of EXEC)
    in gfx9 assembly text.  Each instruction is one wait state, s_nop N is N+1.
    After a label the predecessors are unknown: an inline-asm DPP instruction
    there counts as a hazard unless enough wait states precede it in the block
    (compiler-emitted ones are covered by the compiler).  Returns a list of
    (line number, instruction, reason)."""
    found = []
    hist = []  # recent (wait states, written vgprs, writes exec, is label)
    in_asm = False
    for no, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if t.endswith(":") and not t.startswith(";"):
            hist.append((0, set(), False, True))
            continue
        if not t or t.startswith((";", ".", "#")):
            continue
        t = t.split(";")[0].strip()
        op = t.split()[0]
        args = [a.strip() for a in t[len(op):].split(",")]
        if op == "s_nop":
            hist.append((int(args[0], 0) + 1, set(), False, False))
            continue
        if "_dpp" in op:
            src0 = _vgprs(args[1].split()[0]) if len(args) > 1 else set()
            ws = 0
            for w, dst, wexec, label in reversed(hist):
                if ws >= _DPP_EXEC_WAIT:
                    break
                if label:
                    if in_asm and ws < _DPP_EXEC_WAIT:
                        found.append((no, t, "inline-asm DPP within 5 wait states of a label"))
                    break
                if wexec:
                    found.append((no, t, "VALU write of EXEC %d wait states before" % ws))
                    break
                if ws < _DPP_SRC_WAIT and dst & src0:
                    found.append((no, t, "VALU write of its source %d wait states before" % ws))
                    break
                ws += w
        is_valu = op.startswith("v_")
        dst = _vgprs(args[0]) if is_valu and args and args[0] else set()
        wexec = is_valu and (op.startswith("v_cmpx") or (args and args[0].startswith("exec")))
        hist.append((1, dst, wexec, False))
        hist = hist[-16:]
    return found


def check_dpp_hazards(objdir: str) -> None:
    for path in sorted(glob.glob(os.path.join(objdir, "*-hip-amdgcn-amd-amdhsa-" + ARCH + ".s"))):
        with open(path) as f:
            bad = dpp_hazards(f.read())
        if bad:
            lines = "\n".join(f"  line {n}: {t}  ({why})" for n, t, why in bad[:10])
            raise RuntimeError(f"DPP hazard in {path} ({len(bad)} found):\n{lines}")


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    """Compile every csrc/*.hip to an object (in parallel), check the device
    assembly for DPP hazards and link libssmscan.so."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = hipcc_path()
    jobs = jobs or max(1, min(len(sources), os.cpu_count() or 1))
    objs = [os.path.join(objdir, os.path.basename(src)[:-4] + ".o") for src in sources]
    # -save-temps=obj leaves the device assembly beside each object
    cmds = [[hipcc, *compile_flags(), *extra, "-save-temps=obj", "-c", "-o", obj, src]
            for src, obj in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    check_dpp_hazards(objdir)
    for junk in glob.glob(os.path.join(objdir, "*")):
        if junk.endswith((".bc", ".hipi", ".out", ".hipfb", ".resolution.txt")) or "-host-" in junk:
            os.remove(junk)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
