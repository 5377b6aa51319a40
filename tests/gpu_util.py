"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path, run the oracle, compare.

Error measure: for outputs g (GPU) and o (oracle, fp64),
    err = max_i |g_i - o_i| / max(|o_i|, rms(o)),
computed separately for y and the final state.  The floor at the tensor's
RMS keeps near-zero outputs (y ~ 0 where the SiLU gate is ~ 0) from
dominating.  Any non-finite GPU value fails.  Tolerances: 1e-4 for fp32
storage, 2e-2 for bf16 storage.
"""
import os
import sys

import numpy as np
import torch

from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

TOL = {"f32": 1e-4, "bf16": 2e-2}


def device():
    return torch.device("cuda:0")


def say(msg):
    """Name the case before each GPU step (flushed), so a failing run still says what it was doing."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device(), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def to_dev_f32(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device())


def rel_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), max(rms, 1e-30))
    return float(np.max(np.abs(g - o) / den))


def gpu_scan(x, dtype, softplus=True, with_D=True, with_bias=True, with_z=True, final=True):
    """Run ssm_scan_fwd on numpy inputs; returns float64 numpy (y, final_state or None)."""
    dev_in = dict(u=to_dev(x["u"], dtype), delta=to_dev(x["delta"], dtype), B=to_dev(x["B"], dtype),
                  C=to_dev(x["C"], dtype), z=to_dev(x["z"], dtype) if with_z else None)
    y, fs = ops.ssm_scan_fwd(dev_in["u"], dev_in["delta"], to_dev_f32(x["A"]), dev_in["B"], dev_in["C"],
                             D=to_dev_f32(x["D"]) if with_D else None, z=dev_in["z"],
                             delta_bias=to_dev_f32(x["delta_bias"]) if with_bias else None,
                             softplus=softplus, return_final_state=final)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    fs = fs.cpu().numpy().astype(np.float64) if fs is not None else None
    return y, fs


def oracle_scan(x, softplus=True, with_D=True, with_bias=True, with_z=True, nthreads=8):
    return R.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"] if with_D else None,
                      z=x["z"] if with_z else None, delta_bias=x["delta_bias"] if with_bias else None,
                      softplus=softplus, nthreads=nthreads)


def oracle_threads():
    """Threads for the oracle on whole workloads: the cores this process may use, at most 16."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


class _Env:
    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = os.environ.get(self.name)
        os.environ[self.name] = self.value

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = self.old


class Variant(_Env):
    """Temporarily force a launch variant (states per lane, wavefronts, chunks) through the library's override."""

    def __init__(self, npl, G, K=0):
        super().__init__("SSM_SCAN_VARIANT", f"{npl},{G},{K}")


class Chained(_Env):
    """Temporarily force chunks to chain their carries inside the scan launch (True) or not (False)."""

    def __init__(self, on):
        super().__init__("SSM_SCAN_CHAINED", "1" if on else "0")


class BlockLen(_Env):
    """Temporarily force the readout scan's tokens per block (16 or 32) where the variant has both."""

    def __init__(self, tb):
        super().__init__("SSM_SCAN_TB", str(tb))


class IndexOrder(_Env):
    """Temporarily launch packed sequences in index order instead of longest first."""

    def __init__(self):
        super().__init__("SSM_SCAN_ORDER", "0")


class BwdChained(_Env):
    """Temporarily allow (True) or forbid (False) the chained plan of the backward pass."""

    def __init__(self, on):
        super().__init__("SSM_BWD_CHAINED", "1" if on else "0")


class SsdChained(_Env):
    """Temporarily allow (True) or forbid (False) the chained plan of the SSD layer."""

    def __init__(self, on):
        super().__init__("SSM_SSD_CHAINED", "1" if on else "0")
