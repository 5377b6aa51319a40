"""GPU check of ssm_scan_fwd_noalloc, the forward that allocates nothing: its workspace is a static device array
of the library (one per GPU), so it serves callers that cannot allocate.  Called through the C ABI and compared
with ssm_scan_fwd on the same inputs (same kernels and plan: bitwise equal) and with the oracle, on two calls in
a row, the second smaller than the first (the array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, oracle_scan, rel_err, say, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu


def _noalloc(lib, g, y, fs, dtype_code, stream):
    batch, L, dim = g["u"].shape
    N = g["A"].shape[1]
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return lib.ssm_scan_fwd_noalloc(p(g["u"]), p(g["delta"]), p(g["A"]), p(g["B"]), p(g["C"]), p(g["D"]),
                                    p(g["z"]), p(g["delta_bias"]), 1, p(y), p(fs), batch, L, dim, N, dtype_code,
                                    stream.cuda_stream)


def _inputs(x, dtype):
    return dict(u=to_dev(x["u"], dtype), delta=to_dev(x["delta"], dtype), A=to_dev_f32(x["A"]),
                B=to_dev(x["B"], dtype), C=to_dev(x["C"], dtype), D=to_dev_f32(x["D"]), z=to_dev(x["z"], dtype),
                delta_bias=to_dev_f32(x["delta_bias"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_allocating_entry_point(dtype):
    lib = ops.lib()
    code = ops.SSM_DTYPE_BF16 if dtype == "bf16" else ops.SSM_DTYPE_F32
    stream = torch.cuda.current_stream()
    cases = [(5, 700, 64 * 64, 16),   # 320 tiles: the chained plan (flags, carries)
             (2, 300, 200, 16)]       # smaller, every tile whole: a different layout over the same array
    for i, (batch, L, dim, N) in enumerate(cases):
        rng = np.random.default_rng(900 + i)
        x = I.random_scan_inputs(rng, batch, L, dim, N, dtype=dtype)
        g = _inputs(x, dtype)
        y_ref, fs_ref = ops.ssm_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                                         delta_bias=g["delta_bias"])
        y = torch.empty_like(y_ref)
        fs = torch.empty_like(fs_ref)
        say(f"noalloc call {i}: {batch}x{L}x{dim}x{N} {dtype}")
        rc = _noalloc(lib, g, y, fs, code, stream)
        assert rc == ops.SSM_OK, ops.ssm_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(fs, fs_ref)
        if i == 1:   # the small case also against the oracle, at the forward's tolerance
            yo, fo = oracle_scan(x)
            ey = rel_err(y.float().cpu().numpy(), yo)
            ef = rel_err(fs.cpu().numpy(), fo)
            print(f"[parity] noalloc {dtype}: y {ey:.2e} state {ef:.2e}", flush=True)
            assert ey <= TOL[dtype] and ef <= TOL[dtype]
