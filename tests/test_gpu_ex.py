"""GPU parity of ssm_scan_fwd_ex (initial states, packed variable-length sequences) against the oracle.

Compared element by element with oracle ref.scan_fwd_ex (pinned in
test_oracle_ex.py) on the same seeded inputs, with the tolerances of the
forward tests (1e-4 fp32, 2e-2 bf16; the final state always fp32, 1e-4 unless
the inputs were rounded to bf16).
"""
import numpy as np
import pytest
import torch

from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, Chained, IndexOrder, Variant, rel_err, say, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu


def _gpu_ex(x, dtype, h0=None, cu=None):
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int64, device="cuda:0")
    y, fs = ops.ssm_scan_fwd_ex(to_dev(x["u"], dtype), to_dev(x["delta"], dtype), to_dev_f32(x["A"]),
                                to_dev(x["B"], dtype), to_dev(x["C"], dtype), D=to_dev_f32(x["D"]),
                                z=to_dev(x["z"], dtype), delta_bias=to_dev_f32(x["delta_bias"]),
                                initial_state=to_dev_f32(h0), cu_seqlens=cu_t)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def _check(x, dtype, h0=None, cu=None, label=""):
    say(f"ex {label} shape={x['u'].shape} {dtype}")
    yg, fg = _gpu_ex(x, dtype, h0, cu)
    yo, fo = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                           delta_bias=x["delta_bias"], initial_state=h0, cu_seqlens=cu, nthreads=8)
    ey, ef = rel_err(yg, yo), rel_err(fg, fo)
    print(f"[parity] ex {label}: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL[dtype] and ef <= TOL[dtype], (ey, ef)


def _h0(rng, rows, dim, N):
    return np.asarray(rng.standard_normal((rows, dim, N)) * 0.5, np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("plan", ["whole", "pairs", "chained"])
def test_initial_state_every_plan(plan, dtype):
    rng = np.random.default_rng(500 + len(plan) + (3 if dtype == "bf16" else 0))
    batch, L, dim, N = 2, 1000, 64 * 7 - 8, 16
    x = I.random_scan_inputs(rng, batch, L, dim, N, dtype=dtype)
    h0 = _h0(rng, batch, dim, N)
    if plan == "whole":
        _check(x, dtype, h0=h0, label="h0 whole tiles")
    elif plan == "pairs":
        with Variant(2, 8, 3), Chained(False):
            _check(x, dtype, h0=h0, label="h0 chunk pairs")
    else:
        with Variant(2, 8, 3), Chained(True):
            _check(x, dtype, h0=h0, label="h0 chained")


def test_scan_continues_through_final_state():
    """Scanning a prefix, then the rest from its final state, gives the scan of the whole."""
    rng = np.random.default_rng(510)
    x = I.random_scan_inputs(rng, 2, 700, 136, 16, dtype="f32")
    cut = 333
    part = lambda a, s: None if a is None else np.ascontiguousarray(a[:, s])
    xa = {k: (part(v, slice(0, cut)) if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    xb = {k: (part(v, slice(cut, None)) if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    say("ex continuation")
    ya, fa = _gpu_ex(xa, "f32")
    yb, fb = _gpu_ex(xb, "f32", h0=fa)
    yo, fo = R.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"], delta_bias=x["delta_bias"])
    assert rel_err(np.concatenate([ya, yb], axis=1), yo) <= TOL["f32"] and rel_err(fb, fo) <= TOL["f32"]


@pytest.mark.parametrize("cu", [[0, 900], [0, 1, 2, 300, 300, 777, 900], [0, 450, 900]])
@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_sequences(cu, with_h0, dtype):
    rng = np.random.default_rng(520 + len(cu) + with_h0)
    x = I.random_scan_inputs(rng, 1, 900, 64 * 3 + 8, 16, dtype=dtype)
    h0 = _h0(rng, len(cu) - 1, 200, 16) if with_h0 else None
    _check(x, dtype, h0=h0, cu=cu, label=f"packed {len(cu) - 1} seqs h0={with_h0}")


def test_many_packed_sequences():
    """More (sequence, tile) units than CUs: the readout pass in 16-token blocks."""
    rng = np.random.default_rng(530)
    L = 3000
    cuts = np.sort(rng.choice(np.arange(1, L), size=299, replace=False))
    cu = [0] + [int(c) for c in cuts] + [L]
    x = I.random_scan_inputs(rng, 1, L, 64, 16, dtype="f32")
    _check(x, "f32", h0=_h0(rng, 300, 64, 16), cu=cu, label="300 packed seqs")


@pytest.mark.parametrize("N", [4, 32])
def test_packed_other_state_sizes(N):
    rng = np.random.default_rng(540 + N)
    x = I.random_scan_inputs(rng, 1, 500, 72, N, dtype="f32")
    _check(x, "f32", h0=_h0(rng, 3, 72, N), cu=[0, 100, 101, 500], label=f"packed N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_launch_order_changes_no_result(dtype):
    """Longest-first and index-order launches of the packed units give bit-identical outputs."""
    rng = np.random.default_rng(550)
    cu = [0, 5, 1500, 1500, 1510, 1800, 2000]
    x = I.random_scan_inputs(rng, 1, 2000, 200, 16, dtype=dtype)
    h0 = _h0(rng, len(cu) - 1, 200, 16)
    say(f"ex launch order {dtype}")
    y1, f1 = _gpu_ex(x, dtype, h0, cu)
    with IndexOrder():
        y0, f0 = _gpu_ex(x, dtype, h0, cu)
    assert np.array_equal(y0, y1) and np.array_equal(f0, f1)
    yo, fo = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                           delta_bias=x["delta_bias"], initial_state=h0, cu_seqlens=cu, nthreads=8)
    assert rel_err(y1, yo) <= TOL[dtype] and rel_err(f1, fo) <= TOL[dtype]
