"""GPU parity of ssm_scan_trap_fwd (the Mamba-3 trapezoidal three-term scan) against the oracle.

Compared element by element with oracle ref.scan_trap_fwd_ex (pinned in
test_oracle_trap.py) on the same seeded inputs, with the forward's error
measure and tolerances (1e-4 fp32, 2e-2 bf16 storage).  The kernel scans a
shifted state and adds the left-out part in the epilogue, and hands on h at
every chunk boundary, so the cases cover every plan that cuts a sequence
(chunk pairs, chained chunks, packed sequences) as well as whole tiles.
"""
import numpy as np
import pytest
import torch

from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, BlockLen, Chained, Variant, oracle_threads, rel_err, say, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu


def _gpu(x, dtype, softplus=True, h0=None, cu=None):
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int64, device="cuda:0")
    y, fs = ops.ssm_scan_trap_fwd(to_dev(x["u"], dtype), to_dev(x["delta"], dtype), to_dev_f32(x["A"]),
                                  to_dev(x["B"], dtype), to_dev(x["C"], dtype), D=to_dev_f32(x["D"]),
                                  z=to_dev(x["z"], dtype), delta_bias=to_dev_f32(x["delta_bias"]),
                                  softplus=softplus, initial_state=to_dev_f32(h0), cu_seqlens=cu_t)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def _oracle(x, softplus=True, h0=None, cu=None):
    return R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                              delta_bias=x["delta_bias"], softplus=softplus, initial_state=h0, cu_seqlens=cu,
                              nthreads=8)


def _check(x, dtype, label, softplus=True, h0=None, cu=None):
    say(f"trap {label} shape={x['u'].shape} N={x['A'].shape[1]} {dtype}")
    yg, fg = _gpu(x, dtype, softplus, h0, cu)
    yo, fo = _oracle(x, softplus, h0, cu)
    ey, ef = rel_err(yg, yo), rel_err(fg, fo)
    print(f"[parity] trap {label}: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL[dtype] and ef <= TOL[dtype], (ey, ef)
    return yg, fg


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("plan", ["whole", "pairs", "chained"])
def test_every_plan(plan, dtype):
    rng = np.random.default_rng(600 + len(plan) + (3 if dtype == "bf16" else 0))
    x = I.random_scan_inputs(rng, 2, 1000, 64 * 7 - 8, 16, dtype=dtype)
    if plan == "whole":
        _check(x, dtype, "whole tiles")
    elif plan == "pairs":
        with Variant(2, 8, 3), Chained(False):
            _check(x, dtype, "chunk pairs K=3")
    else:
        with Variant(2, 8, 3), Chained(True):
            _check(x, dtype, "chained K=3")


@pytest.mark.parametrize("npl,G", [(2, 8), (1, 16), (4, 4), (8, 2), (16, 1)])
@pytest.mark.parametrize("K", [1, 5])
def test_every_variant(npl, G, K):
    rng = np.random.default_rng(610 + npl * 10 + G + K)
    x = I.random_scan_inputs(rng, 2, 777, 136, 16, dtype="f32")
    with Variant(npl, G, K):
        _check(x, "f32", f"variant ({npl},{G}) K={K}")


@pytest.mark.parametrize("dtype,N", [("f32", 1), ("f32", 3), ("bf16", 4), ("f32", 7), ("bf16", 32), ("f32", 64)])
def test_other_state_sizes(dtype, N):
    rng = np.random.default_rng(620 + N)
    x = I.random_scan_inputs(rng, 2, 300, 72, N, dtype=dtype)
    _check(x, dtype, f"N={N}")


@pytest.mark.parametrize("L", [1, 2, 17, 129])
def test_short_and_ragged_sequences(L):
    rng = np.random.default_rng(630 + L)
    x = I.random_scan_inputs(rng, 3, L, 70, 16, dtype="f32")
    _check(x, "f32", f"L={L}")


@pytest.mark.parametrize("opts", ["no_gate", "no_skip", "no_bias", "no_softplus"])
def test_optional_inputs(opts):
    rng = np.random.default_rng(640 + len(opts))
    x = I.random_scan_inputs(rng, 2, 200, 100, 16, dtype="f32")
    softplus = True
    if opts == "no_gate":
        x["z"] = None
    elif opts == "no_skip":
        x["D"] = None
    elif opts == "no_bias":
        x["delta_bias"] = None
    else:
        softplus = False
        # delta_raw + bias is the step itself: keep it positive (a negative step grows without bound)
        x["delta"] = np.abs(x["delta"]) * 0.1 + 0.01
        x["delta_bias"] = np.abs(x["delta_bias"]) * 0.01
    _check(x, "f32", opts, softplus=softplus)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cu", [[0, 900], [0, 1, 2, 300, 300, 777, 900]])
def test_packed_sequences_with_initial_states(cu, dtype):
    rng = np.random.default_rng(650 + len(cu))
    x = I.random_scan_inputs(rng, 1, 900, 200, 16, dtype=dtype)
    h0 = np.asarray(rng.standard_normal((len(cu) - 1, 200, 16)) * 0.5, np.float32).astype(np.float64)
    _check(x, dtype, f"packed {len(cu) - 1} seqs", h0=h0, cu=cu)


@pytest.mark.parametrize("plan", ["whole", "pairs"])
def test_initial_state(plan):
    rng = np.random.default_rng(660 + len(plan))
    x = I.random_scan_inputs(rng, 2, 500, 130, 16, dtype="bf16")
    h0 = np.asarray(rng.standard_normal((2, 130, 16)) * 0.5, np.float32).astype(np.float64)
    if plan == "whole":
        _check(x, "bf16", "h0 whole", h0=h0)
    else:
        with Variant(2, 8, 4), Chained(False):
            _check(x, "bf16", "h0 pairs K=4", h0=h0)


def test_block_lengths_agree_bitwise():
    rng = np.random.default_rng(670)
    x = I.random_scan_inputs(rng, 2, 700, 128, 16, dtype="bf16")
    say("trap 16- vs 32-token blocks")
    with BlockLen(16):
        y16, f16 = _gpu(x, "bf16")
    with BlockLen(32):
        y32, f32 = _gpu(x, "bf16")
    assert np.array_equal(y16, y32) and np.array_equal(f16, f32)


def test_full_size_2p8b_layer_all_channels():
    """The 2.8B-shaped layer (batch 4, L 4096, dim 5120, bf16) in its default (chained) plan, every output
    against the oracle."""
    w = I.WORKLOADS["mamba2p8b_bf16"]
    x = I.make_inputs(w, 0)
    say(f"trap full-size {w}")
    yg, fg = _gpu(x, w.dtype)
    yo, fo = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                delta_bias=x["delta_bias"], nthreads=oracle_threads())
    ey, ef = rel_err(yg, yo), rel_err(fg, fo)
    print(f"[parity] trap 2.8B all {w.batch * w.dim} channels: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_deterministic():
    rng = np.random.default_rng(680)
    x = I.random_scan_inputs(rng, 2, 600, 200, 16, dtype="f32")
    say("trap determinism")
    with Variant(2, 8, 3), Chained(True):
        y1, f1 = _gpu(x, "f32")
        y2, f2 = _gpu(x, "f32")
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)
