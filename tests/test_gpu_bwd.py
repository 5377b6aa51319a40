"""GPU parity of the backward pass (ssm_scan_bwd through the C ABI) against the fp64 oracle.

Every gradient is compared element by element with the fp64 oracle on the same
(rounded) inputs: oracle/bwd.py (automatic differentiation) at the small shapes,
the C adjoint recurrence (oracle ref.scan_bwd) on the whole 2.8B-shaped layer;
the error measure is gpu_util.rel_err.  Tolerances:
1e-4 for fp32 storage and for the fp32 outputs (dA, dD, d bias); 2e-2 for the
outputs stored in bf16 (du, d delta, dz, dB, dC), whose rounding alone is up
to 2^-9.
"""
import numpy as np
import pytest
import torch

from oracle import bwd as OB
from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, BwdChained, oracle_threads, rel_err, say, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu

SEQ_OUT = ("du", "ddelta", "dz", "dB", "dC")   # stored in the storage dtype
F32_OUT = ("dA", "dD", "ddelta_bias", "dinitial_state")  # always fp32


def _round(x, dtype):
    return None if x is None else (I.round_to_bf16(x) if dtype == "bf16" else np.asarray(x, np.float32).astype(np.float64))


def _case(rng, batch, L, dim, N, dtype, gated=True, with_D=True, with_bias=True, softplus=True, with_dfs=True):
    x = I.random_scan_inputs(rng, batch, L, dim, N, dtype=dtype)
    if not gated:
        x["z"] = None
    if not with_D:
        x["D"] = None
    if not with_bias:
        x["delta_bias"] = None
    if not softplus:
        # delta + bias is the step itself: keep it positive (a negative step grows the state without bound)
        x["delta"] = _round(np.abs(x["delta"]) + 0.05, dtype)
        if x["delta_bias"] is not None:
            x["delta_bias"] = np.abs(x["delta_bias"]) * 0.01
    dy = _round(rng.standard_normal((batch, L, dim)), dtype)
    dfs = np.asarray(rng.standard_normal((batch, dim, N)), np.float32).astype(np.float64) if with_dfs else None
    return x, dy, dfs


def _run_and_compare(x, dy, dfs, dtype, softplus=True, label="", h0=None):
    say(f"bwd {label} shape={x['u'].shape} N={x['A'].shape[1]} {dtype}")
    g = ops.ssm_scan_bwd(to_dev(x["u"], dtype), to_dev(x["delta"], dtype), to_dev_f32(x["A"]), to_dev(x["B"], dtype),
                         to_dev(x["C"], dtype), to_dev(dy, dtype), D=to_dev_f32(x["D"]),
                         z=to_dev(x["z"], dtype) if x["z"] is not None else None,
                         delta_bias=to_dev_f32(x["delta_bias"]), softplus=softplus,
                         dfinal_state=to_dev_f32(dfs), initial_state=to_dev_f32(h0))
    torch.cuda.synchronize()
    o = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    softplus=softplus, dfinal_state=dfs, initial_state=h0)
    errs = {}
    for k in SEQ_OUT + F32_OUT:
        if o[k] is None:
            assert g[k] is None, k
            continue
        gk = g[k].float().cpu().numpy().astype(np.float64)
        errs[k] = rel_err(gk, o[k])
    print(f"[parity] bwd {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        tol = TOL[dtype] if k in SEQ_OUT else TOL["f32"]
        assert e <= tol, (k, e, tol)
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 4, 1, 33, 48, 64])
def test_bwd_matches_oracle(N, dtype):
    rng = np.random.default_rng(100 + N + (7 if dtype == "bf16" else 0))
    x, dy, dfs = _case(rng, 2, 150, 64 * 2 + 8, N, dtype)
    _run_and_compare(x, dy, dfs, dtype, label=f"N{N}")


@pytest.mark.parametrize("L", [1, 7, 16, 33])
def test_bwd_short_and_ragged_sequences(L):
    rng = np.random.default_rng(200 + L)
    x, dy, dfs = _case(rng, 3, L, 70, 16, "f32")
    _run_and_compare(x, dy, dfs, "f32", label=f"L{L}")


@pytest.mark.parametrize("opts", [
    dict(gated=False), dict(with_D=False), dict(with_bias=False), dict(softplus=False), dict(with_dfs=False),
    dict(gated=False, with_D=False, with_bias=False, softplus=False, with_dfs=False),
])
def test_bwd_optional_inputs(opts):
    rng = np.random.default_rng(300 + len(opts))
    x, dy, dfs = _case(rng, 2, 90, 64 + 12, 16, "f32", **opts)
    _run_and_compare(x, dy, dfs, "f32", softplus=opts.get("softplus", True), label=str(opts))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_bwd_with_initial_state(N, dtype):
    """From an initial state h0: every gradient, and d h0 (the adjoint reaching h_{-1})."""
    rng = np.random.default_rng(450 + N + (5 if dtype == "bf16" else 0))
    x, dy, dfs = _case(rng, 2, 120, 64 + 40, N, dtype)
    h0 = np.asarray(rng.standard_normal((2, 64 + 40, N)) * 0.5, np.float32).astype(np.float64)
    _run_and_compare(x, dy, dfs, dtype, label=f"h0 N{N}", h0=h0)


def test_bwd_is_deterministic():
    rng = np.random.default_rng(400)
    x, dy, dfs = _case(rng, 2, 200, 64 * 3, 16, "f32")
    args = (to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]), to_dev(x["B"], "f32"),
            to_dev(x["C"], "f32"), to_dev(dy, "f32"))
    kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "f32"), delta_bias=to_dev_f32(x["delta_bias"]),
              dfinal_state=to_dev_f32(dfs))
    say("bwd determinism")
    g1 = ops.ssm_scan_bwd(*args, **kw)
    g2 = ops.ssm_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("L", [300, 40, 16])
def test_bwd_chained_plan(L):
    """320 tiles (5 rows x 64 tiles): 256 whole, 64 cut into 4 chunks of blocks handing the adjoint backwards
    (L = 40 leaves the last chunk empty, L = 16 all but chunk 0)."""
    rng = np.random.default_rng(470 + L)
    x, dy, dfs = _case(rng, 5, L, 64 * 64, 16, "bf16")
    h0 = np.asarray(rng.standard_normal((5, 64 * 64, 16)) * 0.5, np.float32).astype(np.float64)
    with BwdChained(True):
        _run_and_compare(x, dy, dfs, "bf16", label=f"chained L{L}", h0=h0)


def test_bwd_chained_plan_fp32_and_deterministic():
    rng = np.random.default_rng(480)
    x, dy, dfs = _case(rng, 5, 200, 64 * 64, 16, "f32")
    with BwdChained(True):
        g1 = _run_and_compare(x, dy, dfs, "f32", label="chained fp32")
        args = (to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]), to_dev(x["B"], "f32"),
                to_dev(x["C"], "f32"), to_dev(dy, "f32"))
        kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "f32"), delta_bias=to_dev_f32(x["delta_bias"]),
                  dfinal_state=to_dev_f32(dfs))
        g2 = ops.ssm_scan_bwd(*args, **kw)
        g3 = ops.ssm_scan_bwd(*args, **kw)
        torch.cuda.synchronize()
    for k in g2:
        if g2[k] is not None:
            assert torch.equal(g2[k], g3[k]), k


@pytest.mark.parametrize("tiles", [257, 384])
def test_bwd_planner_boundaries(tiles):
    """The backward's chained plan at its edges, as the planner chooses it: one tile left over (cut into the most
    chunks), and half as many tiles again as CUs (two chunks each); ragged L."""
    rng = np.random.default_rng(490 + tiles)
    x, dy, dfs = _case(rng, 1, 150, 64 * tiles, 16, "bf16")
    _run_and_compare(x, dy, dfs, "bf16", label=f"planner boundary {tiles} tiles")


def test_bwd_extreme_steps():
    """Steps from ~1e-26 to ~60 (raw values spread over +-60): decays that underflow to 0 and decays of 1, with
    softplus' saturating at 0 and 1, in every gradient."""
    rng = np.random.default_rng(495)
    x, dy, dfs = _case(rng, 2, 200, 136, 16, "f32")
    x["delta"] = _round(np.asarray(x["delta"], np.float64) * 20.0, "f32")
    _run_and_compare(x, dy, dfs, "f32", label="extreme steps")


def test_bwd_full_size_all_outputs():
    """The backward at the shape the benchmark times (4 x 4096 x 5120 x 16 bf16, z, D, bias, softplus on, the
    chained plan: 256 whole tiles and 64 cut into 4 chunks of blocks, the checkpoint pass chained alike), with a
    gradient on the final state: every gradient of every (row, channel) -- du, d delta, dz; dB and dC, each a
    sum over all 5120 channels; dA, dD and d bias, each a sum over all 16384 (row, token) terms -- against the
    C oracle's adjoint recurrence (ref.scan_bwd) on the whole layer."""
    w = I.WORKLOADS["mamba2p8b_bf16"]
    x = I.make_inputs(w, 0)
    rng = np.random.default_rng(4242)
    dy = I.round_to_bf16(rng.standard_normal((w.batch, w.L, w.dim)))
    dfs = np.asarray(rng.standard_normal((w.batch, w.dim, w.dstate)), np.float32).astype(np.float64)
    say(f"bwd full size {w}")
    g = ops.ssm_scan_bwd(to_dev(x["u"], "bf16"), to_dev(x["delta"], "bf16"), to_dev_f32(x["A"]),
                         to_dev(x["B"], "bf16"), to_dev(x["C"], "bf16"), to_dev(dy, "bf16"), D=to_dev_f32(x["D"]),
                         z=to_dev(x["z"], "bf16"), delta_bias=to_dev_f32(x["delta_bias"]),
                         dfinal_state=to_dev_f32(dfs), check_status=True)
    torch.cuda.synchronize()
    got = {k: g[k].float().cpu().numpy().astype(np.float64) for k in SEQ_OUT + ("dA", "dD", "ddelta_bias")}
    del g
    torch.cuda.empty_cache()
    o = R.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                   dfinal_state=dfs, nthreads=oracle_threads())
    errs = {}
    for k in got:
        errs[k] = rel_err(got[k], o[k])
        del o[k]
    print(f"[parity] bwd full size, all {w.batch * w.dim} (row, channel) pairs: " +
          "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in SEQ_OUT:
        assert errs[k] <= TOL["bf16"], (k, errs[k])
    for k in ("dA", "dD", "ddelta_bias"):
        assert errs[k] <= TOL["f32"], (k, errs[k])


def test_bwd_db_dc_full_length_chained(monkeypatch):
    """dB and dC (sums over every channel of a row) at the full 4096 tokens, in the chained plan the benchmark
    runs, on a layer the oracle can finish: 5 tiles (320 channels) planned for a 4-CU device, so 4 whole tiles and
    1 cut into 4 chunks of blocks (and the checkpoint pass into 4 chunks of 1024 tokens).  Every gradient against
    the oracle."""
    monkeypatch.setenv("SSM_NUM_CU", "4")
    rng = np.random.default_rng(4343)
    x, dy, dfs = _case(rng, 1, 4096, 320, 16, "bf16")
    x["A"] = np.tile(-np.arange(1, 17, dtype=np.float64), (320, 1))   # the benchmark's A[d, n] = -(n + 1)
    _run_and_compare(x, dy, dfs, "bf16", label="1 x 4096 x 320 chained for 4 CUs")


def _packed_case(rng, L, dim, N, dtype, cuts):
    x = I.random_scan_inputs(rng, 1, L, dim, N, dtype=dtype)
    nseq = len(cuts) - 1
    dy = _round(rng.standard_normal((1, L, dim)), dtype)
    dfs = np.asarray(rng.standard_normal((nseq, dim, N)), np.float32).astype(np.float64)
    h0 = np.asarray(rng.standard_normal((nseq, dim, N)) * 0.5, np.float32).astype(np.float64)
    return x, dy, dfs, h0, np.asarray(cuts, dtype=np.int64)


def _run_packed(x, dy, dfs, h0, cu, dtype, label):
    say(f"bwd packed {label} L={x['u'].shape[1]} dim={x['u'].shape[2]} nseq={len(cu) - 1} {dtype}")
    g = ops.ssm_scan_bwd(to_dev(x["u"], dtype), to_dev(x["delta"], dtype), to_dev_f32(x["A"]), to_dev(x["B"], dtype),
                         to_dev(x["C"], dtype), to_dev(dy, dtype), D=to_dev_f32(x["D"]), z=to_dev(x["z"], dtype),
                         delta_bias=to_dev_f32(x["delta_bias"]), dfinal_state=to_dev_f32(dfs),
                         initial_state=to_dev_f32(h0), cu_seqlens=torch.tensor(cu, device="cuda:0"),
                         check_status=True)
    torch.cuda.synchronize()
    o = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    dfinal_state=dfs, initial_state=h0, cu_seqlens=cu)
    errs = {k: rel_err(g[k].float().cpu().numpy().astype(np.float64), o[k]) for k in SEQ_OUT + F32_OUT}
    print(f"[parity] bwd packed {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        tol = TOL[dtype] if k in SEQ_OUT else TOL["f32"]
        assert e <= tol, (k, e, tol)
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_bwd_packed_sequences(N, dtype):
    """Packed sequences of one row (an empty one, a one-token one, lengths not multiples of the 16-token block),
    each from its own initial state with its own final-state gradient; every gradient and d initial_state per
    sequence against the oracle over packed sequences (pinned by central differences)."""
    cuts = [0, 37, 37, 38, 150, 151, 300]
    rng = np.random.default_rng(860 + N + (1 if dtype == "bf16" else 0))
    x, dy, dfs, h0, cu = _packed_case(rng, 300, 136, N, dtype, cuts)
    _run_packed(x, dy, dfs, h0, cu, dtype, f"N{N}")


def test_bwd_packed_many_sequences_and_deterministic():
    """40 sequences x 3 tile columns (120 units, longest first): every gradient; two runs bitwise equal."""
    rng = np.random.default_rng(870)
    lens = rng.integers(1, 60, size=40)
    cuts = np.concatenate([[0], np.cumsum(lens)]).tolist()
    x, dy, dfs, h0, cu = _packed_case(rng, cuts[-1], 136, 16, "f32", cuts)
    g1 = _run_packed(x, dy, dfs, h0, cu, "f32", "40 sequences")
    g2 = _run_packed(x, dy, dfs, h0, cu, "f32", "40 sequences again")
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_bwd_packed_one_sequence_equals_unpacked():
    """One packed sequence over the whole row is the plain backward from that initial state (bitwise)."""
    rng = np.random.default_rng(880)
    x, dy, dfs, h0, cu = _packed_case(rng, 200, 72, 16, "f32", [0, 200])
    args = (to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]), to_dev(x["B"], "f32"),
            to_dev(x["C"], "f32"), to_dev(dy, "f32"))
    kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "f32"), delta_bias=to_dev_f32(x["delta_bias"]),
              dfinal_state=to_dev_f32(dfs), initial_state=to_dev_f32(h0))
    say("bwd one packed sequence vs unpacked")
    g1 = ops.ssm_scan_bwd(*args, cu_seqlens=torch.tensor(cu, device="cuda:0"), **kw)
    g2 = ops.ssm_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
