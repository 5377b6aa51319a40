"""GPU parity of the trapezoidal rule's backward (ssm_scan_trap_bwd through the C ABI) against the fp64 oracles:
oracle/bwd.py with rule="trap" at the small shapes (pinned by central differences of the C oracle's trapezoidal
forward in test_oracle_bwd.py), and the C adjoint (ref.scan_bwd, rule="trap", pinned in test_oracle_bwd_c.py) on
the whole 2.8B-shaped layer.  Tolerances as for the two-term backward: 1e-4 for fp32 storage and the fp32 outputs, 2e-2
for the gradients stored in bf16."""
import numpy as np
import pytest
import torch

from oracle import bwd as OB
from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, oracle_threads, rel_err, say, to_dev, to_dev_f32
from .test_gpu_bwd import F32_OUT, SEQ_OUT, _case, _packed_case, _round

pytestmark = pytest.mark.gpu


def _run(x, dy, dfs, dtype, softplus=True, h0=None, cu=None, label=""):
    say(f"trap bwd {label} shape={x['u'].shape} N={x['A'].shape[1]} {dtype}")
    g = ops.ssm_scan_bwd(to_dev(x["u"], dtype), to_dev(x["delta"], dtype), to_dev_f32(x["A"]), to_dev(x["B"], dtype),
                         to_dev(x["C"], dtype), to_dev(dy, dtype), D=to_dev_f32(x["D"]),
                         z=to_dev(x["z"], dtype) if x["z"] is not None else None,
                         delta_bias=to_dev_f32(x["delta_bias"]), softplus=softplus, dfinal_state=to_dev_f32(dfs),
                         initial_state=to_dev_f32(h0), want_dinitial_state=True,
                         cu_seqlens=None if cu is None else torch.tensor(cu, device="cuda:0"), trapezoid=True,
                         check_status=True)
    torch.cuda.synchronize()
    o = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    softplus=softplus, dfinal_state=dfs,
                    initial_state=h0 if h0 is not None else np.zeros_like(g["dinitial_state"].cpu().numpy()),
                    cu_seqlens=cu, rule="trap")
    errs = {}
    for k in SEQ_OUT + F32_OUT:
        if o[k] is None:
            assert g[k] is None, k
            continue
        errs[k] = rel_err(g[k].float().cpu().numpy().astype(np.float64), o[k])
    print(f"[parity] trap bwd {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        tol = TOL[dtype] if k in SEQ_OUT else TOL["f32"]
        assert e <= tol, (k, e, tol)
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 4, 64])
def test_trap_bwd_matches_oracle(N, dtype):
    """Two rows from random initial states, a gradient on the final state, every optional input on; N = 16 (two
    states per lane), 32 and 4 (four), 64 (two launches of 32)."""
    rng = np.random.default_rng(900 + N + (1 if dtype == "bf16" else 0))
    x, dy, dfs = _case(rng, 2, 150, 136, N, dtype)
    h0 = np.asarray(rng.standard_normal((2, 136, N)) * 0.5, np.float32).astype(np.float64)
    _run(x, dy, dfs, dtype, h0=h0, label=f"N{N}")


@pytest.mark.parametrize("L", [1, 2, 17, 33])
def test_trap_bwd_short_and_ragged(L):
    """Shorter than a block, and ragged: the previous input of the first token is zero, the last token has no
    next step."""
    rng = np.random.default_rng(910 + L)
    x, dy, dfs = _case(rng, 2, L, 72, 16, "f32")
    _run(x, dy, dfs, "f32", label=f"L{L}")


@pytest.mark.parametrize("opts", [dict(gated=False), dict(with_D=False), dict(with_bias=False),
                                  dict(softplus=False), dict(with_dfs=False),
                                  dict(gated=False, with_D=False, with_bias=False, with_dfs=False)])
def test_trap_bwd_optional_inputs(opts):
    rng = np.random.default_rng(920 + len(opts))
    x, dy, dfs = _case(rng, 1, 70, 136, 16, "f32", **opts)
    _run(x, dy, dfs, "f32", softplus=opts.get("softplus", True), label=str(opts))


@pytest.mark.parametrize("dtype,N", [("f32", 16), ("bf16", 16), ("f32", 32), ("bf16", 64)])
def test_trap_bwd_packed_sequences(dtype, N):
    """Packed sequences (an empty one, a one-token one, lengths not multiples of the block), each from its own
    initial state: a sequence's first token takes no input from the sequence before it."""
    rng = np.random.default_rng(930 + N + (1 if dtype == "bf16" else 0))
    x, dy, dfs, h0, cu = _packed_case(rng, 300, 136, N, dtype, [0, 37, 37, 38, 150, 151, 300])
    _run(x, dy, dfs, dtype, h0=h0, cu=cu, label=f"packed N{N}")


def test_trap_bwd_extreme_steps():
    rng = np.random.default_rng(940)
    x, dy, dfs = _case(rng, 2, 200, 136, 16, "f32")
    x["delta"] = _round(np.asarray(x["delta"], np.float64) * 20.0, "f32")
    _run(x, dy, dfs, "f32", label="extreme steps")


def test_trap_bwd_deterministic():
    rng = np.random.default_rng(950)
    x, dy, dfs = _case(rng, 2, 300, 200, 16, "bf16")
    args = [to_dev(x[k], "bf16") for k in ("u", "delta")] + [to_dev_f32(x["A"])] + \
        [to_dev(x[k], "bf16") for k in ("B", "C")] + [to_dev(dy, "bf16")]
    kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "bf16"), delta_bias=to_dev_f32(x["delta_bias"]),
              dfinal_state=to_dev_f32(dfs), trapezoid=True)
    say("trap bwd determinism")
    g1 = ops.ssm_scan_bwd(*args, **kw)
    g2 = ops.ssm_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_trap_bwd_full_size_all_outputs():
    """The 2.8B-shaped layer (4 x 4096 x 5120 x 16 bf16, every optional input, a final-state gradient): every
    gradient of every (row, channel) -- du, d delta, dz; dB and dC summed over all 5120 channels; dA, dD and d bias
    summed over all 16384 (row, token) terms -- against the C oracle's trapezoidal adjoint (ref.scan_bwd with
    rule="trap") on the whole layer."""
    w = I.WORKLOADS["mamba2p8b_bf16"]
    x = I.make_inputs(w, 0)
    rng = np.random.default_rng(4545)
    dy = I.round_to_bf16(rng.standard_normal((w.batch, w.L, w.dim)))
    dfs = np.asarray(rng.standard_normal((w.batch, w.dim, w.dstate)), np.float32).astype(np.float64)
    say(f"trap bwd full size {w}")
    g = ops.ssm_scan_bwd(to_dev(x["u"], "bf16"), to_dev(x["delta"], "bf16"), to_dev_f32(x["A"]),
                         to_dev(x["B"], "bf16"), to_dev(x["C"], "bf16"), to_dev(dy, "bf16"), D=to_dev_f32(x["D"]),
                         z=to_dev(x["z"], "bf16"), delta_bias=to_dev_f32(x["delta_bias"]),
                         dfinal_state=to_dev_f32(dfs), trapezoid=True, check_status=True)
    torch.cuda.synchronize()
    got = {k: g[k].float().cpu().numpy().astype(np.float64) for k in SEQ_OUT + ("dA", "dD", "ddelta_bias")}
    del g
    torch.cuda.empty_cache()
    o = R.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                   dfinal_state=dfs, nthreads=oracle_threads(), rule="trap")
    errs = {}
    for k in got:
        errs[k] = rel_err(got[k], o[k])
        del o[k]
    print(f"[parity] trap bwd full size, all {w.batch * w.dim} (row, channel) pairs: " +
          "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in SEQ_OUT:
        assert errs[k] <= TOL["bf16"], (k, errs[k])
    for k in ("dA", "dD", "ddelta_bias"):
        assert errs[k] <= TOL["f32"], (k, errs[k])
