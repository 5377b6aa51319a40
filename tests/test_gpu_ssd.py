"""GPU parity of ssm_ssd_fwd (the Mamba-2 SSD layer on MFMA) against the oracle.

Compared element by element with oracle/ssd.py (the masked-matrix form,
pinned in test_oracle_ssd.py to the recurrent oracle) on the same seeded bf16
inputs.  Tolerance 2e-2 (bf16 storage), with the forward's error measure,
for y and the final state: the kernel multiplies bf16 operands (C B^T masked
and decayed, x, the state and the weighted B each rounded to bf16) with fp32
accumulation, which keeps the error near the bf16 rounding of y (~4e-3).
"""
import numpy as np
import pytest
import torch

from oracle import ssd as S
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, SsdChained, oracle_threads, rel_err, say

pytestmark = pytest.mark.gpu


def _dev(a, f32=False):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")
    return t if f32 else t.to(torch.bfloat16)


def _run(x, softplus=True, h0=None):
    y, fs = ops.ssm_ssd_fwd(_dev(x["x"]), _dev(x["delta"]), _dev(x["A"], True), _dev(x["B"]), _dev(x["C"]),
                            D=_dev(x["D"], True), z=_dev(x["z"]), delta_bias=_dev(x["delta_bias"], True),
                            softplus=softplus, initial_state=_dev(h0, True))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def _check(x, label, softplus=True, tol=TOL["bf16"], h0=None):
    say(f"ssd {label} x={x['x'].shape} B={x['B'].shape}")
    yg, fg = _run(x, softplus, h0)
    yo, fo = S.ssd_fwd(x["x"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                       softplus=softplus, initial_state=h0)
    ey, ef = rel_err(yg, yo), rel_err(fg, fo)
    print(f"[parity] ssd {label}: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= tol and ef <= tol, (ey, ef)


@pytest.mark.parametrize("N", [32, 64, 128])
@pytest.mark.parametrize("L", [64, 300, 1000])
def test_ssd_matches_oracle(N, L):
    x = I.random_ssd_inputs(np.random.default_rng(700 + N + L), 2, L, 3, 64, N)
    _check(x, f"L={L} N={N}")


@pytest.mark.parametrize("L", [1, 17, 63, 65, 129])
def test_ssd_short_and_ragged(L):
    x = I.random_ssd_inputs(np.random.default_rng(720 + L), 3, L, 2, 64, 64)
    _check(x, f"L={L}")


@pytest.mark.parametrize("opts", ["no_gate", "no_skip", "no_bias", "no_softplus"])
def test_ssd_optional_inputs(opts):
    rng = np.random.default_rng(730 + len(opts))
    x = I.random_ssd_inputs(rng, 2, 200, 2, 64, 64, gate=opts != "no_gate")
    softplus = True
    if opts == "no_skip":
        x["D"] = None
    elif opts == "no_bias":
        x["delta_bias"] = None
    elif opts == "no_softplus":
        softplus = False
        x["delta"] = I.round_to_bf16(np.abs(x["delta"]) * 0.1 + 0.01)  # the step itself: keep it positive
        x["delta_bias"] = np.abs(x["delta_bias"]) * 0.01
    _check(x, opts, softplus=softplus)


def test_ssd_slow_decay_long_memory():
    """A near zero: states carry across many chunks (the inter-chunk path dominates)."""
    rng = np.random.default_rng(740)
    x = I.random_ssd_inputs(rng, 1, 700, 2, 64, 64)
    x["A"] = -rng.uniform(0.001, 0.01, 2).astype(np.float32)
    _check(x, "slow decay")


def test_ssd_many_heads_and_batch_rows():
    x = I.random_ssd_inputs(np.random.default_rng(750), 3, 130, 11, 64, 32)
    _check(x, "batch 3, 11 heads")


def test_ssd_full_size_sampled_heads():
    """The 2.7B-shaped layer (batch 4, L 4096, 80 heads of 64, state 128) as bench.py times it; the masked-matrix
    oracle on 6 sampled (batch row, head) pairs."""
    cfg = I.SSD_WORKLOADS["mamba2_2p7b_bf16"]
    x = I.random_ssd_inputs(np.random.default_rng(0), cfg["batch"], cfg["L"], cfg["heads"], cfg["headdim"],
                            cfg["dstate"])
    say("ssd full-size 2.7B layer")
    yg, fg = _run(x)
    assert np.all(np.isfinite(yg))
    ey = ef = 0.0
    for b, h in [(0, 0), (0, 79), (1, 17), (2, 40), (3, 63), (3, 79)]:
        sub = dict(x=x["x"][b:b + 1, :, h:h + 1], z=x["z"][b:b + 1, :, h:h + 1], delta=x["delta"][b:b + 1, :, h:h + 1],
                   B=x["B"][b:b + 1], C=x["C"][b:b + 1], A=x["A"][h:h + 1], D=x["D"][h:h + 1],
                   delta_bias=x["delta_bias"][h:h + 1])
        yo, fo = S.ssd_fwd(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], D=sub["D"], z=sub["z"],
                           delta_bias=sub["delta_bias"])
        ey = max(ey, rel_err(yg[b:b + 1, :, h:h + 1], yo))
        ef = max(ef, rel_err(fg[b:b + 1, h:h + 1], fo))
    print(f"[parity] ssd 2.7B sampled heads: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_ssd_full_size_all_heads_against_the_recurrence():
    """The whole 2.7B-shaped layer against the recurrent C oracle: with one group the layer is the two-term scan
    over heads x headdim channels with A[d][n] = A[head of d] and the head's step on each of its channels (the
    duality tests/test_oracle_ssd.py pins).  Every output of every (row, head) is compared."""
    from oracle import ref as R

    cfg = I.SSD_WORKLOADS["mamba2_2p7b_bf16"]
    bt, L, H, P, N = cfg["batch"], cfg["L"], cfg["heads"], cfg["headdim"], cfg["dstate"]
    x = I.random_ssd_inputs(np.random.default_rng(0), bt, L, H, P, N)
    say("ssd full-size 2.7B layer, all heads")
    yg, fg = _run(x)
    rep = lambda a: np.repeat(np.asarray(a, np.float32), P, axis=-1)  # per head -> per channel (head major)
    yo, fo = R.scan_fwd(x["x"].reshape(bt, L, H * P), rep(x["delta"]),
                        np.repeat(x["A"], P)[:, None] * np.ones((1, N), np.float32), x["B"], x["C"],
                        D=rep(x["D"]), z=x["z"].reshape(bt, L, H * P), delta_bias=rep(x["delta_bias"]),
                        nthreads=oracle_threads())
    ey = rel_err(yg.reshape(bt, L, H * P), yo)
    ef = rel_err(fg.reshape(bt, H * P, N), fo)
    print(f"[parity] ssd 2.7B all {bt * H} (row, head) units: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_ssd_deterministic():
    x = I.random_ssd_inputs(np.random.default_rng(760), 2, 300, 4, 64, 128)
    say("ssd determinism")
    y1, f1 = _run(x)
    y2, f2 = _run(x)
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("L", [700, 130])
def test_ssd_chained_plan(L):
    """270 units (3 rows x 90 heads): 256 whole, 14 cut into 8 segments chained through the workspace (L = 130
    leaves most segments empty).  Equal to the oracle, and bitwise equal to one workgroup per unit (the state is
    handed on exactly)."""
    x = I.random_ssd_inputs(np.random.default_rng(770 + L), 3, L, 90, 64, 64)
    with SsdChained(True):
        _check(x, f"chained L={L}")
        yc, fc = _run(x)
    with SsdChained(False):
        yu, fu = _run(x)
    assert np.array_equal(yc, yu) and np.array_equal(fc, fu)


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_then_decode_step_continues_it(N):
    """An SSD layer is a selective scan whose channels share their head's step and A ([P4] "Mamba-2 and
    Structured State Space Duality"), so its one-token continuation is ssm_state_update with the step and A
    broadcast over the head's channels: the SSD over L-1 tokens, then one decode step from its final state,
    equals the SSD over L tokens (y of the last token and the final state).  Two independent kernels (the
    MFMA chunked form and the per-channel decode) must agree."""
    rng = np.random.default_rng(790 + N)
    batch, L, H, P = 2, 130, 3, 64
    x = I.random_ssd_inputs(rng, batch, L, H, P, N)
    say("ssd then decode")
    y_full, f_full = _run(x)
    head = {k: (v[:, :L - 1] if k in ("x", "delta", "B", "C", "z") else v) for k, v in x.items()}
    _, f_head = _run(head)
    t = L - 1
    rep = lambda a: np.repeat(np.asarray(a, np.float32), P, axis=-1)  # per head -> per channel (h major, p minor)
    state = torch.from_numpy(np.ascontiguousarray(f_head.reshape(batch, H * P, N), dtype=np.float32)).to("cuda:0")
    yd = ops.ssm_state_update(state, _dev(x["x"][:, t].reshape(batch, H * P)), _dev(rep(x["delta"][:, t])),
                              _dev(np.repeat(x["A"], P)[:, None] * np.ones((1, N), np.float32), True),
                              _dev(x["B"][:, t]), _dev(x["C"][:, t]), D=_dev(rep(x["D"]), True),
                              z=_dev(x["z"][:, t].reshape(batch, H * P)), delta_bias=_dev(rep(x["delta_bias"]), True))
    torch.cuda.synchronize()
    ey = rel_err(yd.float().cpu().numpy().astype(np.float64), y_full[:, t].reshape(batch, H * P))
    ef = rel_err(state.cpu().numpy().astype(np.float64), f_full.reshape(batch, H * P, N))
    print(f"[parity] ssd then decode: y {ey:.2e}  state {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= 1e-4, (ey, ef)


@pytest.mark.parametrize("batch,heads", [(1, 257), (4, 96)])
def test_ssd_planner_boundaries(batch, heads):
    """The SSD's chained plan at its edges, as the planner chooses it: one (row, head) unit left over (cut into
    the most segments) and half as many units again as CUs (two segments each); ragged L."""
    x = I.random_ssd_inputs(np.random.default_rng(800 + heads), batch, 200, heads, 64, 32)
    _check(x, f"planner boundary {batch * heads} units")


def test_ssd_extreme_steps():
    """Raw steps spread over +-60: within a chunk the cumulative decay underflows to 0 (the masked matrix and
    the chunk's weights lose every term but the newest) or stays at 1."""
    x = I.random_ssd_inputs(np.random.default_rng(810), 2, 300, 4, 64, 64)
    x["delta"] = I.round_to_bf16(np.asarray(x["delta"], np.float64) * 20.0)
    _check(x, "extreme steps")


@pytest.mark.parametrize("chained", [False, True])
def test_ssd_initial_state(chained):
    """From a given state per (row, head): on one workgroup per unit, and on the chained plan (270 units), where
    a unit's first segment starts from it."""
    rng = np.random.default_rng(820 + chained)
    batch, heads = (2, 5) if not chained else (3, 90)
    x = I.random_ssd_inputs(rng, batch, 200, heads, 64, 64)
    h0 = np.asarray(rng.standard_normal((batch, heads, 64, 64)) * 0.5, np.float32).astype(np.float64)
    with SsdChained(chained):
        _check(x, f"initial state chained={chained}", h0=h0)


def test_ssd_continues_from_its_final_state():
    """Two calls, the second from the first's final state, equal one call over all the tokens (chunked prefill;
    [P1] "The relay")."""
    rng = np.random.default_rng(830)
    x = I.random_ssd_inputs(rng, 2, 300, 3, 64, 128)
    say("ssd continuation")
    y_all, f_all = _run(x)
    cut = 137
    first = {k: (v[:, :cut] if k in ("x", "delta", "B", "C", "z") else v) for k, v in x.items()}
    second = {k: (v[:, cut:] if k in ("x", "delta", "B", "C", "z") else v) for k, v in x.items()}
    y1, f1 = _run(first)
    y2, f2 = _run(second, h0=f1)
    ey = rel_err(np.concatenate([y1, y2], axis=1), y_all)
    ef = rel_err(f2, f_all)
    print(f"[parity] ssd continuation: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= 1e-4, (ey, ef)


@pytest.mark.parametrize("ngroups,heads,N", [(2, 4, 64), (4, 8, 32), (3, 6, 128), (8, 8, 64)])
def test_ssd_groups_match_oracle(ngroups, heads, N):
    """B, C of shape [batch, L, ngroups, dstate]: runs of heads / ngroups heads share a group (the oracle pinned per
    group to the recurrent scan); ragged L, from a given state."""
    rng = np.random.default_rng(790 + ngroups * 10 + heads)
    x = I.random_ssd_inputs(rng, 2, 333, heads, 64, N, ngroups=ngroups)
    h0 = (rng.standard_normal((2, heads, 64, N)) * 0.5).astype(np.float32)
    _check(x, f"{ngroups} groups of {heads // ngroups} heads N={N}", h0=h0)


def test_ssd_groups_chained_plan(monkeypatch):
    """Groups on the chained plan: 10 (row, head) units on a plan for 8 CUs (8 whole, 2 cut into 4 segments)."""
    monkeypatch.setenv("SSM_NUM_CU", "8")
    x = I.random_ssd_inputs(np.random.default_rng(799), 1, 700, 10, 64, 64, ngroups=5)
    _check(x, "5 groups, chained for 8 CUs")
