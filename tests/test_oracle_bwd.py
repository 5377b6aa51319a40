"""Pins of the fp64 backward oracle (oracle/bwd.py), all on the CPU.

The backward oracle is automatic differentiation of its own transcription of
the forward recurrence.  It is pinned against things outside itself:
  - that transcription's forward equals the C oracle's forward (pinned in
    test_oracle_pins.py against the pages and closed forms);
  - central finite differences of the C oracle's forward, for every input,
    with and without the optional inputs, and through the final state;
  - gradients of the pages' two-token relay example ([P1] "The relay"),
    derived by hand.
"""
import numpy as np
import pytest

from oracle import bwd as OB
from oracle import ref as R


def _inputs(rng, batch, L, dim, N, gated=True):
    x = dict(
        u=rng.standard_normal((batch, L, dim)),
        delta=rng.standard_normal((batch, L, dim)) * 0.5 - 1.0,
        A=-np.exp(rng.standard_normal((dim, N)) * 0.5),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(dim),
        z=rng.standard_normal((batch, L, dim)) if gated else None,
        delta_bias=rng.standard_normal(dim) * 0.3,
    )
    return x


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("softplus,gated", [(True, True), (False, False), (True, False)])
def test_transcription_forward_equals_c_oracle(softplus, gated):
    rng = np.random.default_rng(7)
    x = _inputs(rng, 2, 9, 5, 3, gated=gated)
    import torch
    t = {k: (None if v is None else torch.tensor(v)) for k, v in x.items()}
    y, fs = OB.forward_torch(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["delta_bias"], softplus=softplus)
    yo, fo = R.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                        delta_bias=x["delta_bias"], softplus=softplus)
    assert _rel(y.numpy(), yo) < 1e-13 and _rel(fs.numpy(), fo) < 1e-13


def _objective(x, dy, dfs, softplus):
    y, fs = R.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                       delta_bias=x["delta_bias"], softplus=softplus)
    val = float(np.sum(y * dy))
    if dfs is not None:
        val += float(np.sum(fs * dfs))
    return val


@pytest.mark.parametrize("softplus,gated,with_fs", [(True, True, False), (True, True, True), (False, False, True)])
def test_gradients_match_central_differences_of_c_oracle(softplus, gated, with_fs):
    rng = np.random.default_rng(11 + 2 * softplus + gated)
    batch, L, dim, N = 2, 7, 3, 4
    x = _inputs(rng, batch, L, dim, N, gated=gated)
    if not gated:
        x["D"] = None
        x["delta_bias"] = None
    if not softplus:
        # without softplus delta is used as the step as given: keep it a positive step size
        x["delta"] = np.abs(x["delta"]) + 0.05
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N)) if with_fs else None
    g = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                    delta_bias=x["delta_bias"], softplus=softplus, dfinal_state=dfs)
    checked = 0
    for name in ["u", "delta", "A", "B", "C", "D", "z", "delta_bias"]:
        if x[name] is None:
            assert g["d" + name] is None
            continue
        flat = x[name].reshape(-1)
        idx = rng.choice(flat.size, size=min(6, flat.size), replace=False)
        for i in idx:
            h = 1e-6 * max(1.0, abs(flat[i]))
            orig = flat[i]
            flat[i] = orig + h
            fp = _objective(x, dy, dfs, softplus)
            flat[i] = orig - h
            fm = _objective(x, dy, dfs, softplus)
            flat[i] = orig
            fd = (fp - fm) / (2 * h)
            an = g["d" + name].reshape(-1)[i]
            assert abs(an - fd) <= 2e-7 * max(1.0, abs(fd)), (name, i, an, fd)
            checked += 1
    assert checked >= 20


def test_initial_state_gradients_match_central_differences():
    """With an initial state h0 the transcription's forward is the C oracle's (pinned in test_oracle_ex.py)
    and every gradient, d h0 included, matches central differences of that forward."""
    rng = np.random.default_rng(21)
    batch, L, dim, N = 2, 6, 3, 4
    x = _inputs(rng, batch, L, dim, N)
    h0 = rng.standard_normal((batch, dim, N))
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N))

    def obj():
        y, fs = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                              delta_bias=x["delta_bias"], initial_state=h0)
        return float(np.sum(y * dy) + np.sum(fs * dfs))

    g = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    dfinal_state=dfs, initial_state=h0)
    for arr, name in [(h0, "dinitial_state"), (x["delta"], "ddelta"), (x["A"], "dA")]:
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=6, replace=False):
            e = 1e-6 * max(1.0, abs(flat[i]))
            o = flat[i]
            flat[i] = o + e
            fp = obj()
            flat[i] = o - e
            fm = obj()
            flat[i] = o
            fd = (fp - fm) / (2 * e)
            assert abs(g[name].reshape(-1)[i] - fd) <= 2e-7 * max(1.0, abs(fd)), (name, i)


def test_relay_example_gradients_by_hand():
    """[P1] "The relay": two steps (a1,b1) = (0.6, 0.4) and (a2,b2) = (0.5, 1.0) on N = 1 with A = -1,
    C = 1, u = 1, no softplus, bias, D or gate.  Then y = (b1, a2*b1 + b2) = (0.4, 1.2) and, for dy = (1, 1),
    the objective y1 + y2 = b1*(1 + a2) + b2, whose derivatives follow by hand."""
    d1, d2 = -np.log(0.6), -np.log(0.5)
    u = np.ones((1, 2, 1))
    delta = np.array([d1, d2]).reshape(1, 2, 1)
    A = np.array([[-1.0]])
    B = np.array([0.4 / d1, 1.0 / d2]).reshape(1, 2, 1)
    C = np.ones((1, 2, 1))
    dy = np.ones((1, 2, 1))
    g = OB.scan_bwd(u, delta, A, B, C, dy, softplus=False)
    a2, b1 = 0.5, 0.4
    np.testing.assert_allclose(g["dC"].ravel(), [0.4, 1.2], rtol=1e-14)              # dC_t = h_t
    np.testing.assert_allclose(g["du"].ravel(), [b1 * (1 + a2), 1.0], rtol=1e-14)    # b_t is linear in u_t
    np.testing.assert_allclose(g["dB"].ravel(), [d1 * (1 + a2), d2], rtol=1e-14)     # db_t/dB_t = Delta_t u_t
    # d/dDelta_1: only b1 = Delta_1 B_1 depends on it (h_0 = 0 hides a1); d/dDelta_2: a2 = e^{-Delta_2}, b2
    np.testing.assert_allclose(g["ddelta"].ravel(), [(0.4 / d1) * (1 + a2), -a2 * b1 + 1.0 / d2], rtol=1e-13)
    # dA: a2 = exp(Delta_2 A), da2/dA = Delta_2 a2, times d(obj)/da2 = b1
    np.testing.assert_allclose(g["dA"].ravel(), [d2 * a2 * b1], rtol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 3, 3, 9, 10], [0, 10], [0, 1, 5, 10]])
def test_packed_gradients_match_central_differences(cuts):
    """Packed sequences (an empty and a one-token sequence among them): every gradient, d initial_state per
    sequence included, matches central differences of the C oracle's packed forward (scan_fwd_ex with
    cu_seqlens, pinned in test_oracle_ex.py to independent scans of the slices)."""
    rng = np.random.default_rng(31 + len(cuts))
    L, dim, N = cuts[-1], 3, 4
    x = _inputs(rng, 1, L, dim, N)
    nseq = len(cuts) - 1
    h0 = rng.standard_normal((nseq, dim, N))
    dy = rng.standard_normal((1, L, dim))
    dfs = rng.standard_normal((nseq, dim, N))
    cu = np.asarray(cuts, dtype=np.int64)

    def obj():
        y, fs = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                              delta_bias=x["delta_bias"], initial_state=h0, cu_seqlens=cu)
        return float(np.sum(y * dy) + np.sum(fs * dfs))

    g = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    dfinal_state=dfs, initial_state=h0, cu_seqlens=cu)
    checked = 0
    for arr, name in [(h0, "dinitial_state"), (x["u"], "du"), (x["delta"], "ddelta"), (x["A"], "dA"),
                      (x["B"], "dB"), (x["C"], "dC"), (x["D"], "dD"), (x["z"], "dz"), (x["delta_bias"], "ddelta_bias")]:
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            e = 1e-6 * max(1.0, abs(flat[i]))
            o = flat[i]
            flat[i] = o + e
            fp = obj()
            flat[i] = o - e
            fm = obj()
            flat[i] = o
            fd = (fp - fm) / (2 * e)
            assert abs(g[name].reshape(-1)[i] - fd) <= 2e-7 * max(1.0, abs(fd)), (name, i)
            checked += 1
    assert checked >= 40
    # an empty sequence hands its final-state gradient straight to its initial state
    for s in range(nseq):
        if cuts[s + 1] == cuts[s]:
            np.testing.assert_array_equal(g["dinitial_state"][s], dfs[s])


# ---- the trapezoidal rule (oracle/bwd.py rule="trap"): its own transcription of the three-term recurrence,
# pinned to the C oracle's trapezoidal forward (itself pinned in test_oracle_trap.py) and to central
# differences of it

@pytest.mark.parametrize("softplus,gated,h0", [(True, True, False), (False, False, True), (True, False, True)])
def test_trap_transcription_forward_equals_c_oracle(softplus, gated, h0):
    import torch
    rng = np.random.default_rng(70 + softplus + 2 * gated + 4 * h0)
    x = _inputs(rng, 2, 9, 5, 3, gated=gated)
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05
    init = rng.standard_normal((2, 5, 3)) if h0 else None
    t = {k: (None if v is None else torch.tensor(v)) for k, v in x.items()}
    y, fs = OB.forward_trap_torch(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                  delta_bias=t["delta_bias"], softplus=softplus,
                                  initial_state=None if init is None else torch.tensor(init))
    yo, fo = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                delta_bias=x["delta_bias"], softplus=softplus, initial_state=init)
    assert _rel(y.numpy(), yo) < 1e-13 and _rel(fs.numpy(), fo) < 1e-13


def _fd_check(rng, x, names, grads, obj, count=6, tol=2e-7):
    checked = 0
    for name in names:
        arr = x[name]
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(count, flat.size), replace=False):
            e = 1e-6 * max(1.0, abs(flat[i]))
            o = flat[i]
            flat[i] = o + e
            fp = obj()
            flat[i] = o - e
            fm = obj()
            flat[i] = o
            fd = (fp - fm) / (2 * e)
            an = grads["d" + name].reshape(-1)[i]
            assert abs(an - fd) <= tol * max(1.0, abs(fd)), (name, i, an, fd)
            checked += 1
    return checked


@pytest.mark.parametrize("softplus,gated,with_fs", [(True, True, True), (False, False, False), (True, False, True)])
def test_trap_gradients_match_central_differences_of_c_oracle(softplus, gated, with_fs):
    rng = np.random.default_rng(80 + softplus + 2 * gated + 4 * with_fs)
    batch, L, dim, N = 2, 7, 3, 4
    x = _inputs(rng, batch, L, dim, N, gated=gated)
    if not gated:
        x["D"] = None
        x["delta_bias"] = None
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05
    x["initial_state"] = rng.standard_normal((batch, dim, N))
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N)) if with_fs else None

    def obj():
        y, fs = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                   delta_bias=x["delta_bias"], softplus=softplus, initial_state=x["initial_state"])
        return float(np.sum(y * dy) + (0.0 if dfs is None else np.sum(fs * dfs)))

    g = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    softplus=softplus, dfinal_state=dfs, initial_state=x["initial_state"], rule="trap")
    names = [n for n in ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "initial_state"] if x.get(n) is not None]
    assert _fd_check(rng, x, names, g, obj) >= 30


@pytest.mark.parametrize("cuts", [[0, 3, 3, 9, 10], [0, 1, 5, 10]])
def test_trap_packed_gradients_match_central_differences(cuts):
    """Packed sequences under the trapezoidal rule: each sequence's first token has no previous input."""
    rng = np.random.default_rng(90 + len(cuts))
    L, dim, N = 10, 3, 4
    x = _inputs(rng, 1, L, dim, N)
    nseq = len(cuts) - 1
    x["initial_state"] = rng.standard_normal((nseq, dim, N))
    dy = rng.standard_normal((1, L, dim))
    dfs = rng.standard_normal((nseq, dim, N))
    cu = np.asarray(cuts, dtype=np.int64)

    def obj():
        y, fs = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                   delta_bias=x["delta_bias"], initial_state=x["initial_state"], cu_seqlens=cu)
        return float(np.sum(y * dy) + np.sum(fs * dfs))

    g = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    dfinal_state=dfs, initial_state=x["initial_state"], cu_seqlens=cu, rule="trap")
    names = ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "initial_state"]
    assert _fd_check(rng, x, names, g, obj) >= 40


def test_trap_differs_from_euler_gradients():
    """The rule matters: the two recurrences' gradients differ on the same inputs (a guard against the
    rule argument being ignored)."""
    rng = np.random.default_rng(95)
    x = _inputs(rng, 1, 6, 2, 3)
    dy = rng.standard_normal((1, 6, 2))
    ge = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"])
    gt = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                     rule="trap")
    assert _rel(gt["du"], ge["du"]) > 1e-3 and _rel(gt["dB"], ge["dB"]) > 1e-3
