"""Pins of the C backward oracle (oracle/ssm_ref.c: ssm_ref_scan_bwd, front end oracle/ref.py: scan_bwd), CPU only.

It computes the gradients by a hand-derived adjoint recurrence, written apart from the automatic
differentiation of oracle/bwd.py.  It is pinned against things outside itself:
  - central finite differences of the C oracle's forward, for every input, the initial state and the final
    state's gradient included;
  - the pages' two-token relay example ([P1] "The relay"), with its gradients derived by hand;
  - the automatic-differentiation oracle, on every combination of the optional inputs;
  - the number of worker threads, which may change only the order of the cross-channel sums.
"""
import numpy as np
import pytest

from oracle import bwd as OB
from oracle import ref as R


def _inputs(rng, batch, L, dim, N, gated=True, with_D=True, with_bias=True):
    return dict(
        u=rng.standard_normal((batch, L, dim)),
        delta=rng.standard_normal((batch, L, dim)) * 0.5 - 1.0,
        A=-np.exp(rng.standard_normal((dim, N)) * 0.5),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(dim) if with_D else None,
        z=rng.standard_normal((batch, L, dim)) if gated else None,
        delta_bias=rng.standard_normal(dim) * 0.3 if with_bias else None,
    )


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _bwd(x, dy, dfs, softplus=True, h0=None, nthreads=1):
    return R.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                      delta_bias=x["delta_bias"], softplus=softplus, dfinal_state=dfs, initial_state=h0,
                      nthreads=nthreads)


@pytest.mark.parametrize("softplus,gated,with_fs,with_h0", [(True, True, True, True), (True, True, False, False),
                                                            (False, False, True, False), (True, False, True, True)])
def test_gradients_match_central_differences(softplus, gated, with_fs, with_h0):
    rng = np.random.default_rng(31 + 8 * softplus + 4 * gated + 2 * with_fs + with_h0)
    batch, L, dim, N = 2, 7, 3, 4
    x = _inputs(rng, batch, L, dim, N, gated=gated, with_D=gated, with_bias=gated)
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05   # the step as given: keep it positive
    h0 = rng.standard_normal((batch, dim, N)) if with_h0 else None
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N)) if with_fs else None
    g = _bwd(x, dy, dfs, softplus=softplus, h0=h0)

    def obj():
        y, fs = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                              delta_bias=x["delta_bias"], softplus=softplus, initial_state=h0)
        return float(np.sum(y * dy) + (np.sum(fs * dfs) if dfs is not None else 0.0))

    arrays = [(x[n], "d" + n) for n in ["u", "delta", "A", "B", "C", "D", "z", "delta_bias"]]
    if h0 is not None:
        arrays.append((h0, "dinitial_state"))
    checked = 0
    for arr, name in arrays:
        if arr is None:
            assert g[name] is None, name
            continue
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
            an = g[name].reshape(-1)[i]
            assert abs(an - fd) <= 2e-7 * max(1.0, abs(fd)), (name, i, an, fd)
            checked += 1
    assert checked >= 24


def test_relay_example_gradients_by_hand():
    """[P1] "The relay": (a1, b1) = (0.6, 0.4) then (a2, b2) = (0.5, 1.0) on N = 1 with A = -1, C = 1, u = 1 and
    no softplus, bias, D or gate, so y = (0.4, 1.2); for dy = (1, 1) the objective is b1 (1 + a2) + b2."""
    d1, d2 = -np.log(0.6), -np.log(0.5)
    x = dict(u=np.ones((1, 2, 1)), delta=np.array([d1, d2]).reshape(1, 2, 1), A=np.array([[-1.0]]),
             B=np.array([0.4 / d1, 1.0 / d2]).reshape(1, 2, 1), C=np.ones((1, 2, 1)), D=None, z=None,
             delta_bias=None)
    g = _bwd(x, np.ones((1, 2, 1)), None, softplus=False)
    a2, b1 = 0.5, 0.4
    np.testing.assert_allclose(g["dC"].ravel(), [0.4, 1.2], rtol=1e-14)
    np.testing.assert_allclose(g["du"].ravel(), [b1 * (1 + a2), 1.0], rtol=1e-14)
    np.testing.assert_allclose(g["dB"].ravel(), [d1 * (1 + a2), d2], rtol=1e-14)
    np.testing.assert_allclose(g["ddelta"].ravel(), [(0.4 / d1) * (1 + a2), -a2 * b1 + 1.0 / d2], rtol=1e-13)
    np.testing.assert_allclose(g["dA"].ravel(), [d2 * a2 * b1], rtol=1e-13)
    # the gradient reaching the (zero) initial state: through both fades, d obj / d h0 = a1 (1 + a2)
    np.testing.assert_allclose(g["dinitial_state"].ravel(), [0.6 * (1 + a2)], rtol=1e-13)


OPTS = ["all", "no_z", "no_D", "no_bias", "no_softplus", "h0"]


@pytest.mark.parametrize("opts", OPTS)
def test_agrees_with_autograd_oracle(opts):
    rng = np.random.default_rng(50 + OPTS.index(opts))
    batch, L, dim, N = 2, 37, 5, 6
    x = _inputs(rng, batch, L, dim, N, gated=opts != "no_z", with_D=opts != "no_D", with_bias=opts != "no_bias")
    softplus = opts != "no_softplus"
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05
    h0 = rng.standard_normal((batch, dim, N)) * 0.5 if opts == "h0" else None
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N))
    a = _bwd(x, dy, dfs, softplus=softplus, h0=h0, nthreads=3)
    b = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    softplus=softplus, dfinal_state=dfs, initial_state=h0)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias"):
        assert (a[k] is None) == (b[k] is None), k
        if a[k] is not None:
            assert _rel(a[k], b[k]) < 1e-12, (k, _rel(a[k], b[k]))
    if h0 is not None:
        assert _rel(a["dinitial_state"], b["dinitial_state"]) < 1e-12


def test_thread_count_changes_only_the_order_of_sums():
    rng = np.random.default_rng(77)
    x = _inputs(rng, 3, 50, 7, 5)
    dy = rng.standard_normal((3, 50, 7))
    dfs = rng.standard_normal((3, 7, 5))
    g1 = _bwd(x, dy, dfs, nthreads=1)
    g5 = _bwd(x, dy, dfs, nthreads=5)
    for k in ("du", "ddelta", "dz", "dinitial_state"):   # one (row, channel) each: bitwise the same
        assert np.array_equal(g1[k], g5[k]), k
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):     # sums over channels or rows: the order may differ
        assert _rel(g5[k], g1[k]) < 1e-13, k
    assert all(np.array_equal(_bwd(x, dy, dfs, nthreads=5)[k], g5[k]) for k in g5 if g5[k] is not None)


# The trapezoidal rule (ssm_ref_scan_trap_bwd): the backward of ssm_ref_scan_trap_fwd_ex, pinned the same way
# against that forward.

@pytest.mark.parametrize("softplus,gated,with_h0", [(True, True, True), (False, False, False)])
def test_trap_gradients_match_central_differences(softplus, gated, with_h0):
    rng = np.random.default_rng(61 + 2 * softplus + with_h0)
    batch, L, dim, N = 2, 7, 3, 4
    x = _inputs(rng, batch, L, dim, N, gated=gated, with_D=gated, with_bias=gated)
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05
    h0 = rng.standard_normal((batch, dim, N)) if with_h0 else None
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N))
    g = R.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                   softplus=softplus, dfinal_state=dfs, initial_state=h0, rule="trap")

    def obj():
        y, fs = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                   delta_bias=x["delta_bias"], softplus=softplus, initial_state=h0)
        return float(np.sum(y * dy) + np.sum(fs * dfs))

    arrays = [(x[n], "d" + n) for n in ["u", "delta", "A", "B", "C", "D", "z", "delta_bias"]]
    if h0 is not None:
        arrays.append((h0, "dinitial_state"))
    checked = 0
    for arr, name in arrays:
        if arr is None:
            assert g[name] is None, name
            continue
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
            an = g[name].reshape(-1)[i]
            assert abs(an - fd) <= 2e-7 * max(1.0, abs(fd)), (name, i, an, fd)
            checked += 1
    assert checked >= 24


@pytest.mark.parametrize("opts", ["all", "no_z", "no_softplus", "h0"])
def test_trap_agrees_with_autograd_oracle(opts):
    rng = np.random.default_rng(70 + ["all", "no_z", "no_softplus", "h0"].index(opts))
    batch, L, dim, N = 2, 29, 5, 6
    x = _inputs(rng, batch, L, dim, N, gated=opts != "no_z")
    softplus = opts != "no_softplus"
    if not softplus:
        x["delta"] = np.abs(x["delta"]) + 0.05
    h0 = rng.standard_normal((batch, dim, N)) * 0.5 if opts == "h0" else None
    dy = rng.standard_normal((batch, L, dim))
    dfs = rng.standard_normal((batch, dim, N))
    a = R.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                   softplus=softplus, dfinal_state=dfs, initial_state=h0, nthreads=2, rule="trap")
    b = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                    softplus=softplus, dfinal_state=dfs, initial_state=h0, rule="trap")
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias"):
        assert (a[k] is None) == (b[k] is None), k
        if a[k] is not None:
            assert _rel(a[k], b[k]) < 1e-12, (k, _rel(a[k], b[k]))
    if h0 is not None:
        assert _rel(a["dinitial_state"], b["dinitial_state"]) < 1e-12
