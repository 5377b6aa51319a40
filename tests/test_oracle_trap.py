"""Pins of the oracle's Mamba-3 trapezoidal scan (ref.scan_trap_fwd_ex), on the CPU.

The page ("The State That Must Remember Everything", Part 7, "Mamba-3 (2026)")
gives the three-term recurrence h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1}
+ gamma_t B_t x_t and calls it a trapezoidal variant of exponential-Euler; the
oracle reads alpha = exp(delta A), beta = delta/2 exp(delta A), gamma = delta/2
(the trapezoidal rule on the step's input integral).  The pins tie that
reading to facts that do not come from the oracle:
  - the response to one input impulse, derived by hand;
  - the closed form of the recurrence under constant inputs;
  - second-order convergence to the exact solution of the continuous model
    h' = A h + B x(t) (the defining property of a trapezoidal rule, against
    first order for exponential-Euler);
  - with A = 0 the state is numpy's cumulative trapezoid of delta * B x;
  - an initial state only adds its own decay, exp(A * sum delta) h_{-1};
  - packed sequences are independent scans, each with a zero previous input.
"""
import numpy as np
import pytest

from oracle import ref as R
from selective_state_space_33_amd import inputs as I


def _plain(u, dl, A, B, C, **kw):
    """Trapezoidal scan with softplus off, no bias, no D, no gate: delta is used as given."""
    return R.scan_trap_fwd_ex(u, dl, A, B, C, softplus=False, **kw)


def test_impulse_response_by_hand():
    rng = np.random.default_rng(1)
    L, dim, N, tau = 9, 3, 4, 3
    u = np.zeros((1, L, dim))
    u[0, tau] = rng.standard_normal(dim)
    dl = rng.uniform(0.05, 0.6, (1, L, dim))
    A = -rng.uniform(0.2, 2.0, (dim, N))
    B = rng.standard_normal((1, L, N))
    C = rng.standard_normal((1, L, N))
    y, fs = _plain(u, dl, A, B, C)
    assert np.all(y[0, :tau] == 0.0)
    for d in range(dim):
        # token tau: only gamma_tau B_tau u_tau (the previous input is zero)
        h = 0.5 * dl[0, tau, d] * B[0, tau] * u[0, tau, d]
        np.testing.assert_allclose(y[0, tau, d], C[0, tau] @ h, rtol=1e-13, atol=1e-15)
        # later tokens: the impulse enters once more through beta_{tau+1}, then only fades
        w = 0.5 * (dl[0, tau, d] + dl[0, tau + 1, d]) * B[0, tau] * u[0, tau, d]
        for t in range(tau + 1, L):
            h_t = np.exp(A[d] * dl[0, tau + 1:t + 1, d].sum()) * w
            np.testing.assert_allclose(y[0, t, d], C[0, t] @ h_t, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(fs[0, d], h_t, rtol=1e-12, atol=1e-15)


def test_constant_inputs_closed_form():
    L, N = 40, 3
    a_cont = np.array([[-0.3, -1.1, -2.5]])
    dlt, x = 0.25, 0.7
    Bv = np.array([0.4, -1.3, 0.9])
    Cv = np.array([1.2, 0.5, -0.8])
    u = np.full((1, L, 1), x)
    dl = np.full((1, L, 1), dlt)
    B = np.tile(Bv, (1, L, 1))
    C = np.tile(Cv, (1, L, 1))
    y, fs = _plain(u, dl, a_cont, B, C)
    alpha = np.exp(dlt * a_cont[0])
    beta, gamma = 0.5 * dlt * alpha, 0.5 * dlt
    h0 = gamma * Bv * x                               # the first token has no previous input
    hstar = (beta + gamma) * Bv * x / (1.0 - alpha)   # fixed point of h = alpha h + (beta + gamma) B x
    for t in range(L):
        h_t = hstar + (h0 - hstar) * alpha ** t
        np.testing.assert_allclose(y[0, t, 0], Cv @ h_t, rtol=1e-12)
    np.testing.assert_allclose(fs[0, 0], hstar + (h0 - hstar) * alpha ** (L - 1), rtol=1e-12)


def _ode_error(steps, omega=3.0, a=-1.0, T=2.0):
    """|h(T) - exact| for h' = a h + sin(omega s), h(0) = 0, sampled at s = (t+1) T/steps."""
    dt = T / steps
    s = dt * np.arange(1, steps + 1)
    u = np.sin(omega * s).reshape(1, steps, 1)
    dl = np.full((1, steps, 1), dt)
    ones = np.ones((1, steps, 1))
    _, fs = _plain(u, dl, np.array([[a]]), ones, ones)
    exact = (-a * np.sin(omega * T) - omega * np.cos(omega * T) + omega * np.exp(a * T)) / (a * a + omega * omega)
    return abs(fs[0, 0, 0] - exact)


def test_second_order_convergence_to_the_continuous_model():
    # the first token's previous input is x(0) = sin(0) = 0, as the recurrence assumes
    e1, e2, e3 = _ode_error(50), _ode_error(100), _ode_error(200)
    assert e1 < 2e-3
    for coarse, fine in ((e1, e2), (e2, e3)):
        assert 3.6 < coarse / fine < 4.4, (e1, e2, e3)   # halving the step quarters the error


def test_no_decay_is_the_cumulative_trapezoid():
    rng = np.random.default_rng(2)
    L, dim, N = 30, 2, 3
    u = rng.standard_normal((1, L, dim))
    dl = rng.uniform(0.1, 0.5, (1, L, dim))
    B = rng.standard_normal((1, L, N))
    C = rng.standard_normal((1, L, N))
    _, fs = _plain(u, dl, np.zeros((dim, N)), B, C)
    for d in range(dim):
        f = B[0] * u[0, :, d, None]                   # B_t x_t, [L, N]
        fprev = np.vstack([np.zeros((1, N)), f[:-1]])  # zero before the first token
        area = (0.5 * dl[0, :, d, None] * (fprev + f)).sum(axis=0)
        np.testing.assert_allclose(fs[0, d], area, rtol=1e-12)


def test_initial_state_adds_its_own_decay():
    rng = np.random.default_rng(3)
    x = I.random_scan_inputs(rng, 2, 25, 4, 3, dtype="f32")
    h0 = rng.standard_normal((2, 4, 3))
    kw = dict(D=x["D"], delta_bias=x["delta_bias"])
    y0, f0 = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], **kw)
    y1, f1 = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], initial_state=h0, **kw)
    f64 = lambda a: np.asarray(a, np.float64)
    dl = np.logaddexp(0.0, f64(x["delta"]) + f64(x["delta_bias"]))   # softplus(delta_raw + bias)
    decay = np.exp(np.cumsum(dl, axis=1)[..., None] * f64(x["A"]))   # [batch, L, dim, N]
    extra = np.einsum("btn,btdn->btd", f64(x["C"]), decay * h0[:, None])
    np.testing.assert_allclose(y1 - y0, extra, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(f1 - f0, decay[:, -1] * h0, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("cu", [[0, 50], [0, 1, 20, 20, 50], [0, 25, 50]])
def test_packed_sequences_are_independent_trapezoidal_scans(cu):
    rng = np.random.default_rng(4)
    x = I.random_scan_inputs(rng, 1, 50, 5, 4, dtype="f32")
    nseq = len(cu) - 1
    h0 = rng.standard_normal((nseq, 5, 4))
    kw = dict(D=x["D"], delta_bias=x["delta_bias"])
    y, f = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"], z=x["z"], initial_state=h0,
                              cu_seqlens=cu, **kw)
    for s in range(nseq):
        a, b = cu[s], cu[s + 1]
        if a == b:
            np.testing.assert_array_equal(f[s], h0[s])
            continue
        sl = lambda t: np.ascontiguousarray(t[:, a:b])
        ys, fs = R.scan_trap_fwd_ex(sl(x["u"]), sl(x["delta"]), x["A"], sl(x["B"]), sl(x["C"]), z=sl(x["z"]),
                                    initial_state=h0[s:s + 1], **kw)
        np.testing.assert_array_equal(y[:, a:b], ys)
        np.testing.assert_array_equal(f[s], fs[0])


def test_differs_from_exponential_euler():
    """The three-term rule is not the two-term one (guards against a silent fallback)."""
    x = I.random_scan_inputs(np.random.default_rng(5), 1, 20, 3, 2, dtype="f32")
    yt, _ = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"])
    ye, _ = R.scan_fwd_ex(x["u"], x["delta"], x["A"], x["B"], x["C"])
    assert np.abs(yt - ye).max() > 1e-3 * np.abs(ye).max()


def test_skip_and_gate_alone():
    """B = 0 keeps the state at zero, so y = D u SiLU(z) with SiLU(z) = z * expit(z)."""
    from scipy.special import expit

    x = I.random_scan_inputs(np.random.default_rng(6), 2, 15, 4, 3, dtype="f32")
    f64 = lambda a: np.asarray(a, np.float64)
    y, fs = R.scan_trap_fwd_ex(x["u"], x["delta"], x["A"], np.zeros_like(x["B"]), x["C"], D=x["D"], z=x["z"],
                               delta_bias=x["delta_bias"])
    z = f64(x["z"])
    np.testing.assert_allclose(y, f64(x["D"]) * f64(x["u"]) * z * expit(z), rtol=1e-13, atol=1e-15)
    assert np.all(fs == 0.0)
