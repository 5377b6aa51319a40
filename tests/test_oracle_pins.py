"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

None of these tests compares the oracle with itself: each checks it against a
printed worked example, a closed form, a brute-force unrolling written
independently in numpy/scipy, a textbook special function, or an invariant
of the recurrence.  All run on the CPU.
"""
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _golden_relay():
    rows = []
    with open(os.path.join(GOLDEN, "relay_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


# ---------------------------------------------------------------- P-1, P-6
def test_p1_relay_worked_example_composition():
    """'The relay': (0.6, 0.4) then (0.5, 1.0) is (0.3, 1.2); exact in fp64."""
    for a1, b1, a2, b2, a, b in _golden_relay():
        ao, bo = R.pair_then(a1, b1, a2, b2)
        assert ao[()] == a and bo[()] == b


def test_p1_relay_for_any_pad_via_decode():
    """Two decode steps with fade 0.6/add 0.4 then fade 0.5/add 1.0 map any h to 0.3 h + 1.2."""
    (a1, b1, a2, b2, a, b), = _golden_relay()
    rng = np.random.default_rng(1)
    h0 = rng.standard_normal((3, 2, 1)) * 10.0
    A = -np.ones((2, 1))
    st = h0
    for fade, add in ((a1, b1), (a2, b2)):
        dl = -np.log(fade)                  # exp(dl * A) = fade with A = -1
        u = np.ones((3, 2))
        Bm = np.full((3, 1), add / dl)      # dl * B * u = add
        st, _ = R.state_update(st, u, np.full((3, 2), dl), A, Bm, np.ones((3, 1)), softplus=False)
    np.testing.assert_allclose(st, a * h0 + b, rtol=1e-14, atol=1e-14)


def test_p6_relay_end_to_end_scan_n1():
    """Full scan API, one-number state: outputs are the pads 0.4 then 1.2, final pad 1.2."""
    (a1, b1, a2, b2, a, b), = _golden_relay()
    d1, d2 = -np.log(a1), -np.log(a2)
    u = np.ones((1, 2, 1))
    delta = np.array([d1, d2]).reshape(1, 2, 1)
    A = np.array([[-1.0]])
    Bm = np.array([b1 / d1, b2 / d2]).reshape(1, 2, 1)
    Cm = np.ones((1, 2, 1))
    y, fs = R.scan_fwd(u, delta, A, Bm, Cm, D=np.zeros(1), softplus=False)
    np.testing.assert_allclose(y.ravel(), [b1, b], rtol=1e-14)
    np.testing.assert_allclose(fs.ravel(), [b], rtol=1e-14)


# ---------------------------------------------------------------- P-2
def test_p2_associativity_identity_noncommutative():
    rng = np.random.default_rng(2)
    n = 100_000
    a = rng.uniform(0.0, 1.0, size=(3, n))
    b = rng.standard_normal((3, n))
    xy = R.pair_then(a[0], b[0], a[1], b[1])
    left = R.pair_then(xy[0], xy[1], a[2], b[2])
    yz = R.pair_then(a[1], b[1], a[2], b[2])
    right = R.pair_then(a[0], b[0], yz[0], yz[1])
    scale = 1.0 + np.abs(b).sum(axis=0)
    assert np.max(np.abs(left[0] - right[0])) <= 4 * np.finfo(float).eps
    assert np.max(np.abs(left[1] - right[1]) / scale) <= 8 * np.finfo(float).eps
    # identity (1, 0) on either side
    one, zero = np.ones(n), np.zeros(n)
    for ao, bo in (R.pair_then(one, zero, a[0], b[0]), R.pair_then(a[0], b[0], one, zero)):
        assert np.array_equal(ao, a[0]) and np.array_equal(bo, b[0])
    # the order matters: (0.6,0.4) then (0.5,1.0) differs from the reverse
    f = R.pair_then(0.6, 0.4, 0.5, 1.0)
    r = R.pair_then(0.5, 1.0, 0.6, 0.4)
    assert f[1][()] != r[1][()]


# ---------------------------------------------------------------- P-3
def _fold_random_tree(rng, a, b):
    """Compose pairs a[i], b[i] (i ascending) with a random bracketing."""
    if len(a) == 1:
        return a[0], b[0]
    k = int(rng.integers(1, len(a)))
    la, lb = _fold_random_tree(rng, a[:k], b[:k])
    ra, rb = _fold_random_tree(rng, a[k:], b[k:])
    ao, bo = R.pair_then(la, lb, ra, rb)
    return ao[()], bo[()]


def test_p3_any_bracketing_equals_recurrence():
    rng = np.random.default_rng(3)
    L, N = 48, 3
    delta = rng.uniform(0.01, 0.6, size=(1, L, 1))
    A = -rng.uniform(0.2, 3.0, size=(1, N))
    Bm = rng.standard_normal((1, L, N))
    u = rng.standard_normal((1, L, 1))
    for n in range(N):
        Cm = np.zeros((1, L, N))
        Cm[..., n] = 1.0                     # y_t = h_t[n]
        y, _ = R.scan_fwd(u, delta, A, Bm, Cm, D=np.zeros(1), softplus=False)
        a = np.exp(delta[0, :, 0] * A[0, n])
        b = delta[0, :, 0] * Bm[0, :, n] * u[0, :, 0]
        for t in range(L):
            for _ in range(3):
                _, bt = _fold_random_tree(rng, a[: t + 1], b[: t + 1])
                assert abs(bt - y[0, t, 0]) <= 1e-13 * (1 + abs(y[0, t, 0]))
        # chunked: squash each chunk to one pair, combine chunk pairs, then pass pads back
        for chunk in (1, 2, 5, 7, 16, L):
            h = 0.0
            for s in range(0, L, chunk):
                ca, cb = _fold_random_tree(rng, a[s:s + chunk], b[s:s + chunk])
                h = ca * h + cb
                assert abs(h - y[0, min(s + chunk, L) - 1, 0]) <= 1e-13 * (1 + abs(h))


# ---------------------------------------------------------------- P-4
def test_p4_lti_closed_form_convolution():
    """Constant delta, B, C: y = K * u + D u with K_k = sum_n C_n exp(delta A_n)^k delta B_n."""
    rng = np.random.default_rng(4)
    bt, L, dim, N = 2, 300, 3, 4
    dl = rng.uniform(0.005, 0.3, size=dim)
    A = -rng.uniform(0.1, 2.0, size=(dim, N))
    Bc = rng.standard_normal((bt, N))
    Cc = rng.standard_normal((bt, N))
    D = rng.standard_normal(dim)
    u = rng.standard_normal((bt, L, dim))
    delta = np.broadcast_to(dl, (bt, L, dim))
    Bm = np.broadcast_to(Bc[:, None, :], (bt, L, N))
    Cm = np.broadcast_to(Cc[:, None, :], (bt, L, N))
    y, _ = R.scan_fwd(u, delta, A, Bm, Cm, D=D, softplus=False)
    k = np.arange(L)
    for b in range(bt):
        for d in range(dim):
            K = np.zeros(L)
            for n in range(N):
                K += Cc[b, n] * np.exp(dl[d] * A[d, n] * k) * dl[d] * Bc[b, n]
            direct = np.convolve(K, u[b, :, d])[:L] + D[d] * u[b, :, d]
            nfft = 1 << int(np.ceil(np.log2(2 * L)))
            viafft = np.fft.irfft(np.fft.rfft(K, nfft) * np.fft.rfft(u[b, :, d], nfft), nfft)[:L] + D[d] * u[b, :, d]
            assert _rel(y[b, :, d], direct) < 1e-12
            assert _rel(y[b, :, d], viafft) < 1e-11


# ---------------------------------------------------------------- P-5
def _softplus_np(x):
    return np.logaddexp(0.0, x)


def _brute_force(u, draw, A, Bm, Cm, D, z, bias):
    """y_t = [sum_{s<=t} sum_n C_t[n] (prod_{r=s+1..t} a_r[n]) b_s[n] + D u_t] * silu(z_t)."""
    bt, L, dim = u.shape
    N = A.shape[1]
    dl = _softplus_np(draw + bias[None, None, :])
    y = np.zeros_like(u)
    fs = np.zeros((bt, dim, N))
    for b in range(bt):
        for d in range(dim):
            a = np.exp(dl[b, :, d, None] * A[d][None, :])          # [L, N]
            bb = dl[b, :, d, None] * Bm[b] * u[b, :, d, None]        # [L, N]
            # final state: h_{L-1}[n] = sum_s (prod_{r=s+1..L-1} a_r[n]) b_s[n]
            for s in range(L):
                fs[b, d] += np.prod(a[s + 1:L], axis=0) * bb[s]
            for t in range(L):
                acc = 0.0
                for s in range(t + 1):
                    acc += np.sum(Cm[b, t] * np.prod(a[s + 1:t + 1], axis=0) * bb[s])
                v = acc + D[d] * u[b, t, d]
                if z is not None:
                    v *= z[b, t, d] * expit(z[b, t, d])
                y[b, t, d] = v
    return y, fs


@pytest.mark.parametrize("seed,L,N,gate", [(5, 1, 1, True), (6, 7, 2, True), (7, 16, 4, True), (8, 13, 3, False)])
def test_p5_brute_force_unrolling(seed, L, N, gate):
    rng = np.random.default_rng(seed)
    bt, dim = 2, 3
    u = rng.standard_normal((bt, L, dim))
    draw = rng.standard_normal((bt, L, dim))
    A = -rng.uniform(0.05, 2.0, size=(dim, N))        # independent per (d, n): catches a transposed A
    Bm = rng.standard_normal((bt, L, N))
    Cm = rng.standard_normal((bt, L, N))
    D = rng.standard_normal(dim)
    z = rng.standard_normal((bt, L, dim)) if gate else None
    bias = np.log(np.expm1(rng.uniform(1e-3, 0.5, size=dim)))
    yb, fsb = _brute_force(u, draw, A, Bm, Cm, D, z, bias)
    y, fs = R.scan_fwd(u, draw, A, Bm, Cm, D=D, z=z, delta_bias=bias, softplus=True)
    assert _rel(y, yb) < 1e-12
    assert _rel(fs, fsb) < 1e-12


# ---------------------------------------------------------------- P-7
def test_p7_delta_limits():
    rng = np.random.default_rng(9)
    bt, dim, N = 2, 5, 4
    h = rng.standard_normal((bt, dim, N))
    A = -rng.uniform(0.1, 2.0, size=(dim, N))
    u = rng.standard_normal((bt, dim))
    Bm = rng.standard_normal((bt, N))
    Cm = rng.standard_normal((bt, N))
    D = rng.standard_normal(dim)
    # delta = 0: the state is untouched and y reads the old state
    st, y = R.state_update(h, u, np.zeros((bt, dim)), A, Bm, Cm, D=D, softplus=False)
    assert np.array_equal(st, h)
    np.testing.assert_allclose(y, np.einsum("bn,bdn->bd", Cm, h) + D * u, rtol=1e-13, atol=1e-13)
    # tiny delta: almost untouched
    st, _ = R.state_update(h, u, np.full((bt, dim), 1e-12), A, Bm, Cm, softplus=False)
    assert np.max(np.abs(st - h)) < 1e-10
    # large delta with A < 0: the old state is forgotten, h = delta * B * u
    big = 60.0
    st, _ = R.state_update(h, u, np.full((bt, dim), big), A * 0 - 1.0, Bm, Cm, softplus=False)
    expect = big * Bm[:, None, :] * u[:, :, None]
    np.testing.assert_allclose(st, expect, rtol=1e-15, atol=1e-20)


# ---------------------------------------------------------------- P-8, P-9, P-11
def _rand_scan(rng, bt=2, L=40, dim=4, N=3):
    return dict(
        u=rng.standard_normal((bt, L, dim)), delta=rng.standard_normal((bt, L, dim)),
        A=-rng.uniform(0.1, 2.0, size=(dim, N)), B=rng.standard_normal((bt, L, N)),
        C=rng.standard_normal((bt, L, N)), D=rng.standard_normal(dim), z=rng.standard_normal((bt, L, dim)),
        delta_bias=np.log(np.expm1(rng.uniform(1e-3, 0.1, size=dim))))


def test_p8_linearity_in_u():
    rng = np.random.default_rng(10)
    p = _rand_scan(rng)
    p.pop("z")
    u1, u2 = rng.standard_normal(p["u"].shape), rng.standard_normal(p["u"].shape)
    al, be = 0.7, -1.9
    q = dict(p)
    q.pop("u")
    y1, f1 = R.scan_fwd(u1, **q)
    y2, f2 = R.scan_fwd(u2, **q)
    y12, f12 = R.scan_fwd(al * u1 + be * u2, **q)
    assert _rel(y12, al * y1 + be * y2) < 1e-13
    assert _rel(f12, al * f1 + be * f2) < 1e-13


def test_p9_causality_bitwise():
    rng = np.random.default_rng(11)
    p = _rand_scan(rng, L=50)
    y0, _ = R.scan_fwd(**p)
    t0 = 23
    for key in ("u", "delta", "z", "B", "C"):
        q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
        q[key][:, t0:] += rng.standard_normal(q[key][:, t0:].shape)
        y1, _ = R.scan_fwd(**q)
        assert np.array_equal(y1[:, :t0], y0[:, :t0])
        assert not np.array_equal(y1[:, t0], y0[:, t0])


def test_p11_zero_input():
    rng = np.random.default_rng(12)
    p = _rand_scan(rng)
    p["u"] = np.zeros_like(p["u"])
    y, fs = R.scan_fwd(**p)
    assert np.all(y == 0.0) and np.all(fs == 0.0)


# ---------------------------------------------------------------- P-10
def test_p10_scan_equals_repeated_decode_and_continuation():
    rng = np.random.default_rng(13)
    bt, L, dim, N = 2, 30, 5, 4
    p = _rand_scan(rng, bt, L + 1, dim, N)
    full_y, full_fs = R.scan_fwd(**p)
    part = {k: (v[:, :L] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    y, fs = R.scan_fwd(**part)
    assert np.array_equal(y, full_y[:, :L])
    # L decode steps from zero reproduce the scan
    st = np.zeros((bt, dim, N))
    for t in range(L):
        st, yt = R.state_update(st, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t], p["C"][:, t],
                                D=p["D"], z=p["z"][:, t], delta_bias=p["delta_bias"])
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st, fs, rtol=1e-14, atol=1e-14)
    # scan(L) then one decode step equals scan(L + 1)
    st, yt = R.state_update(fs, p["u"][:, L], p["delta"][:, L], p["A"], p["B"][:, L], p["C"][:, L],
                            D=p["D"], z=p["z"][:, L], delta_bias=p["delta_bias"])
    np.testing.assert_allclose(yt, full_y[:, L], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st, full_fs, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- epilogue functions
@pytest.mark.parametrize("x", [-745.0, -40.0, -20.0, -5.0, -1e-3, 0.0, 1e-3, 1.0, 5.0, 20.0, 40.0, 700.0])
def test_softplus_matches_logaddexp(x):
    ref = np.logaddexp(0.0, x)
    assert abs(R.softplus(x) - ref) <= 2e-16 * max(abs(ref), 1e-300) + 1e-320
    # and through the full scan: L = 1, N = 1, u = B = C = 1, D = 0 -> y = softplus(raw + bias)
    y, _ = R.scan_fwd(np.ones((1, 1, 1)), np.array([[[x - 0.25]]]), -np.ones((1, 1)), np.ones((1, 1, 1)),
                      np.ones((1, 1, 1)), D=np.zeros(1), delta_bias=np.array([0.25]), softplus=True)
    assert abs(y[0, 0, 0] - ref) <= 4e-16 * max(abs(ref), 1e-300) + 1e-320


@pytest.mark.parametrize("zz", [-50.0, -5.0, -1.0, -1e-6, 0.0, 1e-6, 1.0, 5.0, 50.0])
def test_silu_gate_matches_expit(zz):
    ref = zz * expit(zz)
    assert abs(R.silu(zz) - ref) <= 4e-16 * max(abs(ref), 1e-300)
    # through the scan: delta = 1 (softplus off), u = B = C = 1, D = 0 -> y = (1 - 0 ... ) = 1 * silu(z)
    y, _ = R.scan_fwd(np.ones((1, 1, 1)), np.ones((1, 1, 1)), -np.ones((1, 1)), np.ones((1, 1, 1)),
                      np.ones((1, 1, 1)), D=np.zeros(1), z=np.array([[[zz]]]), softplus=False)
    assert abs(y[0, 0, 0] - ref) <= 4e-16 * max(abs(ref), 1e-300)


def test_d_skip_alone():
    """B = 0 keeps the state at zero, so y = D u SiLU(z)."""
    rng = np.random.default_rng(14)
    p = _rand_scan(rng)
    p["B"] = np.zeros_like(p["B"])
    y, fs = R.scan_fwd(**p)
    expect = p["D"][None, None, :] * p["u"] * p["z"] * expit(p["z"])
    assert _rel(y, expect) < 1e-15 and np.all(fs == 0.0)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(15)
    p = _rand_scan(rng, bt=3, L=60, dim=7, N=5)
    y1, f1 = R.scan_fwd(**p, nthreads=1)
    y7, f7 = R.scan_fwd(**p, nthreads=7)
    assert np.array_equal(y1, y7) and np.array_equal(f1, f7)


def test_optional_arguments_default_to_zero():
    rng = np.random.default_rng(16)
    p = _rand_scan(rng)
    y_none, _ = R.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], softplus=False)
    y_zero, _ = R.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=np.zeros(p["A"].shape[0]),
                           delta_bias=np.zeros(p["A"].shape[0]), softplus=False)
    assert np.array_equal(y_none, y_zero)


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        R.scan_fwd(np.ones((1, 0, 1)), np.ones((1, 0, 1)), np.ones((1, 1)), np.ones((1, 0, 1)), np.ones((1, 0, 1)))
