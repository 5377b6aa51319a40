"""GPU parity: the HIP path (called through the C ABI) against the fp64 CPU oracle.

Every output is compared element by element with the oracle, the full-size
workloads included (in the default launch plan, the one the benchmark times;
the oracle runs threaded over channels).  Tolerances: max relative error 1e-4
(fp32 storage) and 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from oracle import ref as R
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import (TOL, BlockLen, Chained, Variant, gpu_scan, oracle_scan, oracle_threads, rel_err, say,
                       to_dev, to_dev_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


def _compare_scan(x, dtype, tol=None, **kw):
    tol = TOL[dtype] if tol is None else tol
    y, fs = gpu_scan(x, dtype, **kw)
    yo, fo = oracle_scan(x, **kw)
    ey, ef = rel_err(y, yo), rel_err(fs, fo)
    print(f"[parity] y err {ey:.3e}  final-state err {ef:.3e}  (tol {tol})", flush=True)
    assert ey <= tol and ef <= tol, f"y err {ey:.3e}, final-state err {ef:.3e} (tol {tol})"
    return ey, ef


# ------------------------------------------------------------------ the five workloads
def test_tiny_fp32_full():
    w = I.WORKLOADS["tiny_fp32"]
    say(f"scan {w}")
    _compare_scan(I.make_inputs(w, 0), "f32")


def test_decode_full_size():
    w = I.WORKLOADS["decode_bf16"]
    x = I.make_inputs(w, 0)
    say(f"decode {w}")
    st = to_dev_f32(x["h0"])
    y = ops.ssm_state_update(st, to_dev(x["u"], "bf16"), to_dev(x["delta"], "bf16"), to_dev_f32(x["A"]),
                             to_dev(x["B"], "bf16"), to_dev(x["C"], "bf16"), D=to_dev_f32(x["D"]),
                             z=to_dev(x["z"], "bf16"), delta_bias=to_dev_f32(x["delta_bias"]))
    torch.cuda.synchronize()
    so, yo = R.state_update(x["h0"], x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                            delta_bias=x["delta_bias"])
    ey = rel_err(y.float().cpu().numpy(), yo)
    es = rel_err(st.cpu().numpy(), so)
    print(f"[parity] decode full size: y err {ey:.3e}  state err {es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"], (ey, es)
    # the state is fp32 and its update involves no bf16 rounding of outputs: much tighter in practice
    assert es <= 1e-5, es


@pytest.mark.parametrize("name", ["mamba130m_bf16", "mamba2p8b_bf16", "long_audio_fp32"])
def test_full_size_all_channels(name):
    """Full-size workload in the default launch plan (the one the benchmark times): every output against the
    oracle run on the whole workload (its threads split the independent channels)."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w, 0)
    say(f"full-size scan {w}")
    y, fs = gpu_scan(x, w.dtype, with_z=w.gate)
    yo, fo = oracle_scan(x, with_z=w.gate, nthreads=oracle_threads())
    ey, ef = rel_err(y, yo), rel_err(fs, fo)
    print(f"[parity] {name} all {w.batch * w.dim} channels: y err {ey:.3e}  final-state err {ef:.3e}", flush=True)
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype], f"{name}: y err {ey:.3e}, final-state err {ef:.3e}"


# ------------------------------------------------------------------ reduced shapes, full compare
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("batch,L,dim", [(2, 300, 200), (3, 97, 130), (1, 1, 64), (2, 1000, 68)])
def test_ragged_shapes_default_plan(dtype, batch, L, dim):
    """Tails in time (not a multiple of the token block) and in channels (not a multiple of 64 / of 4)."""
    rng = np.random.default_rng(batch * 1000 + L + dim)
    x = I.random_scan_inputs(rng, batch, L, dim, 16, dtype=dtype)
    say(f"ragged {dtype} {batch}x{L}x{dim}")
    _compare_scan(x, dtype)


VARIANTS = [(2, 8), (1, 16), (4, 4), (8, 2), (16, 1)]


@pytest.mark.parametrize("npl,G", VARIANTS)
@pytest.mark.parametrize("K", [1, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_every_variant_and_chunking(npl, G, K, dtype):
    rng = np.random.default_rng(npl * 100 + G * 10 + K)
    x = I.random_scan_inputs(rng, 2, 777, 136, 16, dtype=dtype)
    say(f"variant npl={npl} G={G} K={K} {dtype}")
    with Variant(npl, G, K):
        _compare_scan(x, dtype)


@pytest.mark.parametrize("dtype,N", [("f32", 1), ("f32", 3), ("f32", 4), ("bf16", 2), ("bf16", 6), ("f32", 8),
                                     ("bf16", 10), ("bf16", 32), ("f32", 64), ("bf16", 64), ("bf16", 15),
                                     ("bf16", 1)])
@pytest.mark.parametrize("K", [1, 4])
def test_other_state_sizes(dtype, N, K):
    rng = np.random.default_rng(N * 7 + K)
    x = I.random_scan_inputs(rng, 2, 401, 72, N, dtype=dtype)
    say(f"dstate {N} {dtype} K={K}")
    npl = 4
    G = 1
    while npl * G < N:
        G *= 2
    with Variant(npl, G, K):
        _compare_scan(x, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [dict(softplus=False), dict(with_D=False), dict(with_bias=False),
                                   dict(with_z=False), dict(final=False),
                                   dict(with_D=False, with_bias=False, with_z=False)])
def test_optional_inputs(dtype, flags):
    rng = np.random.default_rng(21)
    x = I.random_scan_inputs(rng, 2, 300, 96, 16, dtype=dtype)
    if flags.get("softplus") is False:
        # raw delta + bias is used directly as the step: keep it positive
        x["delta"] = I.round_to_bf16(np.abs(x["delta"]) * 0.1) if dtype == "bf16" else np.abs(x["delta"]) * 0.1
        x["delta_bias"] = rng.uniform(0.0, 0.05, size=x["delta_bias"].shape).astype(np.float32)
    say(f"optional inputs {flags} {dtype}")
    y, fs = gpu_scan(x, dtype, **flags)
    kw = {k: v for k, v in flags.items() if k != "final"}
    yo, fo = oracle_scan(x, **kw)
    assert rel_err(y, yo) <= TOL[dtype]
    if flags.get("final", True):
        assert rel_err(fs, fo) <= TOL[dtype]
    else:
        assert fs is None


def test_long_chunked_fp32_reduced():
    """The long audio-style workload at 1/16 length: many chunks, slow fade, full compare."""
    w = I.WORKLOADS["long_audio_fp32"].scaled(L=1 << 16)
    x = I.make_inputs(w, 0)
    say(f"long reduced {w}")
    _compare_scan(x, "f32", with_z=False)


# ------------------------------------------------------------------ invariants
def test_determinism_bitwise():
    rng = np.random.default_rng(31)
    x = I.random_scan_inputs(rng, 2, 900, 192, 16, dtype="bf16")
    say("determinism")
    with Variant(2, 8, 3):
        y1, f1 = gpu_scan(x, "bf16")
        y2, f2 = gpu_scan(x, "bf16")
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


def test_causality_bitwise():
    rng = np.random.default_rng(32)
    x = I.random_scan_inputs(rng, 1, 640, 128, 16, dtype="bf16")
    t0 = 300
    say("causality")
    with Variant(2, 8, 1):
        y0, _ = gpu_scan(x, "bf16")
        for key in ("u", "delta", "z", "B", "C"):
            x2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
            x2[key][:, t0:] = I.round_to_bf16(x2[key][:, t0:] + 1.0)
            y1, _ = gpu_scan(x2, "bf16")
            assert np.array_equal(y1[:, :t0], y0[:, :t0]), key
            assert not np.array_equal(y1[:, t0], y0[:, t0]), key


# ------------------------------------------------------------------ chained chunks (one launch)
@pytest.mark.parametrize("npl,G,K", [(2, 8, 2), (2, 8, 3), (2, 8, 5), (4, 4, 3), (1, 16, 2)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chained_chunks_forced(npl, G, K, dtype):
    """Some tiles cut into K chunks spliced into the other tiles' workgroups, each chunk starting from the
    final state of the chunk before it (one launch)."""
    rng = np.random.default_rng(40 + 10 * K + npl)
    x = I.random_scan_inputs(rng, 2, 1000, 64 * 7 - 8, 16, dtype=dtype)
    say(f"chained npl={npl} G={G} K={K} {dtype}")
    with Variant(npl, G, K), Chained(True):
        _compare_scan(x, dtype)


@pytest.mark.parametrize("K,chained,dtype", [(1, False, "bf16"), (1, False, "f32"), (3, True, "bf16"),
                                             (3, True, "f32"), (3, False, "f32")])
def test_block_length_does_not_change_results(K, chained, dtype):
    """16- and 32-token blocks change only where the barriers fall, not the arithmetic: outputs are bitwise
    equal (whole tiles, chained chunks, and the readout pass of the chunk-pair plan), and match the oracle."""
    rng = np.random.default_rng(50 + K + (10 if chained else 0))
    x = I.random_scan_inputs(rng, 2, 1000, 64 * 7 - 8, 16, dtype=dtype)
    say(f"block length 16/32 K={K} chained={chained} {dtype}")
    outs = []
    for tb in (16, 32):
        with Variant(2, 8, K), Chained(chained), BlockLen(tb):
            outs.append(gpu_scan(x, dtype))
    (y16, f16), (y32, f32_) = outs
    assert np.array_equal(y16, y32) and np.array_equal(f16, f32_)
    yo, fo = oracle_scan(x)
    assert rel_err(y32, yo) <= TOL[dtype] and rel_err(f32_, fo) <= TOL[dtype]


def test_chained_plan_all_channels():
    """272 tiles for 256 CUs: 256 run whole, the 16 left over are cut into chunks spliced into them
    (the planner's own choice).  Every output against the oracle."""
    rng = np.random.default_rng(41)
    batch, L, dim = 1, 1024, 64 * 272
    x = I.random_scan_inputs(rng, batch, L, dim, 16, dtype="bf16")
    say(f"chained plan batch={batch} L={L} dim={dim}")
    y, fs = gpu_scan(x, "bf16")
    yo, fo = oracle_scan(x, nthreads=oracle_threads())
    ey, ef = rel_err(y, yo), rel_err(fs, fo)
    print(f"[parity] chained plan, all {dim} channels: y err {ey:.3e}  final-state err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= 1e-5, (ey, ef)


@pytest.mark.parametrize("tiles", [257, 384, 385])
def test_planner_boundaries(tiles):
    """At the edges of the chained plan: one tile left over (cut into the most chunks), half as many tiles
    again as CUs (two chunks each), and one tile more (every tile whole, two rounds).  Every output against the
    oracle."""
    rng = np.random.default_rng(43 + tiles)
    batch, L, dim = 1, 333, 64 * tiles
    x = I.random_scan_inputs(rng, batch, L, dim, 16, dtype="bf16")
    say(f"planner boundary tiles={tiles} L={L}")
    y, fs = gpu_scan(x, "bf16")
    yo, fo = oracle_scan(x, nthreads=oracle_threads())
    ey, ef = rel_err(y, yo), rel_err(fs, fo)
    print(f"[parity] planner boundary {tiles} tiles: y err {ey:.3e}  final-state err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= 1e-5, (ey, ef)


def test_chained_deterministic_and_matches_other_plans():
    rng = np.random.default_rng(42)
    x = I.random_scan_inputs(rng, 1, 3000, 64 * 12, 16, dtype="f32")
    say("chained determinism")
    with Variant(2, 8, 4):
        with Chained(True):
            y1, f1 = gpu_scan(x, "f32")
            y2, f2 = gpu_scan(x, "f32")
        with Chained(False):
            y3, f3 = gpu_scan(x, "f32")
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)
    # A different cut of the same recurrence: equal up to rounding.  The chunk-pair plan carries a chunk's total
    # fade as one exponential of its summed steps, exp2(A log2e * sum of ~750 deltas); that sum's fp32 rounding and
    # the single exp put ~|A * sum delta| * 2^-24 (up to ~1e-5 here, |A| <= 2) into the fade of a carried state,
    # where the chained plan multiplies the per-token fades.  Both plans stay within 1e-4 of the oracle
    # (test_every_variant_and_chunking, test_chained_plan_*); between each other the bound is 1e-5.
    assert rel_err(y1, y3) <= 1e-5 and rel_err(f1, f3) <= 1e-5


def test_chunk_count_independence():
    rng = np.random.default_rng(33)
    x = I.random_scan_inputs(rng, 1, 4000, 64, 16, dtype="f32")
    say("chunk independence")
    outs = []
    for K in (1, 2, 5, 16):
        with Variant(2, 8, K):
            outs.append(gpu_scan(x, "f32"))
    for y, fs in outs[1:]:
        assert rel_err(y, outs[0][0]) <= 1e-5 and rel_err(fs, outs[0][1]) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_continues_scan(dtype):
    """scan(L) then one decode step equals scan(L + 1) (the state is the hand-over)."""
    rng = np.random.default_rng(34)
    x = I.random_scan_inputs(rng, 3, 257, 80, 16, dtype=dtype)
    L = 256
    part = {k: (v[:, :L] if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
    say(f"decode continues scan {dtype}")
    y_full, f_full = gpu_scan(x, dtype)
    _, f_part = gpu_scan(part, dtype)
    st = to_dev_f32(f_part)
    yd = ops.ssm_state_update(st, to_dev(x["u"][:, L], dtype), to_dev(x["delta"][:, L], dtype), to_dev_f32(x["A"]),
                              to_dev(x["B"][:, L], dtype), to_dev(x["C"][:, L], dtype), D=to_dev_f32(x["D"]),
                              z=to_dev(x["z"][:, L], dtype), delta_bias=to_dev_f32(x["delta_bias"]))
    torch.cuda.synchronize()
    assert rel_err(st.cpu().numpy(), f_full) <= 1e-5
    assert rel_err(yd.float().cpu().numpy(), y_full[:, L]) <= TOL[dtype]


@pytest.mark.parametrize("dtype,N,batch", [("bf16", 16, 5), ("f32", 16, 5), ("f32", 3, 5), ("bf16", 64, 5), ("f32", 1, 5),
                                           ("bf16", 15, 5), ("bf16", 16, 1), ("f32", 8, 2), ("f32", 16, 7),
                                           ("bf16", 128, 5), ("f32", 256, 3), ("f32", 130, 2), ("bf16", 100, 1),
                                           ("bf16", 20, 3), ("f32", 32, 4)])
def test_decode_small_against_oracle(dtype, N, batch):
    """Odd batch sizes leave the last two-row group of the vector kernel half empty; batch 1 runs one row per thread.
    N = 20 gives groups of eight lanes of which the last three hold no states."""
    rng = np.random.default_rng(35 + N + 100 * batch)
    dim = 77
    u = rng.standard_normal((batch, dim)).astype(np.float32)
    dr = rng.standard_normal((batch, dim)).astype(np.float32)
    z = rng.standard_normal((batch, dim)).astype(np.float32)
    B = rng.standard_normal((batch, N)).astype(np.float32)
    C = rng.standard_normal((batch, N)).astype(np.float32)
    if dtype == "bf16":
        u, dr, z, B, C = (I.round_to_bf16(a) for a in (u, dr, z, B, C))
    A = -rng.uniform(0.05, 3.0, size=(dim, N)).astype(np.float32)
    D = rng.standard_normal(dim).astype(np.float32)
    bias = rng.standard_normal(dim).astype(np.float32)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    say(f"decode small {dtype} N={N}")
    st = to_dev_f32(h0)
    y = ops.ssm_state_update(st, to_dev(u, dtype), to_dev(dr, dtype), to_dev_f32(A), to_dev(B, dtype),
                             to_dev(C, dtype), D=to_dev_f32(D), z=to_dev(z, dtype), delta_bias=to_dev_f32(bias))
    torch.cuda.synchronize()
    so, yo = R.state_update(h0, u, dr, A, B, C, D=D, z=z, delta_bias=bias)
    assert rel_err(st.cpu().numpy(), so) <= 1e-5
    assert rel_err(y.float().cpu().numpy(), yo) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_optional_inputs_off(dtype):
    """No D, z or bias, softplus off: the step is delta_raw itself, y = C . h."""
    rng = np.random.default_rng(37)
    batch, dim, N = 5, 130, 16
    u = rng.standard_normal((batch, dim)).astype(np.float32)
    dr = rng.uniform(0.01, 0.5, size=(batch, dim)).astype(np.float32)
    B = rng.standard_normal((batch, N)).astype(np.float32)
    C = rng.standard_normal((batch, N)).astype(np.float32)
    if dtype == "bf16":
        u, dr, B, C = (I.round_to_bf16(a) for a in (u, dr, B, C))
    A = -rng.uniform(0.05, 3.0, size=(dim, N)).astype(np.float32)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    say(f"decode optional inputs off {dtype}")
    st = to_dev_f32(h0)
    y = ops.ssm_state_update(st, to_dev(u, dtype), to_dev(dr, dtype), to_dev_f32(A), to_dev(B, dtype),
                             to_dev(C, dtype), softplus=False)
    torch.cuda.synchronize()
    so, yo = R.state_update(h0, u, dr, A, B, C, softplus=False)
    assert rel_err(st.cpu().numpy(), so) <= 1e-5
    assert rel_err(y.float().cpu().numpy(), yo) <= TOL[dtype]


def test_zero_input_gives_zero():
    rng = np.random.default_rng(36)
    x = I.random_scan_inputs(rng, 2, 100, 64, 16, dtype="f32")
    x["u"][:] = 0.0
    say("zero input")
    y, fs = gpu_scan(x, "f32")
    assert np.all(y == 0.0) and np.all(fs == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_extreme_steps(dtype):
    """Steps from ~1e-26 to ~60 (raw values spread over +-60): the decay underflows to 0 at the large end, so the
    state is just the last input term, and stays at 1 at the small end, so the state is carried unchanged ([P4]
    "The Selection Mechanism": a large step resets, a small one ignores the token)."""
    rng = np.random.default_rng(37)
    x = I.random_scan_inputs(rng, 2, 300, 136, 16, dtype=dtype)
    raw = np.asarray(x["delta"], np.float64) * 20.0
    x["delta"] = I.round_to_bf16(raw) if dtype == "bf16" else np.asarray(raw, np.float32).astype(np.float64)
    say(f"extreme steps {dtype}")
    y, fs = gpu_scan(x, dtype)
    yo, fo = oracle_scan(x)
    ey, ef = rel_err(y, yo), rel_err(fs, fo)
    print(f"[parity] extreme steps {dtype}: y {ey:.2e}  final {ef:.2e}", flush=True)
    assert np.all(np.isfinite(y)) and ey <= TOL[dtype] and ef <= TOL[dtype], (ey, ef)
