"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/ssm_scan.h declares,
carry gfx950 code, and reject bad arguments before any HIP call.  Only
argument-rejecting paths are called here: none of them launches anything.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_33_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

F32, BF16 = ops.SSM_DTYPE_F32, ops.SSM_DTYPE_BF16
INVALID, UNSUPPORTED = ops.SSM_ERR_INVALID_ARG, ops.SSM_ERR_UNSUPPORTED


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(ops.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    L = ops.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_library_carries_gfx950_code():
    data = open(ops.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings():
    assert ops.ssm_status_string(0) == "SSM_OK"
    assert ops.ssm_status_string(1) == "SSM_ERR_INVALID_ARG"
    assert ops.ssm_status_string(2) == "SSM_ERR_UNSUPPORTED"
    assert ops.ssm_status_string(3) == "SSM_ERR_HIP"
    assert ops.ssm_status_string(4) == "SSM_ERR_HANDOFF_TIMEOUT"
    assert ops.ssm_status_string(77) == "SSM_ERR_UNKNOWN"


def test_workspace_status_host_paths():
    """No workspace: nothing chained ran, so OK without any HIP call; a workspace too small for the header or
    misaligned is rejected before any HIP call."""
    L = ops.lib()
    assert L.ssm_workspace_status(None, 0, None) == ops.SSM_OK
    assert L.ssm_workspace_status(0x100000, 0, None) == ops.SSM_OK
    assert L.ssm_workspace_status(0x100000, 8, None) == INVALID
    assert L.ssm_workspace_status(0x100004, 4096, None) == INVALID


def test_workspace_size():
    L = ops.lib()
    # B and C are always repacked into fp32 per-state-group records: at least
    # batch * L(rounded up to 32) * 2 * dstate floats, 256-byte granular
    ws = L.ssm_scan_workspace_size(64, 256, 8192, 16, BF16)
    assert ws >= 64 * 256 * 2 * 16 * 4 and ws % 256 == 0
    # few channels, long sequence: the tile is cut into chunks, which adds
    # chunk pairs and carried-in states on top of the packed B/C (bf16); fp32
    # storage packs nothing, the scan reads B and C directly
    ws_long = L.ssm_scan_workspace_size(1, 1 << 20, 64, 16, BF16)
    assert ws_long > (1 << 20) * 2 * 16 * 4 and ws_long % 256 == 0
    ws_long32 = L.ssm_scan_workspace_size(1, 1 << 20, 64, 16, F32)
    assert ws_long32 == ws_long - ((((1 << 20) + 32) * 2 * 16 * 4 + 255) // 256 * 256)
    # rejected shapes report 0
    assert L.ssm_scan_workspace_size(0, 10, 10, 16, F32) == 0
    assert L.ssm_scan_workspace_size(1, 10, 10, 65, F32) == 0
    assert L.ssm_scan_workspace_size(1, 10, 10, 15, BF16) > 0       # odd dstate is fine with bf16
    assert L.ssm_scan_workspace_size(1, 10, 9_000_000, 16, BF16) == 0  # a token row over 16 MiB
    assert L.ssm_scan_workspace_size(1, 10, 10, 16, 7) == 0


def _scan(lib_, **kw):
    """Call ssm_scan_fwd with fake (never dereferenced) pointers; only rejection paths are used."""
    args = dict(u=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, z=None, bias=None, sp=1,
                y=0x6000, fs=None, batch=1, L=8, dim=8, N=16, dt=F32, ws=None, wsb=0, stream=None)
    args.update(kw)
    a = args
    return lib_.ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["y"],
                          a["fs"], a["batch"], a["L"], a["dim"], a["N"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(u=None), INVALID), (dict(delta=None), INVALID), (dict(A=None), INVALID), (dict(B=None), INVALID),
    (dict(C=None), INVALID), (dict(y=None), INVALID),
    (dict(batch=0), INVALID), (dict(L=0), INVALID), (dict(dim=-1), INVALID), (dict(N=0), INVALID),
    (dict(dt=5), INVALID),
    (dict(u=0x1001), INVALID), (dict(B=0x4002), INVALID), (dict(fs=0x7002), INVALID),
    (dict(dt=BF16, u=0x1001), INVALID),
    (dict(N=65), UNSUPPORTED), (dict(batch=70000), UNSUPPORTED),
    (dict(dim=9_000_000, dt=BF16), UNSUPPORTED),  # a token row over 16 MiB
    # missing / too small workspace
    (dict(batch=1, L=8, dim=8, N=16), INVALID),
    (dict(batch=1, L=1 << 20, dim=64, N=16), INVALID),
    (dict(batch=1, L=1 << 20, dim=64, N=16, ws=0x100000, wsb=1024), INVALID),
])
def test_scan_rejects_bad_arguments_without_launching(kw, expect):
    assert _scan(ops.lib(), **kw) == expect


def test_scan_rejects_misaligned_workspace():
    lib_ = ops.lib()
    need = lib_.ssm_scan_workspace_size(1, 1 << 20, 64, 16, F32)
    assert _scan(lib_, batch=1, L=1 << 20, dim=64, N=16, ws=0x100010, wsb=need) == INVALID


def _upd(lib_, **kw):
    a = dict(state=0x1000, u=0x2000, delta=0x3000, A=0x4000, B=0x5000, C=0x6000, D=None, z=None, bias=None, sp=1,
             y=0x7000, batch=2, dim=8, N=16, dt=F32, stream=None)
    a.update(kw)
    return lib_.ssm_state_update(a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                              a["sp"], a["y"], a["batch"], a["dim"], a["N"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(state=None), INVALID), (dict(u=None), INVALID), (dict(B=None), INVALID), (dict(y=None), INVALID),
    (dict(batch=0), INVALID), (dict(dim=0), INVALID), (dict(N=-3), INVALID), (dict(dt=9), INVALID),
    (dict(state=0x1002), INVALID), (dict(dt=BF16, z=0x8001), INVALID),
    (dict(N=257), UNSUPPORTED),
])
def test_state_update_rejects_bad_arguments_without_launching(kw, expect):
    assert _upd(ops.lib(), **kw) == expect


def _ex(lib_, entry="ssm_scan_fwd_ex", **kw):
    """Call ssm_scan_fwd_ex (or ssm_scan_trap_fwd) with fake (never dereferenced) pointers; only rejection paths
    are used."""
    a = dict(u=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, z=None, bias=None, sp=1, h0=None,
             cu=None, nseq=0, y=0x6000, fs=None, batch=1, L=8, dim=8, N=16, dt=F32, ws=None, wsb=0, stream=None)
    a.update(kw)
    return getattr(lib_, entry)(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"],
                                a["h0"], a["cu"], a["nseq"], a["y"], a["fs"], a["batch"], a["L"], a["dim"], a["N"],
                                a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(u=None), INVALID), (dict(h0=0x7002), INVALID),
    (dict(cu=0x8004, nseq=2), INVALID),                 # offsets must be 8-byte aligned
    (dict(cu=0x8000, nseq=0), INVALID), (dict(cu=0x8000, nseq=2, batch=2), INVALID),
    (dict(cu=0x8000, nseq=2, L=1 << 22, dim=1024), UNSUPPORTED),  # a sequence is never cut
    (dict(N=65), UNSUPPORTED),
    (dict(cu=0x8000, nseq=2), INVALID),                 # no workspace
])
@pytest.mark.parametrize("entry", ["ssm_scan_fwd_ex", "ssm_scan_trap_fwd"])
def test_scan_ex_rejects_bad_arguments_without_launching(kw, expect, entry):
    assert _ex(ops.lib(), entry, **kw) == expect


def test_trap_workspace_size():
    """The trapezoidal rule needs the plain workspace plus C_t . B_t of every token (fp32)."""
    L = ops.lib()
    for args in ((2, 1000, 136, 16, 0, BF16), (1, 1000, 136, 16, 7, F32), (4, 4096, 5120, 16, 0, BF16)):
        plain = L.ssm_scan_fwd_ex_workspace_size(*args)
        trap = L.ssm_scan_trap_fwd_workspace_size(*args)
        batch, Lq = args[0], args[1]
        assert plain > 0 and trap >= plain + batch * Lq * 4 and trap % 256 == 0
    assert L.ssm_scan_trap_fwd_workspace_size(2, 1000, 136, 16, 7, BF16) == 0     # packed needs batch 1
    assert L.ssm_scan_trap_fwd_workspace_size(1, 100, 64, 65, 0, F32) == 0        # dstate > 64


def test_scan_ex_workspace_size():
    L = ops.lib()
    assert L.ssm_scan_fwd_ex_workspace_size(2, 1000, 136, 16, 0, BF16) == L.ssm_scan_workspace_size(2, 1000, 136, 16, BF16)
    ws = L.ssm_scan_fwd_ex_workspace_size(1, 1000, 136, 16, 7, BF16)
    assert ws >= 1000 * 2 * 16 * 4 and ws % 256 == 0
    assert L.ssm_scan_fwd_ex_workspace_size(2, 1000, 136, 16, 7, BF16) == 0       # packed needs batch 1
    assert L.ssm_scan_fwd_ex_workspace_size(1, 1 << 22, 1024, 16, 3, F32) == 0    # rows past 2^31 bytes


def test_bwd_workspace_size():
    L = ops.lib()
    # at least the state entering every 16-token block of every 64-channel tile
    ws = L.ssm_scan_bwd_workspace_size(2, 1000, 136, 16, 0, BF16)
    assert ws >= 2 * 3 * (1024 // 16) * 64 * 16 * 4 and ws % 256 == 0
    assert L.ssm_scan_bwd_workspace_size(2, 1000, 136, 32, 0, F32) > ws
    assert L.ssm_scan_bwd_workspace_size(2, 1000, 136, 33, 0, F32) > 0    # wide states: two halves
    assert L.ssm_scan_bwd_workspace_size(2, 1000, 136, 65, 0, F32) == 0   # backward: dstate <= 64
    assert L.ssm_scan_bwd_workspace_size(0, 10, 10, 16, 0, F32) == 0
    assert L.ssm_scan_bwd_workspace_size(1, 10, 10, 16, 0, 7) == 0
    assert L.ssm_scan_bwd_workspace_size(1, 1 << 24, 1024, 16, 0, F32) == 0  # rows past 2^31 bytes
    # a tile's dB/dC partial row past 2^31 bytes: 40M tokens x 16 states x 4 bytes
    assert L.ssm_scan_bwd_workspace_size(1, 40_000_000, 1, 16, 0, F32) == 0
    assert L.ssm_scan_bwd_workspace_size(1, 20_000_000, 1, 16, 0, F32) > 0
    # wide states keep fp32 partial rows of L * dim: allowed for 16 states, not for 64, at bf16 rows of 1.6 GB
    assert L.ssm_scan_bwd_workspace_size(1, 200_000, 4096, 16, 0, BF16) > 0
    assert L.ssm_scan_bwd_workspace_size(1, 200_000, 4096, 64, 0, BF16) == 0
    # packed sequences: batch 1 only; partial rows per sequence and a few more checkpoints per sequence
    assert L.ssm_scan_bwd_workspace_size(2, 1000, 136, 16, 3, F32) == 0
    assert L.ssm_scan_bwd_workspace_size(1, 1000, 136, 16, 7, F32) > L.ssm_scan_bwd_workspace_size(1, 1000, 136, 16,
                                                                                                   0, F32)


def test_trap_bwd_workspace_size():
    L = ops.lib()
    e = L.ssm_scan_bwd_workspace_size(2, 1000, 136, 16, 0, BF16)
    t = L.ssm_scan_trap_bwd_workspace_size(2, 1000, 136, 16, 0, BF16)
    assert t > 0 and t % 256 == 0 and t <= e   # no chained plan, so no carried adjoints
    assert L.ssm_scan_trap_bwd_workspace_size(1, 1000, 136, 64, 3, F32) > 0   # wide states, packed sequences
    assert L.ssm_scan_trap_bwd_workspace_size(2, 1000, 136, 65, 0, F32) == 0
    assert L.ssm_scan_trap_bwd_workspace_size(2, 1000, 136, 16, 3, F32) == 0   # packed needs batch 1


def _bwd(lib_, **kw):
    """Call ssm_scan_bwd with fake (never dereferenced) pointers; only rejection paths are used."""
    a = dict(u=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, z=None, bias=None, sp=1, dy=0x6000,
             dfs=None, h0=None, cu=None, nseq=0, du=0x7000, dd=0x8000, dA=0x9000, dB=0xa000, dC=0xb000, dD=None,
             dz=None, dbias=None, dh0=None, batch=1, L=8, dim=8, N=16, dt=F32, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib_.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["dy"],
                             a["dfs"], a["h0"], a["cu"], a["nseq"], a["du"], a["dd"], a["dA"], a["dB"], a["dC"],
                             a["dD"], a["dz"],
                             a["dbias"], a["dh0"], a["batch"], a["L"], a["dim"], a["N"], a["dt"], a["ws"], a["wsb"],
                             a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(u=None), INVALID), (dict(dy=None), INVALID), (dict(du=None), INVALID), (dict(dd=None), INVALID),
    (dict(dA=None), INVALID), (dict(dB=None), INVALID), (dict(dC=None), INVALID),
    (dict(batch=0), INVALID), (dict(L=0), INVALID), (dict(N=0), INVALID), (dict(dt=3), INVALID),
    (dict(dy=0x6001), INVALID), (dict(dt=BF16, dB=0xa001), INVALID), (dict(dfs=0xc002), INVALID),
    (dict(h0=0xc002), INVALID), (dict(dh0=0xd001), INVALID),
    (dict(N=65), UNSUPPORTED), (dict(batch=70000), UNSUPPORTED),
    (dict(L=1 << 24, dim=1024), UNSUPPORTED),
    (dict(L=40_000_000, dim=1), UNSUPPORTED),           # the dB/dC partial row of a tile past 2^31 bytes
    (dict(L=200_000, dim=4096, N=64, dt=BF16), UNSUPPORTED),  # wide states' fp32 partial rows past 2^31 bytes
    (dict(), INVALID),                                  # no workspace
    (dict(ws=0x100000, wsb=256), INVALID),              # too small
    (dict(cu=0x8000, nseq=2, batch=2), INVALID),        # packed sequences need batch 1
    (dict(cu=0x8004, nseq=2), INVALID),                 # offsets 8-byte aligned
    (dict(cu=0x8000, nseq=0), INVALID),
])
def test_bwd_rejects_bad_arguments_without_launching(kw, expect):
    assert _bwd(ops.lib(), **kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(u=None), INVALID), (dict(dy=None), INVALID), (dict(N=65), UNSUPPORTED), (dict(), INVALID),
    (dict(ws=0x100000, wsb=256), INVALID), (dict(cu=0x8000, nseq=2, batch=2), INVALID),
])
def test_trap_bwd_rejects_bad_arguments_without_launching(kw, expect, monkeypatch):
    lib_ = ops.lib()
    monkeypatch.setattr(lib_, "ssm_scan_bwd", lib_.ssm_scan_trap_bwd)
    assert _bwd(lib_, **kw) == expect


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        ops.lib()


def _ssd(lib_, **kw):
    """Call ssm_ssd_fwd with fake (never dereferenced) pointers; only rejection paths are used."""
    a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, z=None, bias=None, sp=1, h0=None,
             y=0x6000, fs=None, batch=1, L=8, H=2, P=64, G=1, N=64, dt=BF16, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib_.ssm_ssd_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["h0"],
                            a["y"], a["fs"], a["batch"], a["L"], a["H"], a["P"], a["G"], a["N"], a["dt"], a["ws"],
                            a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), INVALID), (dict(B=None), INVALID), (dict(y=None), INVALID), (dict(L=0), INVALID),
    (dict(H=-1), INVALID), (dict(dt=7), INVALID),
    (dict(x=0x1008), INVALID), (dict(C=0x5004), INVALID), (dict(delta=0x2001), INVALID), (dict(fs=0x7002), INVALID),
    (dict(h0=0x8002), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(P=32), UNSUPPORTED), (dict(N=16), UNSUPPORTED), (dict(N=96), UNSUPPORTED),
    (dict(L=1 << 20, H=40), UNSUPPORTED),   # token rows past 2^31 bytes
    (dict(G=0), INVALID), (dict(H=6, G=4), INVALID),   # ngroups must divide heads
    (dict(L=1 << 22, H=2, G=2, N=128), UNSUPPORTED),    # B/C rows past 2^31 bytes
    (dict(batch=4, H=80), INVALID),           # 320 units: the chained plan needs its workspace
])
def test_ssd_rejects_bad_arguments_without_launching(kw, expect):
    assert _ssd(ops.lib(), **kw) == expect


def test_ssd_workspace_size():
    L = ops.lib()
    assert L.ssm_ssd_fwd_workspace_size(2, 1000, 3, 64, 64, BF16) == 0          # fewer units than CUs
    ws = L.ssm_ssd_fwd_workspace_size(4, 4096, 80, 64, 128, BF16)             # 320 units: 64 left over, 4 segments
    assert ws >= 64 * 4 * 64 * 128 * 4 and ws % 256 == 0
    assert L.ssm_ssd_fwd_workspace_size(4, 4096, 80, 64, 128, F32) == 0        # rejected


def test_binding_argument_counts_match_the_header():
    """Every entry point's ctypes signature has as many arguments as its declaration in include/ssm_scan.h (the
    binding and the header cannot drift apart unnoticed)."""
    import os
    import re

    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ssm_scan.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    L = ops.lib()
    for name in ops.EXPORTED:
        m = re.search(r"\b" + name + r"\s*\(([^;]*?)\)\s*;", hdr, flags=re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(getattr(L, name).argtypes) == len(params), name


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """ssm_scan_fwd_noalloc on a shape whose workspace exceeds its 32 MiB static array: a clear error before any
    HIP call (fake pointers, never dereferenced).  The shape is bf16, whose B/C records are always packed (128 MB
    here); the guard keeps the call from ever being made with a shape that would fit."""
    lib = ops.lib()
    shape = (1, 1 << 20, 64, 16)
    assert lib.ssm_scan_workspace_size(*shape, BF16) > (32 << 20)
    a = (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None, None, None, 1, 0x6000, None)
    assert lib.ssm_scan_fwd_noalloc(*a, *shape, BF16, None) == ops.SSM_ERR_SCRATCH_TOO_SMALL
    assert lib.ssm_scan_fwd_noalloc(*a, 0, 10, 64, 16, F32, None) == INVALID
    assert lib.ssm_scan_fwd_noalloc(*a, 1, 10, 64, 65, F32, None) == UNSUPPORTED


def test_structured_host_paths():
    """ssm_scan_fwd_structured: workspace sizes and rejections before any HIP call."""
    L = ops.lib()
    ws = L.ssm_scan_fwd_structured_workspace_size(4, 4096, 5120, 16, BF16)
    assert ws > 0 and ws % 256 == 0
    # fp32 storage reads B and C directly: no records
    ws32 = L.ssm_scan_fwd_structured_workspace_size(4, 4096, 5120, 16, F32)
    assert 0 < ws32 < ws
    assert L.ssm_scan_fwd_structured_workspace_size(1, 100, 64, 17, F32) == 0   # a lane holds at most 16 states
    assert L.ssm_scan_fwd_structured_workspace_size(0, 100, 64, 16, F32) == 0
    p = ctypes.c_void_p(0x100000)
    args = lambda dstate, ws, nbytes: (p, p, p, p, p, None, None, None, 1, None, p, None, 1, 100, 64, dstate, F32,
                                       ws, nbytes, None)
    assert L.ssm_scan_fwd_structured(*args(17, p, 1 << 20)) == UNSUPPORTED
    assert L.ssm_scan_fwd_structured(*args(16, None, 0)) == INVALID            # no workspace
    assert L.ssm_scan_fwd_structured(*args(16, ctypes.c_void_p(0x100010), 1 << 20)) == INVALID  # misaligned
    assert L.ssm_scan_fwd_structured(None, p, p, p, p, None, None, None, 1, None, p, None, 1, 100, 64, 16, F32, p,
                                     1 << 20, None) == INVALID


def test_structured_base_detection_host():
    import torch

    a0 = torch.tensor([-1.0, -0.3, -7.5])
    A = a0[:, None] * torch.arange(1, 17, dtype=torch.float32)[None, :]
    assert torch.equal(ops.structured_A_base(A), a0)
    A[2, 15] = A[2, 15] * (1 + 1e-6)
    assert ops.structured_A_base(A) is None
