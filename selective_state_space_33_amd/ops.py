"""ctypes binding of libssmscan.so (the gfx950 selective-scan C ABI).

The functions carry the names of the C entry points and only marshal
arguments: tensor checks, default outputs/workspace allocated with torch on
the inputs' device, and the raw device pointers plus the HIP stream handed
to the library.  Every step of the computation runs in the HIP kernels;
there is no fallback.  If the library is missing, ``lib()`` raises.

Streams: the kernels run on ``stream`` (default: the device's current
stream).  Outputs and workspaces allocated here are allocated while that
stream is current, so torch's caching allocator ties their memory to it and
does not hand it to other streams' work while the kernels may still use it.
``check_status=True`` reads the workspace's status word back after the call
(ssm_workspace_status, which synchronises the stream) and raises if a chained
hand-off wait ran out.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_OK, SSM_ERR_INVALID_ARG, SSM_ERR_UNSUPPORTED, SSM_ERR_HIP, SSM_ERR_HANDOFF_TIMEOUT = 0, 1, 2, 3, 4
SSM_ERR_SCRATCH_TOO_SMALL = 5
SSM_DTYPE_F32, SSM_DTYPE_BF16 = 0, 1

# Every symbol include/ssm_scan.h declares.
EXPORTED = ("ssm_scan_workspace_size", "ssm_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_ex_workspace_size", "ssm_scan_fwd_ex",
            "ssm_scan_fwd_structured_workspace_size", "ssm_scan_fwd_structured",
            "ssm_scan_trap_fwd_workspace_size", "ssm_scan_trap_fwd", "ssm_ssd_fwd_workspace_size", "ssm_ssd_fwd",
            "ssm_state_update",
            "ssm_scan_bwd_workspace_size", "ssm_scan_bwd", "ssm_scan_trap_bwd_workspace_size", "ssm_scan_trap_bwd",
            "ssm_workspace_status", "ssm_status_string")

_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class SSMError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where} failed: {ssm_status_string(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Open libssmscan.so (built in-tree by __graft_entry__.build()); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_scan_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_workspace_size.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
        L.ssm_scan_fwd.restype = ctypes.c_int
        L.ssm_scan_fwd.argtypes = ([_vp] * 8 + [ctypes.c_int, _vp, _vp] + [_i64] * 4 +
                                   [ctypes.c_int, _vp, ctypes.c_size_t, _vp])
        L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_scan_fwd_noalloc.argtypes = [_vp] * 8 + [ctypes.c_int, _vp, _vp] + [_i64] * 4 + [ctypes.c_int, _vp]
        L.ssm_state_update.restype = ctypes.c_int
        L.ssm_state_update.argtypes = [_vp] * 9 + [ctypes.c_int, _vp] + [_i64] * 3 + [ctypes.c_int, _vp]
        L.ssm_scan_fwd_ex_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_fwd_ex_workspace_size.argtypes = [_i64] * 5 + [ctypes.c_int]
        L.ssm_scan_fwd_ex.restype = ctypes.c_int
        L.ssm_scan_fwd_ex.argtypes = ([_vp] * 8 + [ctypes.c_int, _vp, _vp, _i64, _vp, _vp] + [_i64] * 4 +
                                      [ctypes.c_int, _vp, ctypes.c_size_t, _vp])
        L.ssm_scan_fwd_structured_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_fwd_structured_workspace_size.argtypes = [_i64] * 4 + [ctypes.c_int]
        L.ssm_scan_fwd_structured.restype = ctypes.c_int
        L.ssm_scan_fwd_structured.argtypes = ([_vp] * 8 + [ctypes.c_int, _vp, _vp, _vp] + [_i64] * 4 +
                                              [ctypes.c_int, _vp, ctypes.c_size_t, _vp])
        L.ssm_scan_trap_fwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_trap_fwd_workspace_size.argtypes = L.ssm_scan_fwd_ex_workspace_size.argtypes
        L.ssm_scan_trap_fwd.restype = ctypes.c_int
        L.ssm_scan_trap_fwd.argtypes = L.ssm_scan_fwd_ex.argtypes
        L.ssm_ssd_fwd.restype = ctypes.c_int
        L.ssm_ssd_fwd.argtypes = ([_vp] * 8 + [ctypes.c_int, _vp, _vp, _vp] + [_i64] * 6 +
                                  [ctypes.c_int, _vp, ctypes.c_size_t, _vp])
        L.ssm_ssd_fwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_ssd_fwd_workspace_size.argtypes = [_i64] * 5 + [ctypes.c_int]
        L.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_bwd_workspace_size.argtypes = [_i64] * 5 + [ctypes.c_int]
        for name in ("ssm_scan_bwd", "ssm_scan_trap_bwd"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = ([_vp] * 8 + [ctypes.c_int] + [_vp] * 4 + [_i64] + [_vp] * 9 + [_i64] * 4 +
                                         [ctypes.c_int, _vp, ctypes.c_size_t, _vp])
        L.ssm_scan_trap_bwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_scan_trap_bwd_workspace_size.argtypes = [_i64] * 5 + [ctypes.c_int]
        L.ssm_workspace_status.restype = ctypes.c_int
        L.ssm_workspace_status.argtypes = [_vp, ctypes.c_size_t, _vp]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def ssm_status_string(code: int) -> str:
    return lib().ssm_status_string(int(code)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSM_DTYPE_F32
    if t == torch.bfloat16:
        return SSM_DTYPE_BF16
    raise TypeError(f"unsupported storage dtype {t}; use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _resolve(device, stream):
    """The torch stream the kernels run on: `stream`, or the device's current stream."""
    return torch.cuda.current_stream(device) if stream is None else stream


def _ws_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def ssm_workspace_status(workspace, stream=None) -> int:
    """Status code the last call that used `workspace` left in it (synchronises `stream`):
    SSM_OK, or SSM_ERR_HANDOFF_TIMEOUT if a chained hand-off wait ran out."""
    dev = workspace.device if workspace is not None else torch.device("cuda", torch.cuda.current_device())
    s = _resolve(dev, stream)
    return int(lib().ssm_workspace_status(_ptr(workspace), _ws_bytes(workspace), s.cuda_stream))


def _check_status(workspace, stream, where):
    rc = ssm_workspace_status(workspace, stream)
    if rc != SSM_OK:
        raise SSMError(rc, where)


def ssm_scan_workspace_size(batch: int, L: int, dim: int, dstate: int, dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_workspace_size(batch, L, dim, dstate, _dtype_code(dtype)))


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                 y=None, final_state=None, workspace=None, return_final_state: bool = True, stream=None,
                 check_status: bool = False):
    """Selective scan from a zero state on the GPU.

    u, delta, z: [batch, L, dim]; B, C: [batch, L, dstate] (float32 or bfloat16,
    all the same); A: [dim, dstate], D, delta_bias: [dim] (float32).
    Returns (y, final_state); final_state is None if not requested.
    """
    batch, L, dim = u.shape
    dstate = A.shape[1]
    dev, dt = u.device, u.dtype
    code = _dtype_code(dt)
    for name, t, shp in (("u", u, (batch, L, dim)), ("delta", delta, (batch, L, dim)), ("z", z, (batch, L, dim)),
                         ("B", B, (batch, L, dstate)), ("C", C, (batch, L, dstate))):
        _check(t, name, dt, shp, dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    s = _resolve(dev, stream)
    with torch.cuda.stream(s):
        if y is None:
            y = torch.empty((batch, L, dim), dtype=dt, device=dev)
        if final_state is None and return_final_state:
            final_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
        need = ssm_scan_workspace_size(batch, L, dim, dstate, dt)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", dt, (batch, L, dim), dev)
    _check(final_state, "final_state", torch.float32, (batch, dim, dstate), dev)
    rc = lib().ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                            1 if softplus else 0, _ptr(y), _ptr(final_state), batch, L, dim, dstate, code,
                            _ptr(workspace), _ws_bytes(workspace), s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_scan_fwd")
    if check_status:
        _check_status(workspace, s, "ssm_scan_fwd")
    return y, final_state


def structured_A_base(A) -> Optional[torch.Tensor]:
    """A0 [dim] if A [dim, dstate] has the structured form A[d, n] = (n + 1) * A0[d] exactly (fp32), else None.

    A one-time check of a weight (it synchronises to read the answer), for callers choosing
    ssm_scan_fwd_structured; the library itself never inspects A."""
    n = torch.arange(1, A.shape[1] + 1, dtype=torch.float32, device=A.device)
    a0 = A[:, 0].contiguous()
    ok = bool(torch.equal(A, a0[:, None] * n[None, :]))
    return a0 if ok else None


def ssm_scan_fwd_structured_workspace_size(batch: int, L: int, dim: int, dstate: int, dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_fwd_structured_workspace_size(batch, L, dim, dstate, _dtype_code(dtype)))


def ssm_scan_fwd_structured(u, delta, A0, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                            initial_state=None, y=None, final_state=None, workspace=None,
                            return_final_state: bool = True, stream=None):
    """The scan for A[d, n] = (n + 1) * A0[d], given A0 [dim] (float32): one exp per (token, channel).

    u, delta, z: [batch, L, dim]; B, C: [batch, L, dstate] with dstate <= 16; initial_state:
    [batch, dim, dstate] float32 or None.  Returns (y, final_state)."""
    batch, L, dim = u.shape
    dstate = B.shape[2]
    dev, dt = u.device, u.dtype
    code = _dtype_code(dt)
    for name, t, shp in (("u", u, (batch, L, dim)), ("delta", delta, (batch, L, dim)), ("z", z, (batch, L, dim)),
                         ("B", B, (batch, L, dstate)), ("C", C, (batch, L, dstate))):
        _check(t, name, dt, shp, dev)
    _check(A0, "A0", torch.float32, (dim,), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _check(initial_state, "initial_state", torch.float32, (batch, dim, dstate), dev)
    s = _resolve(dev, stream)
    with torch.cuda.stream(s):
        if y is None:
            y = torch.empty((batch, L, dim), dtype=dt, device=dev)
        if final_state is None and return_final_state:
            final_state = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
        need = ssm_scan_fwd_structured_workspace_size(batch, L, dim, dstate, dt)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", dt, (batch, L, dim), dev)
    _check(final_state, "final_state", torch.float32, (batch, dim, dstate), dev)
    rc = lib().ssm_scan_fwd_structured(_ptr(u), _ptr(delta), _ptr(A0), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                       _ptr(delta_bias), 1 if softplus else 0, _ptr(initial_state), _ptr(y),
                                       _ptr(final_state), batch, L, dim, dstate, code, _ptr(workspace),
                                       _ws_bytes(workspace), s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_scan_fwd_structured")
    return y, final_state


def ssm_scan_fwd_ex(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                    initial_state=None, cu_seqlens=None, y=None, final_state=None, workspace=None, stream=None,
                    check_status: bool = False):
    """ssm_scan_fwd from given initial states and/or over packed sequences.

    initial_state: [rows, dim, dstate] float32 (rows = batch, or the number of sequences).
    cu_seqlens: int64 device tensor of nseq + 1 offsets into the L axis of batch row 0 (batch must be 1).
    Returns (y, final_state [rows, dim, dstate])."""
    return _fwd_rows("ssm_scan_fwd_ex", u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, cu_seqlens,
                     y, final_state, workspace, stream, check_status)


def ssm_scan_trap_fwd_workspace_size(batch: int, L: int, dim: int, dstate: int, nseq: int,
                                     dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_trap_fwd_workspace_size(batch, L, dim, dstate, nseq, _dtype_code(dtype)))


def ssm_scan_trap_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                      initial_state=None, cu_seqlens=None, y=None, final_state=None, workspace=None, stream=None,
                      check_status: bool = False):
    """The Mamba-3 trapezoidal three-term scan; arguments and results as ssm_scan_fwd_ex."""
    return _fwd_rows("ssm_scan_trap_fwd", u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, cu_seqlens,
                     y, final_state, workspace, stream, check_status)


def _fwd_rows(entry, u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, cu_seqlens, y, final_state,
              workspace, stream, check_status=False):
    batch, L, dim = u.shape
    dstate = A.shape[1]
    dev, dt = u.device, u.dtype
    code = _dtype_code(dt)
    nseq = 0
    rows = batch
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int64 tensor on the device of u")
        nseq = cu_seqlens.numel() - 1
        rows = nseq
        _check(cu_seqlens, "cu_seqlens", torch.int64, (nseq + 1,), dev)
    for name, t, shp in (("u", u, (batch, L, dim)), ("delta", delta, (batch, L, dim)), ("z", z, (batch, L, dim)),
                         ("B", B, (batch, L, dstate)), ("C", C, (batch, L, dstate))):
        _check(t, name, dt, shp, dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _check(initial_state, "initial_state", torch.float32, (rows, dim, dstate), dev)
    s = _resolve(dev, stream)
    with torch.cuda.stream(s):
        if y is None:
            y = torch.empty((batch, L, dim), dtype=dt, device=dev)
        if final_state is None:
            final_state = torch.empty((rows, dim, dstate), dtype=torch.float32, device=dev)
        need = int(getattr(lib(), entry + "_workspace_size")(batch, L, dim, dstate, nseq, code))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", dt, (batch, L, dim), dev)
    _check(final_state, "final_state", torch.float32, (rows, dim, dstate), dev)
    rc = getattr(lib(), entry)(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                               1 if softplus else 0, _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(y),
                               _ptr(final_state), batch, L, dim, dstate, code, _ptr(workspace),
                               _ws_bytes(workspace), s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, entry)
    if check_status:
        _check_status(workspace, s, entry)
    return y, final_state


def ssm_ssd_fwd_workspace_size(batch: int, L: int, heads: int, headdim: int, dstate: int,
                               dtype: torch.dtype) -> int:
    return int(lib().ssm_ssd_fwd_workspace_size(batch, L, heads, headdim, dstate, _dtype_code(dtype)))


def ssm_ssd_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True, initial_state=None,
                y=None, final_state=None, return_final_state: bool = True, workspace=None, stream=None,
                check_status: bool = False):
    """The Mamba-2 SSD layer on the GPU.

    x, z: [batch, L, heads, headdim]; delta: [batch, L, heads]; B, C: [batch, L, dstate] or
    [batch, L, ngroups, dstate] (bfloat16; heads a multiple of ngroups); A, D, delta_bias: [heads] (float32);
    initial_state: [batch, heads, headdim, dstate] (float32) or None.
    Returns (y, final_state [batch, heads, headdim, dstate] or None)."""
    batch, L, heads, headdim = x.shape
    ngroups = 1 if B.dim() == 3 else B.shape[2]
    dstate = B.shape[-1]
    bc_shape = (batch, L, dstate) if B.dim() == 3 else (batch, L, ngroups, dstate)
    dev, dt = x.device, x.dtype
    code = _dtype_code(dt)
    for name, t, shp in (("x", x, (batch, L, heads, headdim)), ("z", z, (batch, L, heads, headdim)),
                         ("delta", delta, (batch, L, heads)), ("B", B, bc_shape), ("C", C, bc_shape)):
        _check(t, name, dt, shp, dev)
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias)):
        _check(t, name, torch.float32, (heads,), dev)
    _check(initial_state, "initial_state", torch.float32, (batch, heads, headdim, dstate), dev)
    s = _resolve(dev, stream)
    with torch.cuda.stream(s):
        if y is None:
            y = torch.empty_like(x)
        if final_state is None and return_final_state:
            final_state = torch.empty((batch, heads, headdim, dstate), dtype=torch.float32, device=dev)
        need = ssm_ssd_fwd_workspace_size(batch, L, heads, headdim, dstate, dt)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", dt, (batch, L, heads, headdim), dev)
    _check(final_state, "final_state", torch.float32, (batch, heads, headdim, dstate), dev)
    rc = lib().ssm_ssd_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                           1 if softplus else 0, _ptr(initial_state), _ptr(y), _ptr(final_state), batch, L, heads,
                           headdim, ngroups, dstate, code, _ptr(workspace), _ws_bytes(workspace), s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_ssd_fwd")
    if check_status:
        _check_status(workspace, s, "ssm_ssd_fwd")
    return y, final_state


def ssm_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
                     y=None, stream=None):
    """One decode step on the GPU; `state` [batch, dim, dstate] (float32) is updated in place.

    u, delta, z: [batch, dim]; B, C: [batch, dstate]. Returns y [batch, dim].
    """
    batch, dim = u.shape
    dstate = A.shape[1]
    dev, dt = u.device, u.dtype
    code = _dtype_code(dt)
    _check(state, "state", torch.float32, (batch, dim, dstate), dev)
    for name, t, shp in (("u", u, (batch, dim)), ("delta", delta, (batch, dim)), ("z", z, (batch, dim)),
                         ("B", B, (batch, dstate)), ("C", C, (batch, dstate))):
        _check(t, name, dt, shp, dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    s = _resolve(dev, stream)
    if y is None:
        with torch.cuda.stream(s):
            y = torch.empty((batch, dim), dtype=dt, device=dev)
    _check(y, "y", dt, (batch, dim), dev)
    rc = lib().ssm_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(delta_bias), 1 if softplus else 0, _ptr(y), batch, dim, dstate, code,
                                s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_state_update")
    return y


def ssm_scan_fwd_ex_workspace_size(batch: int, L: int, dim: int, dstate: int, nseq: int, dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_fwd_ex_workspace_size(batch, L, dim, dstate, nseq, _dtype_code(dtype)))


def ssm_scan_bwd_workspace_size(batch: int, L: int, dim: int, dstate: int, dtype: torch.dtype, nseq: int = 0,
                                trapezoid: bool = False) -> int:
    fn = lib().ssm_scan_trap_bwd_workspace_size if trapezoid else lib().ssm_scan_bwd_workspace_size
    return int(fn(batch, L, dim, dstate, nseq, _dtype_code(dtype)))


def ssm_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus: bool = True,
                 dfinal_state=None, initial_state=None, want_dinitial_state: bool = False, cu_seqlens=None,
                 workspace=None, stream=None, check_status: bool = False, trapezoid: bool = False):
    """Backward of ssm_scan_fwd (or ssm_scan_fwd_ex) on the GPU: gradients of sum(y*dy) +
    sum(final_state*dfinal_state).  trapezoid=True: the backward of ssm_scan_trap_fwd (ssm_scan_trap_bwd).

    Same inputs as ssm_scan_fwd plus dy [batch, L, dim] (storage dtype) and dfinal_state
    [rows, dim, dstate] (float32, optional); cu_seqlens: int64 device offsets of packed sequences of batch
    row 0 (rows = nseq; otherwise rows = batch).  Returns a dict with du, ddelta, dB, dC (storage
    dtype), dA (float32), and dD, dz, ddelta_bias for the optional inputs given (None otherwise);
    dinitial_state [rows, dim, dstate] when an initial state is given or want_dinitial_state.
    """
    batch, L, dim = u.shape
    dstate = A.shape[1]
    dev, dt = u.device, u.dtype
    code = _dtype_code(dt)
    nseq, rows = 0, batch
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int64 tensor on the device of u")
        nseq = rows = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", torch.int64, (nseq + 1,), dev)
    for name, t, shp in (("u", u, (batch, L, dim)), ("delta", delta, (batch, L, dim)), ("z", z, (batch, L, dim)),
                         ("dy", dy, (batch, L, dim)), ("B", B, (batch, L, dstate)), ("C", C, (batch, L, dstate))):
        _check(t, name, dt, shp, dev)
    _check(A, "A", torch.float32, (dim, dstate), dev)
    _check(D, "D", torch.float32, (dim,), dev)
    _check(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _check(dfinal_state, "dfinal_state", torch.float32, (rows, dim, dstate), dev)
    _check(initial_state, "initial_state", torch.float32, (rows, dim, dstate), dev)
    s = _resolve(dev, stream)
    with torch.cuda.stream(s):
        g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(delta), dB=torch.empty_like(B),
                 dC=torch.empty_like(C), dA=torch.empty_like(A),
                 dD=None if D is None else torch.empty_like(D), dz=None if z is None else torch.empty_like(z),
                 ddelta_bias=None if delta_bias is None else torch.empty_like(delta_bias),
                 dinitial_state=(torch.empty((rows, dim, dstate), dtype=torch.float32, device=dev)
                                 if (initial_state is not None or want_dinitial_state) else None))
        need = ssm_scan_bwd_workspace_size(batch, L, dim, dstate, dt, nseq, trapezoid=trapezoid)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    name = "ssm_scan_trap_bwd" if trapezoid else "ssm_scan_bwd"
    rc = getattr(lib(), name)(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                            1 if softplus else 0, _ptr(dy), _ptr(dfinal_state), _ptr(initial_state),
                            _ptr(cu_seqlens), nseq, _ptr(g["du"]),
                            _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                            _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dinitial_state"]), batch, L, dim, dstate,
                            code, _ptr(workspace), _ws_bytes(workspace), s.cuda_stream)
    if rc != SSM_OK:
        raise SSMError(rc, name)
    if check_status:
        _check_status(workspace, s, name)
    return g
