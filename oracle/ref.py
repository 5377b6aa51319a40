"""numpy front end of the fp64 CPU oracle (test infrastructure only).

Each function widens its inputs exactly to float64 (bf16 -> fp32 -> fp64 are
exact widenings), calls the C oracle in ``ssm_ref.c`` and returns float64
arrays.  Shapes follow the pages' notation:
u, delta, z: [batch, L, dim]; B, C: [batch, L, dstate]; A: [dim, dstate];
D, delta_bias: [dim]; state: [batch, dim, dstate].
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.ssm_ref_scan_fwd.restype = ctypes.c_int
        lib.ssm_ref_scan_fwd.argtypes = [_dp] * 8 + [ctypes.c_int, _dp, _dp] + [ctypes.c_long] * 4 + [ctypes.c_int]
        lib.ssm_ref_scan_fwd_ex.restype = ctypes.c_int
        lib.ssm_ref_scan_fwd_ex.argtypes = ([_dp] * 8 + [ctypes.c_int, _dp, ctypes.POINTER(ctypes.c_long), ctypes.c_long,
                                             _dp, _dp] + [ctypes.c_long] * 4 + [ctypes.c_int])
        lib.ssm_ref_scan_trap_fwd_ex.restype = ctypes.c_int
        lib.ssm_ref_scan_trap_fwd_ex.argtypes = lib.ssm_ref_scan_fwd_ex.argtypes
        lib.ssm_ref_state_update.restype = ctypes.c_int
        lib.ssm_ref_state_update.argtypes = [_dp] * 9 + [ctypes.c_int, _dp] + [ctypes.c_long] * 3
        lib.ssm_ref_scan_bwd.restype = ctypes.c_int
        lib.ssm_ref_scan_bwd.argtypes = ([_dp] * 8 + [ctypes.c_int] + [_dp] * 12 + [ctypes.c_long] * 4 +
                                         [ctypes.c_int])
        lib.ssm_ref_scan_trap_bwd.restype = ctypes.c_int
        lib.ssm_ref_scan_trap_bwd.argtypes = lib.ssm_ref_scan_bwd.argtypes
        lib.ssm_ref_pair_then.restype = None
        lib.ssm_ref_pair_then.argtypes = [ctypes.c_long] + [_dp] * 6
        lib.ssm_ref_softplus.restype = ctypes.c_double
        lib.ssm_ref_softplus.argtypes = [ctypes.c_double]
        lib.ssm_ref_silu.restype = ctypes.c_double
        lib.ssm_ref_silu.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(_dp)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, nthreads=1,
             return_final_state=True):
    """Selective scan from a zero state. Returns (y, final_state) in float64."""
    lib = _load()
    u, delta, A, B, C, D, z, bias = map(_f64, (u, delta, A, B, C, D, z, delta_bias))
    batch, L, dim = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    assert D is None or D.shape == (dim,)
    assert bias is None or bias.shape == (dim,)
    y = np.empty((batch, L, dim), dtype=np.float64)
    fs = np.empty((batch, dim, N), dtype=np.float64) if return_final_state else None
    rc = lib.ssm_ref_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(bias),
                              1 if softplus else 0, _ptr(y), _ptr(fs), batch, L, dim, N, int(nthreads))
    if rc != 0:
        raise ValueError("oracle scan rejected its arguments")
    return y, fs


def scan_fwd_ex(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, initial_state=None,
                cu_seqlens=None, nthreads=1):
    """Selective scan from given initial states and/or over packed sequences (see ssm_ref.h).

    initial_state: [rows, dim, dstate] (rows = batch, or the number of sequences), None for zero.
    cu_seqlens: None, or nseq+1 offsets into the L axis of batch row 0 (batch must be 1).
    Returns (y, final_state [rows, dim, dstate]) in float64."""
    return _scan_rows(_load().ssm_ref_scan_fwd_ex, u, delta, A, B, C, D, z, delta_bias, softplus, initial_state,
                      cu_seqlens, nthreads)


def scan_trap_fwd_ex(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, initial_state=None,
                     cu_seqlens=None, nthreads=1):
    """The Mamba-3 trapezoidal three-term scan (ssm_ref_scan_trap_fwd_ex), arguments as scan_fwd_ex."""
    return _scan_rows(_load().ssm_ref_scan_trap_fwd_ex, u, delta, A, B, C, D, z, delta_bias, softplus,
                      initial_state, cu_seqlens, nthreads)


def _scan_rows(fn, u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, cu_seqlens, nthreads):
    u, delta, A, B, C, D, z, bias, h0 = map(_f64, (u, delta, A, B, C, D, z, delta_bias, initial_state))
    batch, L, dim = u.shape
    N = A.shape[1]
    cu = None
    nseq = 0
    rows = batch
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64)).astype(np.dtype("long"))
        nseq = cu.size - 1
        rows = nseq
    assert h0 is None or h0.shape == (rows, dim, N)
    y = np.empty((batch, L, dim), dtype=np.float64)
    fs = np.empty((rows, dim, N), dtype=np.float64)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_long))
    rc = fn(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(bias),
            1 if softplus else 0, _ptr(h0), cu_p, nseq, _ptr(y), _ptr(fs), batch, L, dim, N, int(nthreads))
    if rc != 0:
        raise ValueError("oracle scan rejected its arguments")
    return y, fs


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True, dfinal_state=None,
             initial_state=None, nthreads=1, rule="euler"):
    """Gradients of sum(y*dy) + sum(final_state*dfinal_state) with respect to every input of scan_fwd_ex
    (rule "euler") or scan_trap_fwd_ex (rule "trap"), batch rows, no packed sequences, by the C oracle's adjoint
    recurrence (ssm_ref_scan_bwd, ssm_ref_scan_trap_bwd).

    Returns a dict of float64 arrays: du, ddelta, dA, dB, dC, dinitial_state (zero initial state when none is
    given), and dD, dz, ddelta_bias for the optional inputs that were given (None otherwise)."""
    lib = _load()
    u, delta, A, B, C, D, z, bias, h0, dy, dfs = map(_f64, (u, delta, A, B, C, D, z, delta_bias, initial_state,
                                                           dy, dfinal_state))
    batch, L, dim = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and dy.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    assert h0 is None or h0.shape == (batch, dim, N)
    assert dfs is None or dfs.shape == (batch, dim, N)
    out = {"du": np.empty(u.shape), "ddelta": np.empty(u.shape), "dA": np.empty((dim, N)),
           "dB": np.empty(B.shape), "dC": np.empty(C.shape), "dinitial_state": np.empty((batch, dim, N)),
           "dD": None if D is None else np.empty(dim), "dz": None if z is None else np.empty(u.shape),
           "ddelta_bias": None if bias is None else np.empty(dim)}
    fn = {"euler": lib.ssm_ref_scan_bwd, "trap": lib.ssm_ref_scan_trap_bwd}[rule]
    rc = fn(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(bias), 1 if softplus else 0,
            _ptr(h0), _ptr(dy), _ptr(dfs), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dinitial_state"]),
            batch, L, dim, N, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle backward failed ({rc})")
    return out


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True):
    """One decode step. Returns (new_state, y) in float64; the input state is not modified."""
    lib = _load()
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    u, delta, A, B, C, D, z, bias = map(_f64, (u, delta, A, B, C, D, z, delta_bias))
    batch, dim = u.shape
    N = A.shape[1]
    assert st.shape == (batch, dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    y = np.empty((batch, dim), dtype=np.float64)
    rc = lib.ssm_ref_state_update(_ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(bias), 1 if softplus else 0, _ptr(y), batch, dim, N)
    if rc != 0:
        raise ValueError("oracle state update rejected its arguments")
    return st, y


def pair_then(a1, b1, a2, b2):
    """Elementwise fade-and-add composition '(a1,b1) then (a2,b2)'."""
    lib = _load()
    a1, b1, a2, b2 = map(_f64, (a1, b1, a2, b2))
    shape = a1.shape
    a1, b1, a2, b2 = (np.ascontiguousarray(np.broadcast_to(x, shape)).ravel() for x in (a1, b1, a2, b2))
    ao = np.empty(a1.size, dtype=np.float64)
    bo = np.empty(a1.size, dtype=np.float64)
    lib.ssm_ref_pair_then(a1.size, _ptr(a1), _ptr(b1), _ptr(a2), _ptr(b2), _ptr(ao), _ptr(bo))
    return ao.reshape(shape), bo.reshape(shape)


def softplus(x):
    return _load().ssm_ref_softplus(float(x))


def silu(z):
    return _load().ssm_ref_silu(float(z))
