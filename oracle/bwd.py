"""fp64 CPU oracle for the backward pass of the selective scan.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the test-suite and the
smoke check may call it; the product path never does.

The pages do not spell out a backward pass. They only say that the
intermediate states are recomputed rather than stored when training ([P1]
"Keeping the pad on the desk"; [P4] "The Selection Mechanism: Why Mamba
Works"; [P5] "The Hardware-Aware Way Out", rematerialization).  The
gradients themselves are fixed by the forward definition, so this oracle is
reverse-mode automatic differentiation (torch.autograd, CPU, float64) of a
plain transcription of the forward recurrence:

    x_t  = delta_raw_t + bias                  Delta_t = softplus(x_t) or x_t
    h_t  = exp(Delta_t * A) * h_{t-1} + Delta_t * u_t * B_t      (h_{-1} = 0)
    v_t  = sum_n C_t[n] h_t[n] + D * u_t
    y_t  = v_t * SiLU(z_t)   (or v_t without z)

with softplus(x) = log(1 + e^x) exact (log-add-exp, no threshold) and
SiLU(z) = z * sigmoid(z).  The scalar differentiated is
    sum(y * dy) + sum(final_state * dfinal_state),
so the result is the vector-Jacobian product for output gradients dy (and
dfinal_state, the gradient reaching the final state, if any).

The transcription is independent of the C oracle (ssm_ref.c); the tests pin
it to that oracle's forward and to central finite differences of it.

With rule="trap" the transcribed forward is Mamba-3's trapezoidal
three-term recurrence ("The State That Must Remember Everything", Part 7,
"Mamba-3 (2026)", item 1) with the coefficients as this library reads them
(alpha_t = exp(Delta_t A), beta_t = Delta_t/2 alpha_t, gamma_t = Delta_t/2,
and no previous input at the first token of a recurrence):

    h_t = alpha_t * h_{t-1} + beta_t * B_{t-1} u_{t-1} + gamma_t * B_t u_t

with the same readout, skip and gate.  The tests pin it to central finite
differences of the C oracle's trapezoidal forward.

Packed sequences (cu_seqlens, batch 1): sequence s is tokens cu[s] ..
cu[s+1]-1 of the row, run on its own from initial_state[s] (zero if none)
with its own final state, as the forward's packed scan defines it; the
scalar differentiated sums y*dy over the row and final_state[s] *
dfinal_state[s] over the sequences.
"""
import numpy as np
import torch


def _t(x):
    return None if x is None else torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64)


def forward_torch(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, initial_state=None):
    """The forward recurrence on float64 torch tensors from initial_state (None: zero); returns (y, final_state)."""
    batch, L, dim = u.shape
    N = A.shape[1]
    x = delta if delta_bias is None else delta + delta_bias
    dl = torch.logaddexp(x, torch.zeros_like(x)) if softplus else x
    h = torch.zeros((batch, dim, N), dtype=torch.float64) if initial_state is None else initial_state
    ys = []
    for t in range(L):
        a = torch.exp(dl[:, t, :, None] * A[None, :, :])            # [batch, dim, N]
        b = (dl[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]
        h = a * h + b
        v = (h * C[:, t, None, :]).sum(-1)                           # [batch, dim]
        if D is not None:
            v = v + D[None, :] * u[:, t, :]
        ys.append(v)
    y = torch.stack(ys, dim=1)
    if z is not None:
        y = y * (z * torch.sigmoid(z))
    return y, h


def forward_trap_torch(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, initial_state=None):
    """The trapezoidal three-term recurrence on float64 torch tensors; returns (y, final_state)."""
    batch, L, dim = u.shape
    N = A.shape[1]
    x = delta if delta_bias is None else delta + delta_bias
    dl = torch.logaddexp(x, torch.zeros_like(x)) if softplus else x
    h = torch.zeros((batch, dim, N), dtype=torch.float64) if initial_state is None else initial_state
    ys = []
    for t in range(L):
        step = dl[:, t, :, None]                                     # [batch, dim, 1]
        alpha = torch.exp(step * A[None, :, :])
        beta = 0.5 * step * alpha
        gamma = 0.5 * step
        cur = u[:, t, :, None] * B[:, t, None, :]                    # B_t u_t
        h = alpha * h + gamma * cur
        if t > 0:
            h = h + beta * (u[:, t - 1, :, None] * B[:, t - 1, None, :])
        v = (h * C[:, t, None, :]).sum(-1)
        if D is not None:
            v = v + D[None, :] * u[:, t, :]
        ys.append(v)
    y = torch.stack(ys, dim=1)
    if z is not None:
        y = y * (z * torch.sigmoid(z))
    return y, h


def forward_packed_torch(u, delta, A, B, C, D, z, delta_bias, softplus, initial_state, cu_seqlens,
                         forward=forward_torch):
    """`forward` over each packed sequence of batch row 0, from its own initial state (None: zero).
    Returns (y [1, L, dim], final_state [nseq, dim, N])."""
    nseq = len(cu_seqlens) - 1
    dim, N = A.shape
    ys, fss = [], []
    for s in range(nseq):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        sl = lambda t: None if t is None else t[:, a:b]  # noqa: E731
        h0 = None if initial_state is None else initial_state[s:s + 1]
        if b > a:
            y, fs = forward(sl(u), sl(delta), A, sl(B), sl(C), D=D, z=sl(z), delta_bias=delta_bias,
                            softplus=softplus, initial_state=h0)
            ys.append(y)
        else:
            fs = torch.zeros((1, dim, N), dtype=torch.float64) if h0 is None else h0
        fss.append(fs)
    return torch.cat(ys, dim=1), torch.cat(fss, dim=0)


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True, dfinal_state=None,
             initial_state=None, cu_seqlens=None, rule="euler"):
    """Gradients of sum(y*dy) + sum(final_state*dfinal_state) with respect to every input.

    rule: "euler" (the two-term recurrence) or "trap" (the trapezoidal three-term one).

    With cu_seqlens (batch 1) the row holds packed sequences: initial_state, dfinal_state and the returned
    dinitial_state are [nseq, dim, N].
    Returns a dict of float64 numpy arrays: du, ddelta, dA, dB, dC, and dD, dz,
    ddelta_bias, dinitial_state for the optional inputs that were given (None otherwise)."""
    names = ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "initial_state"]
    vals = [u, delta, A, B, C, D, z, delta_bias, initial_state]
    ts = {}
    for n, v in zip(names, vals):
        tv = _t(v)
        if tv is not None:
            tv.requires_grad_(True)
        ts[n] = tv
    fwd = {"euler": forward_torch, "trap": forward_trap_torch}[rule]
    if cu_seqlens is not None:
        y, fs = forward_packed_torch(ts["u"], ts["delta"], ts["A"], ts["B"], ts["C"], ts["D"], ts["z"],
                                     ts["delta_bias"], softplus, ts["initial_state"], list(cu_seqlens), forward=fwd)
    else:
        y, fs = fwd(ts["u"], ts["delta"], ts["A"], ts["B"], ts["C"], D=ts["D"], z=ts["z"],
                    delta_bias=ts["delta_bias"], softplus=softplus, initial_state=ts["initial_state"])
    obj = (y * _t(dy)).sum()
    if dfinal_state is not None:
        obj = obj + (fs * _t(dfinal_state)).sum()
    leaves = [ts[n] for n in names if ts[n] is not None]
    grads = torch.autograd.grad(obj, leaves, allow_unused=True)
    out = {}
    gi = iter(grads)
    for n in names:
        if ts[n] is None:
            out["d" + n] = None
        else:
            g = next(gi)
            out["d" + n] = np.zeros(np.shape(ts[n].detach().numpy())) if g is None else g.detach().numpy()
    return out
