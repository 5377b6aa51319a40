"""fp64 CPU oracle for the Mamba-2 state-space-duality (SSD) layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the test-suite, the smoke
check and the benchmark's CPU baseline may call it; the product path never
does.

What it computes.  Mamba-2 restricts the state matrix of every head to one
number times the identity ("State Space Models and the Post-Transformer Era",
"Mamba-2 and Structured State Space Duality"; "Mamba is attention all you
really need, part 2", the Mamba-2 entry of the lineage), and the page shows
the resulting sequence map to be multiplication by a causal 1-semiseparable
matrix, the same object masked linear attention multiplies by ("The State That
Must Remember Everything", Part 4).  Reading (the pages give no shapes): a head
is a group of `headdim` channels sharing the step delta_t and the scalar A of
the head; B_t and C_t (dstate each) are shared by all heads, as in the
two-term scan.  Per batch row and head, with x_t the head's headdim inputs:

    H_t = exp(delta_t A) H_{t-1} + delta_t x_t B_t^T      (H: headdim x dstate, H_{-1} = 0 or given)
    y_t = H_t C_t + D x_t,  then times SiLU(z_t) when z is given

This oracle evaluates the other ordering of the same computation, the
quadratic "attention" form, literally:

    M[t, s] = (C_t . B_s) * exp(A * (cs_t - cs_s)) * delta_s   for s <= t, else 0,
    cs_t = delta_0 + ... + delta_t,
    y = M x + D x,   final state H_{L-1} = sum_s exp(A (cs_{L-1} - cs_s)) delta_s x_s B_s^T,

and from a given H_{-1} the same plus its decay: exp(A cs_t) H_{-1} C_t in y_t and
exp(A cs_{L-1}) H_{-1} in the final state (the state a previous call hands on,
"Mamba is attention all you really need, part 2", "The relay"),

with numpy matrix products.  delta_t = softplus(delta_raw + bias) with the
exact log-add-exp, or delta_raw + bias when softplus is off.  The tests pin it
to the recurrent oracle (ssm_ref.c) on head-broadcast inputs and to plain
causal linear attention at A = 0, delta = 1.

Groups.  The page's equivalence casts B_t as the keys and C_t as the queries
of masked linear attention, shared by the heads; letting groups of heads
share them, as grouped attention shares keys and queries, is the reading taken
for B, C of shape [batch, L, ngroups, dstate]: heads are split into ngroups
runs of heads / ngroups consecutive heads, and run g uses B[..., g, :] and
C[..., g, :].  One group is the shape [batch, L, dstate] above.
"""
import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def ssd_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, initial_state=None):
    """SSD layer in the masked-matrix form.

    x, z: [batch, L, heads, headdim]; delta: [batch, L, heads]; A, D, delta_bias: [heads];
    B, C: [batch, L, dstate], or [batch, L, ngroups, dstate] with heads a multiple of ngroups;
    initial_state: [batch, heads, headdim, dstate] or None (zero).
    Returns (y [batch, L, heads, headdim], final_state [batch, heads, headdim, dstate]) in float64."""
    x, delta, A, B, C, D, z, bias, h0 = map(_f64, (x, delta, A, B, C, D, z, delta_bias, initial_state))
    batch, L, H, P = x.shape
    if B.ndim == 3:
        B, C = B[:, :, None, :], C[:, :, None, :]
    ngroups, N = B.shape[2], B.shape[3]
    assert delta.shape == (batch, L, H) and A.shape == (H,) and H % ngroups == 0
    assert B.shape == (batch, L, ngroups, N) and C.shape == (batch, L, ngroups, N)
    per_group = H // ngroups
    raw = delta if bias is None else delta + bias
    dl = np.logaddexp(raw, 0.0) if softplus else raw                       # [batch, L, H]
    y = np.empty((batch, L, H, P))
    fs = np.empty((batch, H, P, N))
    causal = np.tril(np.ones((L, L), dtype=bool))
    for b in range(batch):
        for h in range(H):
            g = h // per_group
            Bg, Cg = B[b, :, g], C[b, :, g]                                 # [L, N] of the head's group
            G = Cg @ Bg.T                                                   # [t, s] = C_t . B_s
            cs = np.cumsum(dl[b, :, h])
            decay = np.exp(np.where(causal, A[h] * (cs[:, None] - cs[None, :]), -np.inf))
            M = G * decay * dl[b, None, :, h]                               # [t, s]
            y[b, :, h] = M @ x[b, :, h]
            if D is not None:
                y[b, :, h] += D[h] * x[b, :, h]
            w = np.exp(A[h] * (cs[-1] - cs)) * dl[b, :, h]                  # weight of token s in H_{L-1}
            fs[b, h] = (x[b, :, h] * w[:, None]).T @ Bg
            if h0 is not None:
                y[b, :, h] += np.exp(A[h] * cs)[:, None] * (Cg @ h0[b, h].T)     # [t, p]: e^{A cs_t} H_{-1} C_t
                fs[b, h] += np.exp(A[h] * cs[-1]) * h0[b, h]
    if z is not None:
        y = y * (z / (1.0 + np.exp(-z)))
    return y, fs
