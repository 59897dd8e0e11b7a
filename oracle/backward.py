"""Gradients of the Mamba-3 SSM sequence mixer -- test infrastructure.

Only the tests may import this module.  It shares no code with the HIP
library.

``forward_rot`` is the mixer written out in the rotated (RoPE) frame of the
Mamba-3 review, section 3.2.2, Proposition 3.2.3, with the coefficients of
section 3.1.1, eq. (6), and the rank-R products of section 3.3: per (b, h),

    Phi_t  = Phi_{-1} + sum_{s<=t} theta_s             (per row pair)
    B~_t   = R(-Phi_t) B_t,   C~_t = R(-Phi_t) C_t
    h~_t   = alpha_t h~_{t-1} + beta_t B~_{t-1} x_{t-1}^T + gamma_t B~_t x_t^T
    y_t    = C~_t^T h~_t
    alpha_t = exp(dt_t A),  beta_t = (1 - lam_t) dt_t alpha_t,  gamma_t = lam_t dt_t

with the carried state (h~_{-1}, Phi_{-1}, B~_{-1}, x_{-1}) given in that
frame (zeros: a fresh sequence).  It is plain fp64 torch on the CPU, one token
at a time, and it is a different formulation from the complex true-frame
recurrence of ``m3_oracle.c``; the pins check that the two agree.

``grad`` differentiates it with torch autograd for the loss
L = sum(gy * y), plus, when given, the inner products of incoming gradients
with the final carried state (h~_T, Phi_T, B~_{T-1}, x_{T-1}): the gradients
of every input and of the initial carried state.  The pins check them
against central finite differences of ``m3_oracle.c``, and the final-state
terms against the chain rule over split calls.
"""
from __future__ import annotations

import numpy as np
import torch

NAMES = ("x", "dt", "A", "lam", "theta", "B", "C")
INIT = ("h0", "phi0", "prevB0", "prevx0")


def _rot_neg(V, phi):
    """R(-phi) on row pairs (2k, 2k+1) of the last axis; phi has N/2 entries
    on its last axis and broadcasts against V's leading axes."""
    c, s = torch.cos(phi), torch.sin(phi)
    u, v = V[..., 0::2], V[..., 1::2]
    out = torch.stack((c * u + s * v, -s * u + c * v), dim=-1)
    return out.flatten(-2)


def forward_rot(x, dt, A, lam, theta, B, C, h0=None, phi0=None, prevB0=None, prevx0=None, final=False):
    """The mixer in the rotated frame (fp64 torch tensors).

    Shapes: x [b,T,H,R,P], dt/lam [b,T,H], A [H], theta [b,T,H,K], B/C
    [b,T,H,R,N]; h0 [b,H,N,P], phi0 [b,H,K], prevB0 [b,H,R,N] (rotated),
    prevx0 [b,H,R,P].  Returns y [b,T,H,R,P] and the final h~ [b,H,N,P];
    with ``final=True`` also Phi_T (unwrapped), B~_{T-1} and x_{T-1}.
    """
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    z = x.new_zeros
    h = h0 if h0 is not None else z(b, H, N, P)
    Phi = phi0 if phi0 is not None else z(b, H, N // 2)
    Bprev = prevB0 if prevB0 is not None else z(b, H, R, N)
    xprev = prevx0 if prevx0 is not None else z(b, H, R, P)
    ys = []
    for t in range(T):
        Phi = Phi + theta[:, t]
        Bt = _rot_neg(B[:, t], Phi[:, :, None, :])
        Ct = _rot_neg(C[:, t], Phi[:, :, None, :])
        d, l = dt[:, t], lam[:, t]
        alpha = torch.exp(d * A)
        beta = (1.0 - l) * d * alpha
        gamma = l * d
        h = (alpha[..., None, None] * h
             + beta[..., None, None] * torch.einsum("bhrn,bhrp->bhnp", Bprev, xprev)
             + gamma[..., None, None] * torch.einsum("bhrn,bhrp->bhnp", Bt, x[:, t]))
        ys.append(torch.einsum("bhrn,bhnp->bhrp", Ct, h))
        Bprev, xprev = Bt, x[:, t]
    if final:
        return torch.stack(ys, dim=1), h, Phi, Bprev, xprev
    return torch.stack(ys, dim=1), h


def grad(inputs: dict, gy, init: dict | None = None, gfinal: dict | None = None):
    """Gradients of L = sum(gy * y) + <gfinal, final state> (fp64).

    ``inputs``: x, dt, A, lam, theta, B, C as numpy arrays; ``init``: any of
    h0, phi0, prevB0, prevx0 (rotated frame); ``gfinal``: any of h, phi,
    prev_B, prev_x, the incoming gradients of the final h~_T, Phi_T, B~_{T-1}
    and x_{T-1}.  Returns (y, dict of gradients keyed like the inputs, with
    g_h0, g_phi0, g_prevB0, g_prevx0 for the carried state; a missing carried
    state gets the gradient at zero).
    """
    t = {k: torch.tensor(np.asarray(inputs[k], dtype=np.float64), requires_grad=True) for k in NAMES}
    b, T, H, R, P = t["x"].shape
    N = t["B"].shape[-1]
    shapes = dict(h0=(b, H, N, P), phi0=(b, H, N // 2), prevB0=(b, H, R, N), prevx0=(b, H, R, P))
    init = init or {}
    s = {k: torch.tensor(np.asarray(init[k], dtype=np.float64) if k in init else np.zeros(shapes[k]),
                         requires_grad=True) for k in INIT}
    y, hT, phiT, bT, xT = forward_rot(*(t[k] for k in NAMES), **s, final=True)
    loss = (y * torch.tensor(np.asarray(gy, dtype=np.float64))).sum()
    for k, v in zip(("h", "phi", "prev_B", "prev_x"), (hT, phiT, bT, xT)):
        if gfinal and gfinal.get(k) is not None:
            loss = loss + (v * torch.tensor(np.asarray(gfinal[k], dtype=np.float64))).sum()
    loss.backward()
    out = {k: t[k].grad.numpy() for k in NAMES}
    out.update({"g_" + k: s[k].grad.numpy() for k in INIT})
    return y.detach().numpy(), out
