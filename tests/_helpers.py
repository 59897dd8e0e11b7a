"""Shared test helpers: run the HIP path and the oracle on the same inputs and
compare them with the error metric of the parity bar.

Error metric (per output tensor): for every (batch, head) slice
    err = max|gpu - ref| / max|ref|
and the reported error is the maximum over slices.  Bars: 1e-4 for fp32 I/O,
2e-2 for bf16 I/O with fp32 state.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def slice_err(g, r, head_axes):
    """max over (b, h) slices of max|g - r| / max|r|.  head_axes: the axes that
    index (batch, head) in g/r (e.g. (0, 2) for [b,T,H,R,P])."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    other = tuple(i for i in range(r.ndim) if i not in head_axes)
    num = np.max(np.abs(g - r), axis=other)
    den = np.max(np.abs(r), axis=other)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def torch_io(io):
    import torch
    return torch.float32 if io == "f32" else torch.bfloat16


def to_dev(d, io, device="cuda"):
    """numpy inputs (fp32 values already rounded to the I/O dtype) -> device tensors."""
    import torch
    dt = torch_io(io)
    out = {}
    for k, v in d.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device=device, dtype=torch.float32 if k == "A" else dt).contiguous()
    return out


def gpu_state(state):
    """State of torch tensors -> dict of fp64 numpy arrays."""
    return dict(h=state.h.double().cpu().numpy(), phi=state.phi.double().cpu().numpy(),
                prev_B=state.prev_B.double().cpu().numpy(),
                prev_x=state.prev_x.float().cpu().numpy().astype(np.float64))


def run_gpu_prefill(d, io, init=None, want_final=True, chunk=64):
    """d: numpy inputs.  init: mixer.State or None.  Returns (y fp64, State)."""
    from mamba_selective_ssm_ssd_amd import mixer
    t = to_dev(d, io)
    y, st = mixer.prefill(t["x"], t["dt"], t["A"], t["lam"], t["theta"], t["B"], t["C"],
                          state=init, want_final=want_final, chunk=chunk)
    return y.double().cpu().numpy(), st


def oracle_init_from_rot(h_rot, phi, prevB_rot, prevx):
    """Carried state in the rotated frame -> oracle (state's own frame) inputs."""
    return dict(h0=oracle.state_to_true(h_rot, phi), prevB0=oracle.prevB_to_true(prevB_rot, phi),
                prevx0=prevx)


def run_oracle(d, init_rot=None, nthreads=0):
    """Oracle on numpy inputs d; init_rot = dict(h, phi, prev_B, prev_x) in the
    rotated frame (or None).  Returns (y, h_true_final, Phi_final fp64)."""
    kw = {}
    phi0 = None
    if init_rot is not None:
        kw = oracle_init_from_rot(init_rot["h"], init_rot["phi"], init_rot["prev_B"], init_rot["prev_x"])
        phi0 = init_rot["phi"]
    y, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                          nthreads=nthreads, **kw)
    phiT = oracle.cumulative_angle(d["theta"], phi0)
    return y, hT, phiT


def check_final_state(st, d, hT_ref, phiT_ref, io, tol):
    """Compare a GPU final state with the oracle's, in the state's own frame."""
    g = gpu_state(st)
    h_true = oracle.state_to_true(g["h"], phiT_ref)
    e_h = slice_err(h_true, hT_ref, (0, 1))
    dphi = oracle.wrap_angle(g["phi"] - phiT_ref)
    e_phi = float(np.max(np.abs(dphi)))
    B_last = oracle.heads_from_groups(d["B"][:, -1], d["x"].shape[2], axis=1).astype(np.float64)  # [b,H,R,N]
    e_B = slice_err(oracle.prevB_to_true(g["prev_B"], phiT_ref), B_last, (0, 1))
    x_last = d["x"][:, -1].astype(np.float64)
    assert np.array_equal(g["prev_x"], x_last), "prev_x must be the last token's x, bit for bit"
    assert e_h <= tol, f"final state error {e_h:.3e} > {tol}"
    assert e_phi <= 1e-4, f"final angle error {e_phi:.3e}"
    assert e_B <= 1e-4, f"prev_B error {e_B:.3e}"
    return e_h, e_phi, e_B
