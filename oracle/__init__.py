"""fp64 CPU oracle for the Mamba-3 SSM sequence mixer -- test infrastructure.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with the HIP library and never calls
it; the HIP library never imports it.

``run`` drives ``m3_oracle.c`` (the sequential fp64 recurrence with an explicit
complex diagonal state, see the header of that file for the equations and their
sources on the Mamba-3 review page, sections 3.1-3.3).  The helpers below it
only move states between the state's own frame and the rotated (RoPE) frame
in which the GPU library keeps its carried state:

    h_rot = R(-Phi) h_true,   Phi = Phi_{-1} + sum_{s<=t} theta_s   (per pair)

(Mamba-3 review, section 3.2.1, Proposition 3.2.2 and section 3.2.2,
Proposition 3.2.3: the RoPE form rotates B and C by the transpose of the
cumulative product of the per-token rotations.)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "libm3oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libm3oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.m3o_run.restype = ctypes.c_int
        lib.m3o_run.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                ctypes.c_int]
        lib.m3o_default_threads.restype = ctypes.c_int
        lib.m3o_default_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return int(_load().m3o_default_threads())


def heads_from_groups(V, H: int, axis: int = 2):
    """B or C shared by head groups -> one copy per head.

    V has G groups on ``axis`` (G divides H); head h reads group h // (H // G),
    i.e. consecutive heads share a group.  This is the shared B, C projection
    of the MIMO instantiation (Mamba-3 review, section 3.3) written out: with
    G = H it returns V unchanged.
    """
    V = np.asarray(V)
    G = V.shape[axis]
    if H % G:
        raise ValueError(f"{G} groups do not divide {H} heads")
    return V if G == H else np.repeat(V, H // G, axis=axis)


def run(x, dt, A, lam, theta, B, C, h0=None, prevB0=None, prevx0=None,
        nthreads: int = 0):
    """Run the fp64 recurrence.

    Shapes (any float dtype; converted to fp64): x [b,T,H,R,P], dt/lam [b,T,H],
    A [H], theta [b,T,H,N/2], B/C [b,T,H,R,N] or [b,T,G,R,N] (shared by head
    groups, see ``heads_from_groups``); optional carried state in the state's
    own frame: h0 [b,H,N,P], prevB0 [b,H,R,N], prevx0 [b,H,R,P].

    Returns (y [b,T,H,R,P], hT [b,H,N,P] true frame, threads used).
    """
    H = np.shape(x)[2]
    B, C = heads_from_groups(B, H), heads_from_groups(C, H)
    x, dt, A, lam, theta, B, C = map(_f64, (x, dt, A, lam, theta, B, C))
    h0, prevB0, prevx0 = map(_f64, (h0, prevB0, prevx0))
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    assert dt.shape == (b, T, H) and lam.shape == (b, T, H) and A.shape == (H,)
    assert theta.shape == (b, T, H, N // 2)
    assert B.shape == (b, T, H, R, N) and C.shape == (b, T, H, R, N)
    if h0 is not None:
        assert h0.shape == (b, H, N, P)
    if prevB0 is not None:
        assert prevB0.shape == (b, H, R, N)
    if prevx0 is not None:
        assert prevx0.shape == (b, H, R, P)
    y = np.zeros((b, T, H, R, P), dtype=np.float64)
    hT = np.zeros((b, H, N, P), dtype=np.float64)
    rc = _load().m3o_run(b, T, H, P, N, R, _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                         _ptr(theta), _ptr(B), _ptr(C), _ptr(h0), _ptr(prevB0),
                         _ptr(prevx0), _ptr(y), _ptr(hT), int(nthreads))
    if rc <= 0:
        raise RuntimeError(f"m3o_run failed with code {rc}")
    return y, hT, rc


# ---------------------------------------------------------------------------
# Frame helpers (fp64).  Row pair (2k, 2k+1) of the N axis is rotated by the
# angle of pair k; R(phi) = [[cos, -sin], [sin, cos]] (counter-clockwise, the
# real form of multiplying z = h[2k] + i h[2k+1] by exp(i phi)).
# ---------------------------------------------------------------------------

def cumulative_angle(theta, phi0=None):
    """Phi_{T-1} = Phi_{-1} + sum_t theta_t, fp64, unwrapped.  theta [b,T,H,K]."""
    tot = np.asarray(theta, dtype=np.float64).sum(axis=1)
    if phi0 is not None:
        tot = tot + np.asarray(phi0, dtype=np.float64)
    return tot


def rotate_pairs(v, phi, axis: int):
    """Apply R(phi_k) to row pairs (2k, 2k+1) along ``axis`` of ``v``.

    ``phi`` must broadcast against ``v`` with the pair axis in place of ``axis``
    (length N/2 instead of N).
    """
    v = np.asarray(v, dtype=np.float64)
    v = np.moveaxis(v, axis, -1)
    phi = np.moveaxis(np.asarray(phi, dtype=np.float64), axis, -1)
    even, odd = v[..., 0::2], v[..., 1::2]
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty_like(v)
    out[..., 0::2] = c * even - s * odd
    out[..., 1::2] = s * even + c * odd
    return np.moveaxis(out, -1, axis)


def state_to_true(h_rot, phi):
    """h_true = R(Phi) h_rot; h_rot [b,H,N,P], phi [b,H,N/2]."""
    return rotate_pairs(h_rot, np.asarray(phi)[..., None], axis=2)


def prevB_to_true(prevB_rot, phi):
    """B_true = R(Phi) B_rot; prevB [b,H,R,N], phi [b,H,N/2]."""
    return rotate_pairs(prevB_rot, np.asarray(phi)[:, :, None, :], axis=3)


def wrap_angle(phi):
    """Map angles to [-pi, pi) in fp64."""
    phi = np.asarray(phi, dtype=np.float64)
    return phi - 2.0 * np.pi * np.floor((phi + np.pi) / (2.0 * np.pi))


# ---------------------------------------------------------------------------
# Block prologue and epilogue around the mixer (fp64, plain numpy).
#
# Mamba-3 review, section 3.4 (Mamba-3 architecture; "BC/QK normalisation" and
# "B, C biases"): after the B and C projections each is RMS-normalised, then a
# learnable per-head, per-channel bias is added; the mixer output then passes
# the block's output gate.  The pages give no formulas; the readings taken:
#   - the RMS is over the N state channels of each (token, head, rank) row,
#     with eps inside the square root, followed by an optional per-(head, rank,
#     channel) weight (the usual RMS-norm scale) and the bias;
#   - the gate is y * silu(z) = y * z / (1 + exp(-z)), z shaped like y.
# ---------------------------------------------------------------------------

def bc_norm(V, weight=None, bias=None, eps=1e-6, norm=True):
    """Prologue on B or C: V [b,T,H,R,N] (or [b,H,R,N] for one decode step).

    Returns V / sqrt(mean_n V^2 + eps) * weight[h,r,n] + bias[h,r,n] (fp64);
    ``norm=False`` skips the division, ``None`` weight/bias mean 1 and 0.
    """
    V = np.asarray(V, dtype=np.float64)
    if norm:
        V = V / np.sqrt(np.mean(V * V, axis=-1, keepdims=True) + float(eps))
    if weight is not None:
        V = V * np.asarray(weight, dtype=np.float64)
    if bias is not None:
        V = V + np.asarray(bias, dtype=np.float64)
    return V


def gate(y, z):
    """Epilogue: y * silu(z) = y * z / (1 + exp(-z)) (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    return np.asarray(y, dtype=np.float64) * z / (1.0 + np.exp(-z))


def run_block(x, dt, A, lam, theta, B, C, block=None, h0=None, prevB0=None,
              prevx0=None, nthreads: int = 0):
    """``run`` with the block prologue applied to B and C and the gate to y.

    ``block``: dict with optional keys bc_norm (bool), eps, B_weight, B_bias,
    C_weight, C_bias ([H,R,N]) and z (shaped like y).  The carried previous B
    (prevB0) is taken as already prologued (it is the previous token's B).
    """
    block = block or {}
    H = np.shape(x)[2]
    B, C = heads_from_groups(B, H), heads_from_groups(C, H)
    nrm, eps = bool(block.get("bc_norm", False)), block.get("eps", 1e-6)
    Bp = bc_norm(B, block.get("B_weight"), block.get("B_bias"), eps, nrm)
    Cp = bc_norm(C, block.get("C_weight"), block.get("C_bias"), eps, nrm)
    y, hT, used = run(x, dt, A, lam, theta, Bp, Cp, h0, prevB0, prevx0, nthreads)
    if block.get("z") is not None:
        y = gate(y, block["z"])
    return y, hT, used
