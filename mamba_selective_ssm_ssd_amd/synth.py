"""Seeded synthetic inputs for the Mamba-3 SSM sequence mixer.

This module holds no arithmetic of the method: it only draws inputs.  Both the
GPU path and the fp64 oracle are fed from it, so it must never compute a
recurrence, a rotation or a decay.

Distributions (per element unless stated), standing in for the 1.5B-scale
workloads of the Mamba-3 review's experiments (section 4; appendix D):
    x, B, C ~ N(0, 1)
    dt      = softplus(N(0, 1) - 1)
    lam     = sigmoid(N(0, 1))
    theta   ~ U(0, pi)                  per (b, t, h, pair)
    A       = -exp(U(0, ln 16))         per head, kept in fp32
and for the block prologue/epilogue (``block_inputs``):
    B/C weight = 1 + 0.25 N(0, 1),  B/C bias = 0.5 N(0, 1)   per (h, r, n), fp32
    z       ~ N(0, 1)                   shaped like x
Every tensor has its own stream: ``numpy.random.default_rng([seed, cfg, id])``
(with the decode step appended for per-step decode inputs).  bf16 values are
obtained from the fp32 draw by round-to-nearest-even; dt and lam are computed
in fp32 before rounding.

Two backends draw the same distributions: ``numpy`` on the host (used for
everything the oracle checks element by element) and ``torch`` on a device
(used only to fill large benchmark buffers quickly; its values are different
numbers from the same distributions).
"""
from __future__ import annotations

import math

import numpy as np

# Named workloads.  Sizes: batch, T tokens, H heads, P head dim, N state
# (even), R MIMO rank, chunk 64.
CONFIGS = {
    0: dict(name="tiny_siso_prefill_fp32", kind="prefill", batch=1, T=256, H=2,
            P=16, N=16, R=1, io="f32"),
    1: dict(name="siso_prefill_b4_T2048_H64_P64_N128", kind="prefill", batch=4,
            T=2048, H=64, P=64, N=128, R=1, io="bf16"),
    2: dict(name="mimo_prefill_b4_T2048_H64_P64_N64_R4", kind="prefill", batch=4,
            T=2048, H=64, P=64, N=64, R=4, io="bf16"),
    3: dict(name="long_mimo_prefill_b1_T65536_H64_P64_N64_R4", kind="prefill",
            batch=1, T=65536, H=64, P=64, N=64, R=4, io="bf16"),
    4: dict(name="mimo_decode_b256_H64_P64_N64_R4_x1000", kind="decode",
            batch=256, T=1000, H=64, P=64, N=64, R=4, io="bf16"),
}

TENSOR_IDS = dict(x=1, dt=2, A=3, lam=4, theta=5, B=6, C=7, h0=8, B_weight=9, B_bias=10,
                  C_weight=11, C_bias=12, z=13)


def to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_io(a, io: str) -> np.ndarray:
    """Values of ``a`` after storage in the I/O dtype, returned as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if io == "f32":
        return a
    if io == "bf16":
        return bf16_bits_to_f32(to_bf16_bits(a))
    raise ValueError(io)


def _rng(seed, cfg, name, step=None):
    key = [int(seed), int(cfg), TENSOR_IDS[name]]
    if step is not None:
        key.append(int(step))
    return np.random.default_rng(key)


def _softplus(v):
    return np.logaddexp(np.float32(0.0), v).astype(np.float32)


def _sigmoid(v):
    return (1.0 / (1.0 + np.exp(-v))).astype(np.float32)


def head_decay(H: int, seed: int = 0, cfg: int = 0) -> np.ndarray:
    """A = -exp(U(0, ln 16)) per head, fp32."""
    u = _rng(seed, cfg, "A").uniform(0.0, math.log(16.0), size=H)
    return (-np.exp(u)).astype(np.float32)


def prefill_inputs(batch, T, H, P, N, R, io="bf16", seed=0, cfg=0, step=None, G=None):
    """Draw one batch of mixer inputs with numpy.

    Returns a dict of fp32 arrays holding exactly the values the I/O dtype
    stores: x [b,T,H,R,P], dt [b,T,H], lam [b,T,H], theta [b,T,H,N/2],
    B [b,T,G,R,N], C [b,T,G,R,N] (G = H unless given: B/C head groups); and
    A [H] (always fp32).
    """
    if N % 2:
        raise ValueError("N must be even")
    G = H if G is None else G
    f32 = np.float32
    x = _rng(seed, cfg, "x", step).standard_normal((batch, T, H, R, P), dtype=f32)
    B = _rng(seed, cfg, "B", step).standard_normal((batch, T, G, R, N), dtype=f32)
    C = _rng(seed, cfg, "C", step).standard_normal((batch, T, G, R, N), dtype=f32)
    dt = _softplus(_rng(seed, cfg, "dt", step).standard_normal((batch, T, H), dtype=f32) - f32(1.0))
    lam = _sigmoid(_rng(seed, cfg, "lam", step).standard_normal((batch, T, H), dtype=f32))
    theta = _rng(seed, cfg, "theta", step).uniform(0.0, math.pi, size=(batch, T, H, N // 2)).astype(f32)
    out = dict(x=x, dt=dt, lam=lam, theta=theta, B=B, C=C)
    out = {k: round_io(v, io) for k, v in out.items()}
    out["A"] = head_decay(H, seed, cfg)
    return out


def block_inputs(batch, T, H, P, N, R, io="bf16", seed=0, cfg=0, step=None):
    """Draw the block prologue/epilogue parameters with numpy: B_weight,
    B_bias, C_weight, C_bias [H,R,N] fp32 (per layer, so no ``step``) and the
    gate input z [b,T,H,R,P] rounded to the I/O dtype (T=None drops the token
    axis, as for one decode step)."""
    f32 = np.float32
    out = {}
    for name, (mean, std) in (("B_weight", (1.0, 0.25)), ("B_bias", (0.0, 0.5)),
                              ("C_weight", (1.0, 0.25)), ("C_bias", (0.0, 0.5))):
        v = _rng(seed, cfg, name).standard_normal((H, R, N), dtype=f32)
        out[name] = (f32(mean) + f32(std) * v).astype(f32)
    zshape = (batch, H, R, P) if T is None else (batch, T, H, R, P)
    out["z"] = round_io(_rng(seed, cfg, "z", step).standard_normal(zshape, dtype=f32), io)
    return out


def initial_state(batch, H, N, P, seed=0, cfg=0, std=0.1) -> np.ndarray:
    """Carried state drawn N(0, std) (standard deviation ``std``), fp32."""
    return (_rng(seed, cfg, "h0").standard_normal((batch, H, N, P), dtype=np.float32)
            * np.float32(std)).astype(np.float32)


def config_inputs(cfg: int, seed: int = 0, **override):
    """numpy inputs of a named configuration (sizes may be overridden)."""
    c = dict(CONFIGS[cfg])
    c.update(override)
    return prefill_inputs(c["batch"], c["T"], c["H"], c["P"], c["N"], c["R"],
                          io=c["io"], seed=seed, cfg=cfg)


def torch_inputs(batch, T, H, P, N, R, io="bf16", seed=0, device="cuda", G=None):
    """Same distributions drawn on a device with torch (large benchmark buffers).

    Returns device tensors in the I/O dtype (A in fp32); B/C have G head
    groups (G = H unless given).
    """
    G = H if G is None else G
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    dtype = torch.float32 if io == "f32" else torch.bfloat16
    f32 = torch.float32

    def normal(shape):
        return torch.randn(shape, generator=g, device=device, dtype=f32)

    x = normal((batch, T, H, R, P)).to(dtype)
    B = normal((batch, T, G, R, N)).to(dtype)
    C = normal((batch, T, G, R, N)).to(dtype)
    dt = torch.nn.functional.softplus(normal((batch, T, H)) - 1.0).to(dtype)
    lam = torch.sigmoid(normal((batch, T, H))).to(dtype)
    theta = (torch.rand((batch, T, H, N // 2), generator=g, device=device, dtype=f32)
             * math.pi).to(dtype)
    A = torch.from_numpy(head_decay(H, seed, 0)).to(device)
    return dict(x=x, dt=dt, lam=lam, theta=theta, B=B, C=C, A=A)
