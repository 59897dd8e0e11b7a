"""torch-facing wrapper of the C ABI: prefill, decode_step and the carried State.

torch is used only to hold device memory and to name the current stream;
every step of the mixer runs in the HIP kernels of libm3ssm.so.  Tensors must
be contiguous, on the current HIP device, in the layouts of include/m3_ssm.h:
    x [b,T,H,R,P], B/C [b,T,G,R,N] (G divides H; G = H: per head), dt/lam
    [b,T,H], theta [b,T,H,N/2] (I/O dtype: float32 or bfloat16), A [H] float32.
With a ``Block`` (and/or a gate input ``z`` shaped like y) the Mamba-3
block's B/C normalisation, B/C weight and bias and output gate run inside the
same kernels (include/m3_ssm_block.h).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import capi

_IO = {torch.float32: capi.M3_DTYPE_F32, torch.bfloat16: capi.M3_DTYPE_BF16}


@dataclass
class State:
    """Carried state in the rotated frame (see include/m3_ssm.h)."""
    h: torch.Tensor       # [b,H,N,P] float32 or bfloat16 (state_dtype)
    phi: torch.Tensor     # [b,H,N/2] float32
    prev_B: torch.Tensor  # [b,H,R,N] float32
    prev_x: torch.Tensor  # [b,H,R,P] I/O dtype

    @staticmethod
    def zeros(batch, H, N, P, R, io_dtype=torch.bfloat16, device="cuda",
              state_dtype=torch.float32) -> "State":
        f = dict(device=device, dtype=torch.float32)
        return State(torch.zeros(batch, H, N, P, device=device, dtype=state_dtype),
                     torch.zeros(batch, H, N // 2, **f),
                     torch.zeros(batch, H, R, N, **f),
                     torch.zeros(batch, H, R, P, device=device, dtype=io_dtype))

    def c(self) -> capi.m3_state_t:
        for t in (self.h, self.phi, self.prev_B, self.prev_x):
            if not t.is_contiguous():
                raise ValueError("state tensors must be contiguous")
        return capi.m3_state_t(self.h.data_ptr(), self.phi.data_ptr(),
                               self.prev_B.data_ptr(), self.prev_x.data_ptr())

    def clone(self) -> "State":
        return State(self.h.clone(), self.phi.clone(), self.prev_B.clone(), self.prev_x.clone())


@dataclass
class Block:
    """Per-layer parameters of the block prologue: RMS normalisation of the
    B and C rows over N (``bc_norm``, ``eps``), then per-head, per-channel
    weight and bias, each [H,R,N] float32 or None (1 / 0)."""
    bc_norm: bool = True
    eps: float = 1e-6
    B_weight: torch.Tensor | None = None
    B_bias: torch.Tensor | None = None
    C_weight: torch.Tensor | None = None
    C_bias: torch.Tensor | None = None


def _block_c(block: Block | None, z, io, H, R, N) -> capi.m3_block_t | None:
    if block is None and z is None:
        return None
    blk = block if block is not None else Block(bc_norm=False)
    c = capi.m3_block_t(int(bool(blk.bc_norm)), float(blk.eps))
    for name in ("B_weight", "B_bias", "C_weight", "C_bias"):
        t = getattr(blk, name)
        if t is not None:
            if tuple(t.shape) != (H, R, N):
                raise ValueError(f"{name} must be [H,R,N] = {(H, R, N)}, got {tuple(t.shape)}")
            setattr(c, name, _ptr(t, name, torch.float32))
    if z is not None:
        c.z = _ptr(z, "z", io)
    return c


def _ptr(t: torch.Tensor, name: str, dtype) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check_bc(B, C, lead, R, N):
    """B and C: lead + (G, R, N), the same shape (G checked by the library)."""
    if tuple(B.shape) != tuple(C.shape) or tuple(B.shape[:len(lead)]) != tuple(lead) \
            or tuple(B.shape[len(lead) + 1:]) != (R, N):
        raise ValueError(f"B/C must be {tuple(lead)} + (G, {R}, {N}), got {tuple(B.shape)}, {tuple(C.shape)}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_shape(batch, T, H, P, N, R, io_dtype, chunk=64, G=0,
               state_dtype=torch.float32) -> capi.m3_shape_t:
    """G: B/C head groups (0 or H: per head); state_dtype: storage of h~."""
    return capi.m3_shape_t(int(batch), int(T), int(H), int(P), int(N), int(R), int(chunk),
                           int(_IO[io_dtype]), int(G), int(_IO[state_dtype]))


def workspace_bytes(batch, T, H, P, N, R, io_dtype=torch.bfloat16, chunk=64) -> int:
    return capi.m3_ssm_prefill_workspace_bytes(make_shape(batch, T, H, P, N, R, io_dtype, chunk=chunk))


def prefill(x, dt, A, lam, theta, B, C, state: State | None = None, final: State | None = None,
            want_final: bool = True, y=None, workspace=None, block: Block | None = None, z=None,
            state_dtype=None, chunk: int = 64):
    """Chunked prefill.  Returns (y, final_state or None).

    ``chunk``: tokens per chunk, 64 (sub-chunks of 64/R tokens where a
    64-token chunk does not fit on chip) or 64/R (32 for R = 3) to take the
    small chunk always; the result is the same up to rounding.

    The carried state's h~ is float32 or bfloat16: the dtype of the given
    state(s), else ``state_dtype`` (default float32) for a new final state.

    ``block`` / ``z`` (shaped like x) add the block prologue and output gate.

    ``state`` is the carried state to start from (None: fresh sequence).
    The final state goes to ``final`` if given, else to ``state`` (in place)
    when a state was given, else to a new State -- unless want_final=False.
    """
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    io = x.dtype
    _check_bc(B, C, (b, T), R, N)
    given = [s.h.dtype for s in (state, final) if s is not None]
    sd = given[0] if given else (state_dtype or torch.float32)
    if any(d != sd for d in given) or (state_dtype is not None and state_dtype != sd):
        raise ValueError("initial and final states must share one state dtype")
    shape = make_shape(b, T, H, P, N, R, io, chunk=chunk, G=B.shape[2], state_dtype=sd)
    if y is None:
        y = torch.empty_like(x)
    if want_final and final is None:
        final = state if state is not None else State(
            torch.empty(b, H, N, P, device=x.device, dtype=sd),
            torch.empty(b, H, N // 2, device=x.device, dtype=torch.float32),
            torch.empty(b, H, R, N, device=x.device, dtype=torch.float32),
            torch.empty(b, H, R, P, device=x.device, dtype=io))
    if not want_final:
        final = None
    need = capi.m3_ssm_prefill_workspace_bytes(shape)
    if need == 0:
        raise capi.M3Error(capi.M3_ERR_UNSUPPORTED if N % 2 == 0 else capi.M3_ERR_INVALID_ARGUMENT,
                           "m3_ssm_prefill_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, device=x.device, dtype=torch.uint8)
    if z is not None and tuple(z.shape) != tuple(x.shape):
        raise ValueError("z must be shaped like x")
    args = [shape, _ptr(x, "x", io), _ptr(dt, "dt", io), _ptr(A, "A", torch.float32),
            _ptr(lam, "lam", io), _ptr(theta, "theta", io), _ptr(B, "B", io), _ptr(C, "C", io)]
    tail = [state.c() if state is not None else None, final.c() if final is not None else None,
            _ptr(y, "y", io), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream()]
    blk = _block_c(block, z, io, H, R, N)
    if blk is None:
        rc, fn = capi.m3_ssm_prefill(*args, *tail), "m3_ssm_prefill"
    else:
        rc, fn = capi.m3_ssm_prefill_block(*args, blk, *tail), "m3_ssm_prefill_block"
    if rc != capi.M3_OK:
        raise capi.M3Error(rc, fn)
    return y, final


def prefill_stage(stage: int, x, dt, A, lam, theta, B, C, state, final, y, workspace, chunk: int = 64):
    """Enqueue one stage of the prefill (include/m3_ssm_stages.h) with the
    arguments of a full prefill; used to time the kernels one at a time."""
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    io = x.dtype
    _check_bc(B, C, (b, T), R, N)
    rc = capi.m3_ssm_prefill_stage(
        stage, make_shape(b, T, H, P, N, R, io, chunk=chunk, G=B.shape[2],
                          state_dtype=next((q.h.dtype for q in (state, final) if q is not None), torch.float32)),
        _ptr(x, "x", io), _ptr(dt, "dt", io),
        _ptr(A, "A", torch.float32), _ptr(lam, "lam", io), _ptr(theta, "theta", io),
        _ptr(B, "B", io), _ptr(C, "C", io), state.c() if state is not None else None,
        final.c() if final is not None else None, _ptr(y, "y", io), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream())
    if rc != capi.M3_OK:
        raise capi.M3Error(rc, "m3_ssm_prefill_stage")


def decode_step(x, dt, A, lam, theta, B, C, state: State, y=None, block: Block | None = None,
                z=None):
    """One decode step (token axis dropped: x [b,H,R,P], ...).  Updates
    ``state`` in place and returns y [b,H,R,P].  ``block`` / ``z`` (shaped
    like x) add the block prologue and output gate."""
    b, H, R, P = x.shape
    N = B.shape[-1]
    io = x.dtype
    _check_bc(B, C, (b,), R, N)
    shape = make_shape(b, 1, H, P, N, R, io, G=B.shape[1], state_dtype=state.h.dtype)
    if y is None:
        y = torch.empty_like(x)
    if z is not None and tuple(z.shape) != tuple(x.shape):
        raise ValueError("z must be shaped like x")
    args = [shape, _ptr(x, "x", io), _ptr(dt, "dt", io), _ptr(A, "A", torch.float32),
            _ptr(lam, "lam", io), _ptr(theta, "theta", io), _ptr(B, "B", io), _ptr(C, "C", io)]
    blk = _block_c(block, z, io, H, R, N)
    if blk is None:
        rc, fn = capi.m3_ssm_decode_step(*args, state.c(), _ptr(y, "y", io), _stream()), "m3_ssm_decode_step"
    else:
        rc, fn = (capi.m3_ssm_decode_step_block(*args, blk, state.c(), _ptr(y, "y", io), _stream()),
                  "m3_ssm_decode_step_block")
    if rc != capi.M3_OK:
        raise capi.M3Error(rc, fn)
    return y


def backward(x, dt, A, lam, theta, B, C, gy, state: State | None = None, workspace=None,
             gfinal: dict | None = None):
    """Gradients of sum(gy * y) for y = prefill(x, ..., state=state).

    ``gfinal``: incoming gradients of the final carried state, a dict with
    any of h, phi, prev_B, prev_x (fp32 device tensors shaped like the
    State's fields); they add <gfinal, final state> to the loss, so that the
    gradients a later call returns for its initial state chain into this one.

    Returns a dict of fp32 tensors: x, dt, A, lam, theta, B, C and, when a
    carried state is given, h, phi, prev_B, prev_x (its gradients).
    """
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    io = x.dtype
    _check_bc(B, C, (b, T), R, N)
    if tuple(gy.shape) != tuple(x.shape):
        raise ValueError("gy must be shaped like x")
    shape = make_shape(b, T, H, P, N, R, io, G=B.shape[2],
                       state_dtype=state.h.dtype if state is not None else torch.float32)
    need = capi.m3_ssm_prefill_backward_workspace_bytes(shape)
    if need == 0:
        raise capi.M3Error(capi.M3_ERR_UNSUPPORTED, "m3_ssm_prefill_backward_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, device=x.device, dtype=torch.uint8)
    f = dict(device=x.device, dtype=torch.float32)
    g = {k: torch.empty(v.shape, **f) for k, v in dict(x=x, dt=dt, A=A, lam=lam, theta=theta, B=B, C=C).items()}
    if state is not None:
        g.update(h=torch.empty(state.h.shape, **f), phi=torch.empty(state.phi.shape, **f),
                 prev_B=torch.empty(state.prev_B.shape, **f), prev_x=torch.empty(state.prev_x.shape, **f))
    gs = capi.m3_grads_t(*(g[k].data_ptr() if k in g else None for k in
                           ("x", "dt", "A", "lam", "theta", "B", "C", "h", "phi", "prev_B", "prev_x")))
    gf = None
    if gfinal:
        want = dict(h=(b, H, N, P), phi=(b, H, N // 2), prev_B=(b, H, R, N), prev_x=(b, H, R, P))
        ptrs = {}
        for k, t in gfinal.items():
            if k not in want:
                raise ValueError(f"gfinal: unknown entry {k}")
            if t is None:
                continue
            if tuple(t.shape) != want[k]:
                raise ValueError(f"gfinal[{k}] must be {want[k]}, got {tuple(t.shape)}")
            ptrs[k] = _ptr(t, "gfinal." + k, torch.float32)
        gf = capi.m3_final_grads_t(*(ptrs.get(k) for k in ("h", "phi", "prev_B", "prev_x")))
    rc = capi.m3_ssm_prefill_backward_ex(
        shape, _ptr(x, "x", io), _ptr(dt, "dt", io), _ptr(A, "A", torch.float32),
        _ptr(lam, "lam", io), _ptr(theta, "theta", io), _ptr(B, "B", io), _ptr(C, "C", io),
        state.c() if state is not None else None, _ptr(gy, "gy", io), gf, gs,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    if rc != capi.M3_OK:
        raise capi.M3Error(rc, "m3_ssm_prefill_backward_ex")
    return g
