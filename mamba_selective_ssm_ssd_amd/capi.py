"""ctypes binding of libm3ssm.so: the C ABI declared in include/m3_ssm*.h.

The functions here have the same names and arguments as the C entry points
and only marshal arguments.  Loading fails loudly when the library has not
been built; there is no other implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libm3ssm.so")

M3_DTYPE_F32 = 0
M3_DTYPE_BF16 = 1

M3_OK = 0
M3_ERR_INVALID_ARGUMENT = 1
M3_ERR_UNSUPPORTED = 2
M3_ERR_WORKSPACE = 3
M3_ERR_HIP = 4

# Every function the headers under include/ declare.
EXPORTED = ("m3_ssm_prefill_workspace_bytes", "m3_ssm_prefill", "m3_ssm_decode_step",
            "m3_status_string", "m3_ssm_prefill_stage", "m3_ssm_prefill_block",
            "m3_ssm_decode_step_block", "m3_ssm_prefill_backward_workspace_bytes",
            "m3_ssm_prefill_backward", "m3_ssm_prefill_backward_ex", "m3_ssm_prefill_backward_plan",
            "m3_ssm_prefill_noalloc",
            "m3_ssm_prefill_plan",
            "m3_ceiling_mfma", "m3_ceiling_stream")

# Size of the static workspace of m3_ssm_prefill_noalloc (include/m3_ssm_noalloc.h).
M3_NOALLOC_SCRATCH_BYTES = 32 << 20

# Stages of the prefill (include/m3_ssm_stages.h).
M3_STAGE_SEGMENT_STATE = 0
M3_STAGE_OUTPUT = 1
STAGES = {"segment_state": 0, "output": 1}


class m3_shape_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("state_dtype", ctypes.c_int32)]


class m3_state_t(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("phi", ctypes.c_void_p),
                ("prev_B", ctypes.c_void_p), ("prev_x", ctypes.c_void_p)]


class m3_block_t(ctypes.Structure):
    """Block prologue/epilogue (include/m3_ssm_block.h)."""
    _fields_ = [("bc_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("B_weight", ctypes.c_void_p), ("B_bias", ctypes.c_void_p),
                ("C_weight", ctypes.c_void_p), ("C_bias", ctypes.c_void_p),
                ("z", ctypes.c_void_p)]


class m3_grads_t(ctypes.Structure):
    """Gradient outputs of the backward pass (include/m3_ssm_backward.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x", "dt", "A", "lam", "theta", "B", "C", "h", "phi", "prev_B", "prev_x")]


class m3_final_grads_t(ctypes.Structure):
    """Incoming gradients of the final carried state (include/m3_ssm_backward.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("h", "phi", "prev_B", "prev_x")]


class M3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {m3_status_string(status)} ({status})")
        self.status = status


_lib = None


def load():
    """Load libm3ssm.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mamba_selective_ssm_ssd_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sp = ctypes.c_void_p, ctypes.POINTER(m3_shape_t)
    stp = ctypes.POINTER(m3_state_t)
    lib.m3_ssm_prefill_workspace_bytes.argtypes = [sp]
    lib.m3_ssm_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.m3_ssm_prefill.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, stp, stp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.m3_ssm_prefill.restype = ctypes.c_int
    lib.m3_ssm_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, stp, vp, vp]
    lib.m3_ssm_decode_step.restype = ctypes.c_int
    lib.m3_ssm_prefill_stage.argtypes = [ctypes.c_int32, sp, vp, vp, vp, vp, vp, vp, vp, stp, stp,
                                         vp, vp, ctypes.c_size_t, vp]
    lib.m3_ssm_prefill_stage.restype = ctypes.c_int
    bkp = ctypes.POINTER(m3_block_t)
    lib.m3_ssm_prefill_block.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, bkp, stp, stp, vp, vp,
                                         ctypes.c_size_t, vp]
    lib.m3_ssm_prefill_block.restype = ctypes.c_int
    lib.m3_ssm_decode_step_block.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, bkp, stp, vp, vp]
    lib.m3_ssm_decode_step_block.restype = ctypes.c_int
    gp = ctypes.POINTER(m3_grads_t)
    lib.m3_ssm_prefill_backward_workspace_bytes.argtypes = [sp]
    lib.m3_ssm_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.m3_ssm_prefill_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, stp, vp, gp, vp,
                                            ctypes.c_size_t, vp]
    lib.m3_ssm_prefill_backward.restype = ctypes.c_int
    lib.m3_ssm_prefill_backward_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, stp, vp,
                                               ctypes.POINTER(m3_final_grads_t), gp, vp,
                                               ctypes.c_size_t, vp]
    lib.m3_ssm_prefill_backward_ex.restype = ctypes.c_int
    lib.m3_ssm_prefill_backward_plan.argtypes = [sp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    lib.m3_ssm_prefill_backward_plan.restype = ctypes.c_int
    lib.m3_ssm_prefill_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, stp, stp, vp, vp]
    lib.m3_ssm_prefill_noalloc.restype = ctypes.c_int
    i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.m3_ssm_prefill_plan.argtypes = [sp, ctypes.c_int32, i32p, i32p, i32p, i64p, i32p]
    lib.m3_ssm_prefill_plan.restype = ctypes.c_int
    lib.m3_ceiling_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.m3_ceiling_mfma.restype = ctypes.c_int
    lib.m3_ceiling_stream.argtypes = [ctypes.c_int32, vp, vp, ctypes.c_int64, ctypes.c_int32, vp]
    lib.m3_ceiling_stream.restype = ctypes.c_int
    lib.m3_status_string.argtypes = [ctypes.c_int]
    lib.m3_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def m3_status_string(status: int) -> str:
    return load().m3_status_string(int(status)).decode()


def m3_ssm_prefill_workspace_bytes(shape: m3_shape_t) -> int:
    return int(load().m3_ssm_prefill_workspace_bytes(ctypes.byref(shape)))


def m3_ssm_prefill(shape, x, dt, A, lam, theta, B, C, init, final_state, y, workspace,
                   workspace_bytes, stream) -> int:
    """Pointers are ints (device addresses) or None; init/final_state are
    m3_state_t or None.  Returns the m3_status_t value."""
    return int(load().m3_ssm_prefill(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(init) if init is not None else None,
        ctypes.byref(final_state) if final_state is not None else None,
        y, workspace, int(workspace_bytes), stream))


def m3_ssm_prefill_noalloc(shape, x, dt, A, lam, theta, B, C, init, final_state, y, stream) -> int:
    """m3_ssm_prefill with the library's static workspace (no workspace argument)."""
    return int(load().m3_ssm_prefill_noalloc(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(init) if init is not None else None,
        ctypes.byref(final_state) if final_state is not None else None, y, stream))


def m3_ssm_prefill_plan(shape, block=False):
    """(status, chunk_pre, chunk_out, segments, segment_tokens, prepass_pieces)
    of a shape; block: whether the call carries block pieces."""
    q1, q2, sg, kp = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = ctypes.c_int64(0)
    rc = int(load().m3_ssm_prefill_plan(ctypes.byref(shape), 1 if block else 0, ctypes.byref(q1),
                                        ctypes.byref(q2), ctypes.byref(sg), ctypes.byref(st),
                                        ctypes.byref(kp)))
    return rc, q1.value, q2.value, sg.value, st.value, kp.value


def m3_ceiling_mfma(kind, nblocks, iters, sink, stream) -> int:
    return int(load().m3_ceiling_mfma(int(kind), int(nblocks), int(iters), sink, stream))


def m3_ceiling_stream(mode, src, dst, n, nblocks, stream) -> int:
    return int(load().m3_ceiling_stream(int(mode), src, dst, int(n), int(nblocks), stream))


def m3_ssm_prefill_stage(stage, shape, x, dt, A, lam, theta, B, C, init, final_state, y,
                         workspace, workspace_bytes, stream) -> int:
    return int(load().m3_ssm_prefill_stage(
        int(stage), ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(init) if init is not None else None,
        ctypes.byref(final_state) if final_state is not None else None,
        y, workspace, int(workspace_bytes), stream))


def m3_ssm_decode_step(shape, x, dt, A, lam, theta, B, C, state, y, stream) -> int:
    return int(load().m3_ssm_decode_step(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(state) if state is not None else None, y, stream))


def m3_ssm_prefill_block(shape, x, dt, A, lam, theta, B, C, block, init, final_state, y,
                         workspace, workspace_bytes, stream) -> int:
    """m3_ssm_prefill with ``block`` (an m3_block_t or None)."""
    return int(load().m3_ssm_prefill_block(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(block) if block is not None else None,
        ctypes.byref(init) if init is not None else None,
        ctypes.byref(final_state) if final_state is not None else None,
        y, workspace, int(workspace_bytes), stream))


def m3_ssm_decode_step_block(shape, x, dt, A, lam, theta, B, C, block, state, y, stream) -> int:
    """m3_ssm_decode_step with ``block`` (an m3_block_t or None)."""
    return int(load().m3_ssm_decode_step_block(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(block) if block is not None else None,
        ctypes.byref(state) if state is not None else None, y, stream))


def m3_ssm_prefill_backward_workspace_bytes(shape: m3_shape_t) -> int:
    return int(load().m3_ssm_prefill_backward_workspace_bytes(ctypes.byref(shape)))


def m3_ssm_prefill_backward(shape, x, dt, A, lam, theta, B, C, init, gy, grads, workspace,
                            workspace_bytes, stream) -> int:
    """grads: an m3_grads_t of device addresses."""
    return int(load().m3_ssm_prefill_backward(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(init) if init is not None else None, gy,
        ctypes.byref(grads) if grads is not None else None,
        workspace, int(workspace_bytes), stream))


def m3_ssm_prefill_backward_ex(shape, x, dt, A, lam, theta, B, C, init, gy, gfinal, grads, workspace,
                               workspace_bytes, stream) -> int:
    """m3_ssm_prefill_backward with gfinal (an m3_final_grads_t or None)."""
    return int(load().m3_ssm_prefill_backward_ex(
        ctypes.byref(shape), x, dt, A, lam, theta, B, C,
        ctypes.byref(init) if init is not None else None, gy,
        ctypes.byref(gfinal) if gfinal is not None else None,
        ctypes.byref(grads) if grads is not None else None,
        workspace, int(workspace_bytes), stream))


def m3_ssm_prefill_backward_plan(shape):
    """(status, segments per sequence, tokens per segment) of the backward pass."""
    sg, tk = ctypes.c_int32(0), ctypes.c_int64(0)
    rc = int(load().m3_ssm_prefill_backward_plan(ctypes.byref(shape), ctypes.byref(sg), ctypes.byref(tk)))
    return rc, sg.value, tk.value
