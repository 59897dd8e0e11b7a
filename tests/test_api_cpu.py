"""C ABI checks that need no GPU: the library loads, exports every function
include/m3_ssm.h declares, and rejects bad arguments with the documented
status codes.  Every call here fails validation before any HIP call, so no
device is touched (the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from mamba_selective_ssm_ssd_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

FAKE = 0x10000          # aligned, never dereferenced
FAKE_MISALIGNED = 0x10002


def _declared_functions():
    names = set()
    for f in os.listdir(INCLUDE):
        if f.endswith(".h"):
            text = open(os.path.join(INCLUDE, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(m3_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = capi.load()
    names = _declared_functions()
    assert set(names) == set(capi.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert capi.m3_status_string(capi.M3_OK) == "M3_OK"
    assert capi.m3_status_string(capi.M3_ERR_WORKSPACE) == "M3_ERR_WORKSPACE"
    assert capi.m3_status_string(99) == "M3_ERR_UNKNOWN"


def _shape(**kw):
    d = dict(batch=2, seqlen=100, nheads=3, headdim=64, dstate=64, rank=4, chunk=64,
             io_dtype=capi.M3_DTYPE_BF16)
    d.update(kw)
    return capi.m3_shape_t(**d)


def test_workspace_bytes():
    ws = capi.m3_ssm_prefill_workspace_bytes(_shape())
    # b2 T100 H3: 6 sequences of 2 chunks -> 2 segments of one chunk each
    bh, S, N, P, K = 6, 2, 64, 64, 32
    at_least = bh * S * N * P * 4 + bh * S * 4 + bh * S * K * 8 + bh * N * P * 4 + bh * K * 8
    assert at_least <= ws <= at_least + 5 * 256
    # one segment per sequence once batch * heads fills the chip
    big = capi.m3_ssm_prefill_workspace_bytes(_shape(batch=4, nheads=64, seqlen=2048))
    bh = 256
    assert big <= bh * N * P * 4 * 2 + bh * (4 + K * 8 + K * 8) + 5 * 256
    # invalid or unsupported shapes report 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=63)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=48)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(headdim=128)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(rank=5)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(chunk=32)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(seqlen=0)) == 0
    # a whole fp32 chunk at N=128, R>=2 or N=64, R=4 does not fit in LDS; every bf16 shape does
    f32 = capi.M3_DTYPE_F32
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=128, rank=2, io_dtype=f32)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=128, rank=1, io_dtype=f32)) > 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(io_dtype=f32)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(rank=3, io_dtype=f32)) > 0
    for n in (16, 32, 64, 128):
        for r in (1, 2, 3, 4):
            for pd in (16, 32, 64):
                assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=n, rank=r, headdim=pd)) > 0


def _prefill(shape, **over):
    args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, init=None,
                final_state=None, y=FAKE, workspace=FAKE, workspace_bytes=0, stream=None)
    args.update(over)
    return capi.m3_ssm_prefill(shape, **args)


@pytest.mark.parametrize("field,value,expect", [
    ("dstate", 63, capi.M3_ERR_INVALID_ARGUMENT),
    ("dstate", 48, capi.M3_ERR_UNSUPPORTED),
    ("headdim", 0, capi.M3_ERR_INVALID_ARGUMENT),
    ("headdim", 128, capi.M3_ERR_UNSUPPORTED),
    ("rank", 0, capi.M3_ERR_INVALID_ARGUMENT),
    ("rank", 5, capi.M3_ERR_UNSUPPORTED),
    ("seqlen", 0, capi.M3_ERR_INVALID_ARGUMENT),
    ("batch", 0, capi.M3_ERR_INVALID_ARGUMENT),
    ("nheads", -1, capi.M3_ERR_INVALID_ARGUMENT),
    ("chunk", 32, capi.M3_ERR_UNSUPPORTED),
    ("chunk", 0, capi.M3_ERR_INVALID_ARGUMENT),
    ("io_dtype", 7, capi.M3_ERR_INVALID_ARGUMENT),
])
def test_prefill_shape_errors(field, value, expect):
    assert _prefill(_shape(**{field: value})) == expect


@pytest.mark.parametrize("name", ["x", "dt", "A", "lam", "theta", "B", "C", "y"])
def test_prefill_pointer_errors(name):
    assert _prefill(_shape(), **{name: None}) == capi.M3_ERR_INVALID_ARGUMENT
    assert _prefill(_shape(), **{name: FAKE_MISALIGNED}) == capi.M3_ERR_INVALID_ARGUMENT


def test_prefill_state_errors():
    bad = capi.m3_state_t(FAKE, None, FAKE, FAKE)
    assert _prefill(_shape(), init=bad) == capi.M3_ERR_INVALID_ARGUMENT
    assert _prefill(_shape(), final_state=bad) == capi.M3_ERR_INVALID_ARGUMENT
    mis = capi.m3_state_t(FAKE, FAKE, FAKE_MISALIGNED, FAKE)
    assert _prefill(_shape(), init=mis) == capi.M3_ERR_INVALID_ARGUMENT


def test_prefill_workspace_errors():
    need = capi.m3_ssm_prefill_workspace_bytes(_shape())
    assert _prefill(_shape(), workspace=None, workspace_bytes=need) == capi.M3_ERR_WORKSPACE
    assert _prefill(_shape(), workspace_bytes=need - 1) == capi.M3_ERR_WORKSPACE
    assert _prefill(_shape(), workspace=FAKE_MISALIGNED, workspace_bytes=need) == capi.M3_ERR_WORKSPACE


def test_stage_errors():
    need = capi.m3_ssm_prefill_workspace_bytes(_shape())
    args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, init=None,
                final_state=None, y=FAKE, workspace=FAKE, workspace_bytes=need, stream=None)
    for bad in (-1, 2, 100):
        assert capi.m3_ssm_prefill_stage(bad, _shape(), **args) == capi.M3_ERR_INVALID_ARGUMENT
    args["workspace_bytes"] = need - 1
    assert capi.m3_ssm_prefill_stage(0, _shape(), **args) == capi.M3_ERR_WORKSPACE
    assert capi.m3_ssm_prefill_stage(1, _shape(dstate=5), **args) == capi.M3_ERR_INVALID_ARGUMENT


def test_decode_errors():
    st = capi.m3_state_t(FAKE, FAKE, FAKE, FAKE)

    def dec(shape, **over):
        args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, state=st,
                    y=FAKE, stream=None)
        args.update(over)
        return capi.m3_ssm_decode_step(shape, **args)

    assert dec(_shape(), state=None) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(_shape(), state=capi.m3_state_t(FAKE, FAKE, None, FAKE)) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(_shape(), x=None) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(_shape(dstate=7)) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(_shape(rank=9)) == capi.M3_ERR_UNSUPPORTED
    assert dec(_shape(io_dtype=3)) == capi.M3_ERR_INVALID_ARGUMENT


def test_null_shape():
    lib = capi.load()
    assert lib.m3_ssm_prefill_workspace_bytes(None) == 0
    st = capi.m3_state_t(FAKE, FAKE, FAKE, FAKE)
    assert lib.m3_ssm_decode_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  ctypes.byref(st), FAKE, None) == capi.M3_ERR_INVALID_ARGUMENT
    assert lib.m3_ssm_prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                              FAKE, FAKE, 1 << 30, None) == capi.M3_ERR_INVALID_ARGUMENT


def test_product_path_does_not_import_the_oracle():
    """The package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "mamba_selective_ssm_ssd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "m3_oracle" not in text and "libm3oracle" not in text, f


def _prefill_block(shape, block, **over):
    args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, block=block,
                init=None, final_state=None, y=FAKE, workspace=FAKE, workspace_bytes=0,
                stream=None)
    args.update(over)
    return capi.m3_ssm_prefill_block(shape, **args)


def test_block_errors():
    """Validation of the block prologue/epilogue (include/m3_ssm_block.h).
    Valid blocks reach the workspace check, which fails (0 bytes given)."""
    W = capi.M3_ERR_WORKSPACE
    assert _prefill_block(_shape(), None) == W
    assert _prefill_block(_shape(), capi.m3_block_t(1, 1e-6, FAKE, FAKE, FAKE, FAKE, FAKE)) == W
    assert _prefill_block(_shape(), capi.m3_block_t(0, -1.0)) == W          # eps unused
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _prefill_block(_shape(), capi.m3_block_t(1, eps)) == capi.M3_ERR_INVALID_ARGUMENT
    for i in range(5):
        ptrs = [None] * 5
        ptrs[i] = FAKE_MISALIGNED
        assert _prefill_block(_shape(), capi.m3_block_t(0, 0.0, *ptrs)) == capi.M3_ERR_INVALID_ARGUMENT
    # bf16, N = 128, P = 64, R = 4: the weight table no longer fits in LDS
    big = _shape(dstate=128, rank=4)
    assert _prefill_block(big, None) == W
    assert _prefill_block(big, capi.m3_block_t(1, 1e-6)) == capi.M3_ERR_UNSUPPORTED
    st = capi.m3_state_t(FAKE, FAKE, FAKE, FAKE)

    def dec(block, **over):
        args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, block=block,
                    state=st, y=FAKE, stream=None)
        args.update(over)
        return capi.m3_ssm_decode_step_block(_shape(), **args)

    assert dec(capi.m3_block_t(1, -2.0)) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(capi.m3_block_t(0, 0.0, None, None, None, None, FAKE_MISALIGNED)) == capi.M3_ERR_INVALID_ARGUMENT
    assert dec(capi.m3_block_t(1, 1e-6), x=None) == capi.M3_ERR_INVALID_ARGUMENT


def test_group_errors():
    """ngroups (B/C shared by head groups) must divide nheads; 0 means per head."""
    W = capi.M3_ERR_WORKSPACE
    assert _prefill(_shape(nheads=6, ngroups=0)) == W
    assert _prefill(_shape(nheads=6, ngroups=3)) == W
    assert _prefill(_shape(nheads=6, ngroups=1)) == W
    assert _prefill(_shape(nheads=6, ngroups=6)) == W
    for g in (-1, 4, 7):
        assert _prefill(_shape(nheads=6, ngroups=g)) == capi.M3_ERR_INVALID_ARGUMENT
        assert capi.m3_ssm_prefill_workspace_bytes(_shape(nheads=6, ngroups=g)) == 0
    st = capi.m3_state_t(FAKE, FAKE, FAKE, FAKE)
    assert capi.m3_ssm_decode_step(_shape(nheads=6, ngroups=4), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, st, FAKE, None) == capi.M3_ERR_INVALID_ARGUMENT
    # group count does not change the workspace
    assert (capi.m3_ssm_prefill_workspace_bytes(_shape(nheads=6, ngroups=2))
            == capi.m3_ssm_prefill_workspace_bytes(_shape(nheads=6)))


def test_state_dtype_errors():
    W = capi.M3_ERR_WORKSPACE
    assert _prefill(_shape(state_dtype=capi.M3_DTYPE_F32)) == W
    assert _prefill(_shape(state_dtype=capi.M3_DTYPE_BF16)) == W
    for sd in (-1, 2, 9):
        assert _prefill(_shape(state_dtype=sd)) == capi.M3_ERR_INVALID_ARGUMENT
    st = capi.m3_state_t(FAKE, FAKE, FAKE, FAKE)
    assert capi.m3_ssm_decode_step(_shape(state_dtype=5), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, st, FAKE, None) == capi.M3_ERR_INVALID_ARGUMENT


def test_backward_errors():
    """Validation of the backward entry (include/m3_ssm_backward.h)."""
    W = capi.M3_ERR_WORKSPACE
    g = capi.m3_grads_t(*([FAKE] * 7 + [None] * 4))

    def bwd(shape, **over):
        args = dict(x=FAKE, dt=FAKE, A=FAKE, lam=FAKE, theta=FAKE, B=FAKE, C=FAKE, init=None, gy=FAKE,
                    grads=g, workspace=FAKE, workspace_bytes=0, stream=None)
        args.update(over)
        return capi.m3_ssm_prefill_backward(shape, **args)

    assert bwd(_shape()) == W
    assert capi.m3_ssm_prefill_backward_workspace_bytes(_shape()) > 0
    assert bwd(_shape(nheads=6, ngroups=2)) == capi.M3_ERR_UNSUPPORTED
    assert bwd(_shape(state_dtype=capi.M3_DTYPE_BF16)) == capi.M3_ERR_UNSUPPORTED
    assert capi.m3_ssm_prefill_backward_workspace_bytes(_shape(nheads=6, ngroups=3)) == 0
    assert bwd(_shape(), gy=None) == capi.M3_ERR_INVALID_ARGUMENT
    assert bwd(_shape(), grads=None) == capi.M3_ERR_INVALID_ARGUMENT
    for i in range(7):
        ptrs = [FAKE] * 7 + [None] * 4
        ptrs[i] = None
        assert bwd(_shape(), grads=capi.m3_grads_t(*ptrs)) == capi.M3_ERR_INVALID_ARGUMENT
    assert bwd(_shape(), grads=capi.m3_grads_t(*([FAKE] * 7 + [FAKE_MISALIGNED, None, None, None]))) \
        == capi.M3_ERR_INVALID_ARGUMENT
    assert bwd(_shape(dstate=5)) == capi.M3_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("b,T,H,P,N,R", [(4, 2048, 64, 64, 128, 1), (4, 2048, 64, 64, 64, 4),
                                        (1, 150, 2, 32, 64, 3), (2, 1, 3, 16, 16, 2)])
def test_backward_workspace_size_as_documented(b, T, H, P, N, R):
    """include/m3_ssm_backward.h: per (batch, head), one fp32 state and one
    fp64 angle vector per chunk of 32 / R tokens, plus alignment and 4 bytes."""
    import math
    torch = pytest.importorskip("torch")
    from mamba_selective_ssm_ssd_amd import capi, mixer
    got = capi.m3_ssm_prefill_backward_workspace_bytes(mixer.make_shape(b, T, H, P, N, R, torch.bfloat16))
    est = b * H * math.ceil(T / (32 // R)) * (N * P * 4 + N // 2 * 8) + 4 * b * H
    assert est <= got <= est + 3 * 256
