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


def test_library_imports_no_allocation_copy_or_synchronisation():
    """The library never allocates, frees, copies or synchronises
    (include/m3_ssm.h; m3_ssm_prefill_noalloc takes a static array): none of
    its dynamic imports is a HIP allocation, free, memset, memcpy or
    synchronisation routine."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not installed")
    out = subprocess.run([nm, "-D", "--undefined-only", capi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = [line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()]
    assert any(n == "hipLaunchKernel" for n in names)       # the listing is the library's
    banned = re.compile(r"^hip(Malloc|Free|HostMalloc|HostAlloc|HostFree|HostRegister|ExtMalloc|"
                        r"MemAlloc|MemPool|Memset|Memcpy|DeviceSynchronize|StreamSynchronize|"
                        r"EventSynchronize|MallocAsync|FreeAsync)")
    bad = sorted(n for n in names if banned.match(n))
    assert not bad, f"allocation / copy / synchronisation imports: {bad}"


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


def _segments(bh, T, Q, slots=256):
    """Segments per sequence for a chunk length Q: enough (batch, head,
    segment) workgroups to fill 256 compute units, no empty segment."""
    nC = -(-T // Q)
    s = max(1, min(1 if bh >= slots else slots // bh, nC))
    c = -(-nC // s)
    return -(-nC // c)


def test_workspace_bytes():
    ws = capi.m3_ssm_prefill_workspace_bytes(_shape())
    # b2 T100 H3 R4 bf16: 6 sequences of two 64-token pre-pass chunks -> 2
    # segments; the pre-pass covers the first, one aggregate per sequence
    assert capi.m3_ssm_prefill_plan(_shape()) == (0, 64, 16, 2, 64, 1)
    assert _segments(6, 100, 64) == 2
    bh, N, P, K, NA = 6, 64, 64, 32, 1
    at_least = bh * NA * N * P * 4 + bh * NA * 4 + bh * NA * K * 8 + bh * N * P * 4 + bh * K * 8
    assert at_least <= ws <= at_least + 5 * 256
    # one segment per sequence once batch * heads fills the chip: unused
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(batch=4, nheads=64, seqlen=2048)) == 256
    # never more than the allocation-free entry point's static array
    # (include/m3_ssm_noalloc.h): aggregates below 16 MiB, the carried state
    # of fewer than 256 sequences
    worst = 0
    for n in (16, 64, 128):
        for pd in (16, 64):
            for r in (1, 4):
                for bh_ in (1, 2, 3, 5, 17, 32, 63, 64, 85, 100, 127, 128, 200, 255, 256):
                    for T in (1, 100, 2048, 5000, 65536):
                        w = capi.m3_ssm_prefill_workspace_bytes(
                            _shape(batch=1, nheads=bh_, seqlen=T, dstate=n, headdim=pd, rank=r))
                        assert 0 < w <= capi.M3_NOALLOC_SCRATCH_BYTES, (n, pd, r, bh_, T, w)
                        worst = max(worst, w)
    assert worst <= 27e6
    # invalid or unsupported shapes report 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=63)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(dstate=48)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(headdim=128)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(rank=5)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(seqlen=0)) == 0
    # chunk: 64 or the rank's small chunk (64/R tokens; 32 for R = 3)
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(chunk=32)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(chunk=16)) > 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(chunk=128)) == 0
    for r, q in ((1, 64), (2, 32), (3, 32), (4, 16)):
        assert capi.m3_ssm_prefill_workspace_bytes(_shape(rank=r, chunk=q)) > 0
        for bad in (8, 16, 32, 48):
            if bad != q:
                assert capi.m3_ssm_prefill_workspace_bytes(_shape(rank=r, chunk=bad)) == 0
    # every (N, P, R) in both I/O types: with fp32 I/O a 64-token chunk at
    # N = 128 with R >= 2 or N = 64 with R = 4 exceeds the LDS and takes the
    # small chunk
    for io in (capi.M3_DTYPE_F32, capi.M3_DTYPE_BF16):
        for n in (16, 32, 64, 128):
            for r in (1, 2, 3, 4):
                for pd in (16, 32, 64):
                    assert capi.m3_ssm_prefill_workspace_bytes(
                        _shape(dstate=n, rank=r, headdim=pd, io_dtype=io)) > 0


def test_prefill_plan_prepass_pieces():
    """The long-context MIMO shape (b1 T65536 H64): 4 segments of 16384 tokens;
    the pre-pass's 3 x 64 = 192 workgroups would leave a quarter of 256 compute
    units idle, so each segment is cut into 4 pieces (768 workgroups, three
    full rounds).  The output pass takes 16-token chunks, the pre-pass 64."""
    sh = _shape(batch=1, nheads=64, seqlen=65536, dstate=64, headdim=64, rank=4)
    assert capi.m3_ssm_prefill_plan(sh) == (0, 64, 16, 4, 16384, 4)
    ws = capi.m3_ssm_prefill_workspace_bytes(sh)
    NA = 12                                           # (4 - 1) x 4 aggregates per sequence
    at_least = 64 * NA * (64 * 64 * 4 + 4 + 32 * 8) + 64 * (64 * 64 * 4 + 32 * 8)
    assert at_least <= ws <= at_least + 5 * 256
    # whole rounds already: no pieces (b1 H128 -> 2 segments, 128 pre-pass workgroups -> 2 pieces)
    assert capi.m3_ssm_prefill_plan(_shape(batch=1, nheads=128, seqlen=4096))[3:] == (2, 2048, 2)
    assert capi.m3_ssm_prefill_plan(_shape(batch=1, nheads=256, seqlen=4096))[3:] == (1, 4096, 1)
    # aggregates would pass 16 MiB: no pieces (N = 128, P = 64: 32 KiB each, 192 x 4 = 768 of them)
    assert capi.m3_ssm_prefill_plan(_shape(batch=1, nheads=64, seqlen=65536, dstate=128, rank=1))[3:] == (4, 16384, 1)


def test_in_chunk_offsets_stay_32_bit():
    """Offsets within a chunk are 32-bit: 64 * H * R * max(N, P) must stay
    below 2^31 (a larger shape would wrap them); the boundary is exact."""
    H = 2 ** 31 // (64 * 4 * 64)                      # 64 * H * 4 * 64 == 2^31
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(batch=1, nheads=H)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(batch=1, nheads=H - 1)) > 0
    H2 = 2 ** 31 // (64 * 1 * 128)
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(batch=1, nheads=H2, rank=1, dstate=128)) == 0
    assert capi.m3_ssm_prefill_workspace_bytes(_shape(batch=1, nheads=H2 - 1, rank=1, dstate=128)) > 0
    assert capi.m3_ssm_prefill_backward_workspace_bytes(_shape(batch=1, nheads=H)) == 0
    # decode: the same limit
    rc = capi.m3_ssm_decode_step(_shape(batch=1, nheads=H), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, capi.m3_state_t(FAKE, FAKE, FAKE, FAKE), FAKE, None)
    assert rc == capi.M3_ERR_UNSUPPORTED


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
    # bf16, N = 128, P = 64, R = 4: with the weight table the 64-token chunk no
    # longer fits in LDS, and the block kernels take 16-token chunks
    big = _shape(dstate=128, rank=4)
    assert _prefill_block(big, None) == W
    assert _prefill_block(big, capi.m3_block_t(1, 1e-6)) == W
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
                                        (1, 150, 2, 32, 64, 3), (2, 1, 3, 16, 16, 2),
                                        (1, 65536, 64, 64, 64, 4), (1, 1000, 1, 16, 32, 2)])
def test_backward_workspace_size_as_documented(b, T, H, P, N, R):
    """include/m3_ssm_backward.h: per (batch, head), one fp32 state and one
    fp64 angle vector per chunk of 32 / R tokens, plus alignment, 4 bytes per
    (batch, head, segment) and the aggregates of split sequences."""
    import math
    torch = pytest.importorskip("torch")
    from mamba_selective_ssm_ssd_amd import capi, mixer
    shape = mixer.make_shape(b, T, H, P, N, R, torch.bfloat16)
    got = capi.m3_ssm_prefill_backward_workspace_bytes(shape)
    rc, S, _ = capi.m3_ssm_prefill_backward_plan(shape)
    assert rc == capi.M3_OK
    est = b * H * math.ceil(T / (32 // R)) * (N * P * 4 + N // 2 * 8) + 4 * b * H * S
    if S > 1:
        lo = b * H * S * (1 * (8 * N * P + 4 + 4 * N) + 4 + 4 * N)
        hi = b * H * S * (8 * (8 * N * P + 4 + 4 * N) + 4 + 4 * N)
        assert est + lo <= got <= est + hi + 9 * 256
        return
    assert est <= got <= est + 9 * 256


@pytest.mark.parametrize("b,T,H,R,S,tokens", [
    (4, 2048, 64, 1, 1, 2048),        # 256 sequences fill the chip
    (4, 2048, 64, 4, 1, 2048),
    (1, 65536, 64, 4, 4, 16384),      # long context: 64 sequences, 4 segments
    (1, 150, 2, 1, 2, 96),            # 5 chunks of 32 tokens: 2 segments of 3, 2 chunks
    (2, 150, 2, 4, 7, 24),            # 19 chunks of 8 tokens: segments of 3 chunks
    (1, 64, 1, 1, 1, 64),             # 2 chunks: too short to split
    (1, 100000, 1, 2, 64, 1568),      # at most 64 segments
])
def test_backward_plan(b, T, H, R, S, tokens):
    """m3_ssm_prefill_backward_plan: fewer than 256 sequences are cut into
    segments of at least two chunks (at most 64) so that the grid fills the
    256 CUs; the segments cover the sequence and none is empty."""
    import math
    torch = pytest.importorskip("torch")
    from mamba_selective_ssm_ssd_amd import capi, mixer
    rc, got_s, got_t = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(b, T, H, 64, 64, R, torch.bfloat16))
    assert rc == capi.M3_OK
    assert (got_s, got_t) == (S, tokens)
    Q = 32 // R
    assert got_t % Q == 0 and (got_s - 1) * got_t < T <= got_s * got_t
    assert got_s == 1 or got_t >= 2 * Q
    rc, _, _ = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(b, T, H, 64, 5, R, torch.bfloat16))
    assert rc == capi.M3_ERR_INVALID_ARGUMENT


def test_ceiling_errors():
    """The on-box ceiling kernels reject bad arguments before any launch."""
    for mode in (-1, 4, 9):
        assert capi.m3_ceiling_stream(mode, FAKE, FAKE, 64, 8, None) == capi.M3_ERR_INVALID_ARGUMENT
    for mode in (0, 2):  # copies need a source
        assert capi.m3_ceiling_stream(mode, None, FAKE, 64, 8, None) == capi.M3_ERR_INVALID_ARGUMENT
        assert capi.m3_ceiling_stream(mode, FAKE_MISALIGNED, FAKE, 64, 8, None) == capi.M3_ERR_INVALID_ARGUMENT
    for mode in range(4):
        assert capi.m3_ceiling_stream(mode, FAKE, None, 64, 8, None) == capi.M3_ERR_INVALID_ARGUMENT
        assert capi.m3_ceiling_stream(mode, FAKE, FAKE, 0, 8, None) == capi.M3_ERR_INVALID_ARGUMENT
        assert capi.m3_ceiling_stream(mode, FAKE, FAKE, 64, 0, None) == capi.M3_ERR_INVALID_ARGUMENT
    for kind in (-1, 2):
        assert capi.m3_ceiling_mfma(kind, 8, 1, FAKE, None) == capi.M3_ERR_INVALID_ARGUMENT
    assert capi.m3_ceiling_mfma(0, 0, 1, FAKE, None) == capi.M3_ERR_INVALID_ARGUMENT
    assert capi.m3_ceiling_mfma(0, 8, 1, None, None) == capi.M3_ERR_INVALID_ARGUMENT
