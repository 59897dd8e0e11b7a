"""GPU parity of the backward pass (m3_ssm_prefill_backward) against the
oracle's gradients (fp64 autograd, pinned by finite differences of the C
oracle): every input and the carried state, SISO and MIMO, both I/O types,
several chunks with a ragged tail, fresh and carried states.

Bar: 1e-4 per (b, h) slice of each gradient, max|g - r| / max|r|, for both
I/O types: the kernel computes in fp32 (angles in fp64) from the stored input
values, and no intermediate is rounded to bf16, so the fp32 bar of the
forward applies to both (measured: 1e-7 .. 7e-6).
"""
import numpy as np
import pytest

from oracle import backward as ob
from mamba_selective_ssm_ssd_amd import synth
from _helpers import slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BAR = 1e-4

# (b, h) axes of each gradient for the per-slice error
AXES = dict(x=(0, 2), dt=(0, 2), lam=(0, 2), theta=(0, 2), B=(0, 2), C=(0, 2),
            h=(0, 1), phi=(0, 1), prev_B=(0, 1), prev_x=(0, 1))


def _run(b, T, H, P, N, R, io, seed, with_init):
    from mamba_selective_ssm_ssd_amd import mixer
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=90)
    d["A"] *= 0.2                                  # slower decay: long-range terms matter
    rng = np.random.default_rng(900 + seed)
    gy = synth.round_io(rng.standard_normal((b, T, H, R, P)), io)
    init_np, st = None, None
    if with_init:
        init_np = dict(h0=rng.standard_normal((b, H, N, P)).astype(np.float32) * 0.5,
                       phi0=rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32),
                       prevB0=rng.standard_normal((b, H, R, N)).astype(np.float32),
                       prevx0=synth.round_io(rng.standard_normal((b, H, R, P)), io))
        st = mixer.State(*(torch.from_numpy(init_np[k]).cuda() for k in ("h0", "phi0", "prevB0")),
                         torch.from_numpy(init_np["prevx0"]).to("cuda", torch_io(io)))
    t = to_dev(d, io)
    gyd = torch.from_numpy(gy).to("cuda", torch_io(io))
    g = mixer.backward(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")), gyd, state=st)
    torch.cuda.synchronize()
    _, r = ob.grad(d, gy, {k: v.astype(np.float64) for k, v in init_np.items()} if init_np else None)
    errs = {}
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        errs[k] = slice_err(g[k].double().cpu().numpy(), r[k], AXES[k])
    gA, rA = g["A"].double().cpu().numpy(), r["A"]
    errs["A"] = float(np.max(np.abs(gA - rA)) / np.max(np.abs(rA)))
    if with_init:
        for k, rk in (("h", "g_h0"), ("phi", "g_phi0"), ("prev_B", "g_prevB0"), ("prev_x", "g_prevx0")):
            errs[k] = slice_err(g[k].double().cpu().numpy(), r[rk], AXES[k])
    return errs


@pytest.mark.parametrize("N,P,R,io", [
    (16, 16, 1, "f32"), (32, 32, 2, "f32"), (64, 32, 3, "f32"), (128, 32, 2, "f32"),
    (64, 64, 4, "bf16"), (128, 64, 1, "bf16"), (32, 64, 4, "bf16"),
])
@pytest.mark.parametrize("with_init", [False, True])
def test_backward_parity(N, P, R, io, with_init):
    errs = _run(2, 150, 2, P, N, R, io, seed=N + P + R, with_init=with_init)
    print(f"backward N{N} P{P} R{R} {io} init={with_init}: "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200])
def test_backward_short_and_ragged(T):
    errs = _run(1, T, 3, 16, 32, 2, "f32", seed=T, with_init=True)
    for k, v in errs.items():
        assert v <= BAR, f"T={T}: gradient of {k}: error {v:.3e}"


@pytest.mark.parametrize("seed", range(16))
def test_backward_random_case(seed):
    """Seeded random configurations: N, P, R, I/O type, batch, heads, T
    (several chunks with a ragged tail, or fewer tokens than one chunk) and a
    carried state or none."""
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.choice([16, 32, 64, 128]))
    P = int(rng.choice([16, 32, 64]))
    R = int(rng.integers(1, 5))
    io = str(rng.choice(["f32", "bf16"]))
    b, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    T = int(rng.integers(1, 320))
    with_init = bool(rng.random() < 0.5)
    from mamba_selective_ssm_ssd_amd import capi, mixer
    if capi.m3_ssm_prefill_backward_workspace_bytes(mixer.make_shape(b, T, H, P, N, R, torch_io(io))) == 0:
        pytest.skip(f"shape outside the compiled set (the shapes m3_ssm_prefill supports): N{N} P{P} R{R} {io}")
    errs = _run(b, T, H, P, N, R, io, seed=4000 + seed, with_init=with_init)
    print(f"case {seed}: N{N} P{P} R{R} {io} b{b} H{H} T{T} init={with_init}: "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"case {seed}: gradient of {k}: error {v:.3e}"
