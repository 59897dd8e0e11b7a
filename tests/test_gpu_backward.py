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


def _run(b, T, H, P, N, R, io, seed, with_init, with_gfinal=False):
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
    gf_np, gf = None, None
    if with_gfinal:
        gf_np = dict(h=rng.standard_normal((b, H, N, P)), phi=rng.standard_normal((b, H, N // 2)),
                     prev_B=rng.standard_normal((b, H, R, N)), prev_x=rng.standard_normal((b, H, R, P)))
        gf_np = {k: v.astype(np.float32) for k, v in gf_np.items()}
        gf = {k: torch.from_numpy(v).cuda() for k, v in gf_np.items()}
    t = to_dev(d, io)
    gyd = torch.from_numpy(gy).to("cuda", torch_io(io))
    g = mixer.backward(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")), gyd, state=st,
                       gfinal=gf)
    torch.cuda.synchronize()
    _, r = ob.grad(d, gy, {k: v.astype(np.float64) for k, v in init_np.items()} if init_np else None,
                   gf_np)
    errs = {}
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        errs[k] = slice_err(g[k].double().cpu().numpy(), r[k], AXES[k])
    gA, rA = g["A"].double().cpu().numpy(), r["A"]
    den = np.max(np.abs(rA))          # 0 when no decay reaches a loss term (T = 1, fresh state)
    errs["A"] = float(np.max(np.abs(gA - rA)) / den) if den > 0 else float(np.max(np.abs(gA)))
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
    assert capi.m3_ssm_prefill_backward_workspace_bytes(mixer.make_shape(b, T, H, P, N, R, torch_io(io))) > 0, \
        f"every shape of the tile set is compiled: N{N} P{P} R{R} {io}"
    errs = _run(b, T, H, P, N, R, io, seed=4000 + seed, with_init=with_init)
    print(f"case {seed}: N{N} P{P} R{R} {io} b{b} H{H} T{T} init={with_init}: "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"case {seed}: gradient of {k}: error {v:.3e}"


@pytest.mark.parametrize("N,P,R,io,T", [
    (16, 16, 1, "f32", 150), (64, 32, 3, "f32", 64), (128, 32, 2, "f32", 1),
    (64, 64, 4, "bf16", 200), (32, 64, 2, "bf16", 63),
])
@pytest.mark.parametrize("with_init", [False, True])
def test_backward_final_state_gradient(N, P, R, io, T, with_init):
    """An incoming gradient of every part of the final state (h, angle,
    previous B and x) adds <gfinal, final state> to the loss."""
    errs = _run(2, T, 2, P, N, R, io, seed=7 * N + P + R + T, with_init=with_init, with_gfinal=True)
    print(f"backward+gfinal N{N} P{P} R{R} {io} T{T} init={with_init}: "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"


@pytest.mark.parametrize("N,P,R,io,T1,T2,handoff", [
    (32, 32, 2, "f32", 100, 90, "prefill"), (64, 64, 4, "f32", 64, 137, "prefill"),
    (16, 16, 1, "f32", 1, 70, "prefill"), (64, 64, 4, "bf16", 7, 137, "decode"),
    (128, 32, 3, "bf16", 5, 64, "decode"),
])
def test_backward_chains_over_split_calls(N, P, R, io, T1, T2, handoff):
    """A sequence run as two calls (the second starts from the first's final
    state): the second call's backward gives the gradient of its initial state,
    which flows into the first call's backward as the final-state gradient.
    The gradients of both halves and of the first call's initial state match
    the oracle's gradients of the whole sequence.

    The state handed over is part of the second call's input, so it must be
    as exact as the backward's bar: it comes from the prefill at fp32 I/O, and
    from decode steps (fp32 arithmetic) at bf16 I/O -- the bf16 prefill's
    products run on bf16 MFMA and its state carries the forward's bf16 error."""
    from mamba_selective_ssm_ssd_amd import mixer
    b, H, T = 2, 2, T1 + T2
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=T1 * T2, cfg=91)
    d["A"] *= 0.2
    rng = np.random.default_rng(T1 + 31 * T2)
    gy = synth.round_io(rng.standard_normal((b, T, H, R, P)), io)
    init_np = dict(h0=rng.standard_normal((b, H, N, P)).astype(np.float32) * 0.5,
                   phi0=rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32),
                   prevB0=rng.standard_normal((b, H, R, N)).astype(np.float32),
                   prevx0=synth.round_io(rng.standard_normal((b, H, R, P)), io))
    st0 = mixer.State(*(torch.from_numpy(init_np[k]).cuda() for k in ("h0", "phi0", "prevB0")),
                      torch.from_numpy(init_np["prevx0"]).to("cuda", torch_io(io)))
    t = to_dev(d, io)
    names = ("x", "dt", "A", "lam", "theta", "B", "C")
    half = [{k: (t[k] if k == "A" else t[k][:, lo:hi].contiguous()) for k in names}
            for lo, hi in ((0, T1), (T1, T))]
    gyd = torch.from_numpy(gy).to("cuda", torch_io(io))
    if handoff == "prefill":
        _, st1 = mixer.prefill(*(half[0][k] for k in names), state=st0.clone())   # final in place
    else:
        st1 = st0.clone()
        for i in range(T1):
            mixer.decode_step(*((t[k] if k == "A" else t[k][:, i].contiguous()) for k in names), st1)
    g2 = mixer.backward(*(half[1][k] for k in names), gyd[:, T1:].contiguous(), state=st1)
    g1 = mixer.backward(*(half[0][k] for k in names), gyd[:, :T1].contiguous(), state=st0,
                        gfinal={k: g2[k] for k in ("h", "phi", "prev_B", "prev_x")})
    torch.cuda.synchronize()
    _, r = ob.grad(d, gy, {k: v.astype(np.float64) for k, v in init_np.items()})
    errs = {}
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        gk = torch.cat([g1[k], g2[k]], dim=1).double().cpu().numpy()
        errs[k] = slice_err(gk, r[k], AXES[k])
    gA, rA = (g1["A"] + g2["A"]).double().cpu().numpy(), r["A"]
    errs["A"] = float(np.max(np.abs(gA - rA)) / np.max(np.abs(rA)))
    for k, rk in (("h", "g_h0"), ("phi", "g_phi0"), ("prev_B", "g_prevB0"), ("prev_x", "g_prevx0")):
        errs[k] = slice_err(g1[k].double().cpu().numpy(), r[rk], AXES[k])
    print(f"split N{N} P{P} R{R} {io} {T1}+{T2}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"


@pytest.mark.parametrize("N,P,R,io,T", [
    (32, 32, 2, "f32", 1000), (64, 64, 4, "bf16", 600), (16, 16, 1, "f32", 2000), (128, 32, 3, "bf16", 500),
])
@pytest.mark.parametrize("with_init", [False, True])
def test_backward_split_sequence(N, P, R, io, T, with_init):
    """One sequence cut into 20 or more segments (one workgroup each): the
    state entering each segment comes from the earlier segments' aggregates,
    the gradient leaving it from the later segments' adjoint aggregates, and
    the dtheta suffix sums and the boundary tokens' delta gradients are
    completed afterwards.  With a carried state the incoming final-state
    gradients are given too, so every cross-segment term is exercised."""
    from mamba_selective_ssm_ssd_amd import capi, mixer
    rc, S, L = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(1, T, 1, P, N, R, torch_io(io)))
    assert rc == capi.M3_OK and S >= 20, (S, L)
    errs = _run(1, T, 1, P, N, R, io, seed=11 * R + T, with_init=with_init, with_gfinal=with_init)
    print(f"split backward N{N} P{P} R{R} {io} T{T} ({S} segments of {L} tokens) init={with_init}: "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"


@pytest.mark.parametrize("T", [512, 480])
def test_backward_split_with_aggregate_pieces(T):
    """32 sequences of 64 (T = 512) or 60 (T = 480) chunks of 8 tokens: 8
    segments each, whose aggregates are cut into 4 pieces so that their launch
    (2 x 7 x 32 x 4 = 1792 workgroups) fills whole rounds of the compute
    units; with T = 480 the last segment is half as long and its last pieces
    are empty.  Carried state and final-state gradients included."""
    from mamba_selective_ssm_ssd_amd import capi, mixer
    rc, S, L = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(1, T, 32, 64, 64, 4, torch.bfloat16))
    assert rc == capi.M3_OK and (S, L) == (8, 64)
    errs = _run(1, T, 32, 64, 64, 4, "bf16", seed=T, with_init=True, with_gfinal=True)
    print(f"split backward with pieces T{T}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"


def test_backward_at_the_largest_accepted_head_count():
    """SISO N128 P64 with the largest head count the shape check accepts
    (262143 heads, T = 64): the whole batch runs on the GPU, and the first,
    middle and last heads (whose 32-bit in-chunk offsets are the largest)
    match the oracle's gradients."""
    from mamba_selective_ssm_ssd_amd import capi, mixer
    H, N, P, R, T = 2 ** 31 // (64 * 1 * 128) - 1, 128, 64, 1, 64
    assert capi.m3_ssm_prefill_backward_workspace_bytes(mixer.make_shape(1, T, H, P, N, R, torch.bfloat16)) > 0
    inp = synth.torch_inputs(1, T, H, P, N, R, io="bf16", seed=5)
    g = torch.Generator(device="cuda")
    g.manual_seed(55)
    gy = torch.randn(inp["x"].shape, generator=g, device="cuda").to(torch.bfloat16)
    names = ("x", "dt", "A", "lam", "theta", "B", "C")
    grads = mixer.backward(*(inp[k] for k in names), gy)
    torch.cuda.synchronize()
    for hi in (0, H // 2, H - 1):
        d = {k: inp[k][:, :, hi:hi + 1].float().cpu().numpy() for k in names if k != "A"}
        d["A"] = inp["A"][hi:hi + 1].cpu().numpy()
        _, r = ob.grad(d, gy[:, :, hi:hi + 1].float().cpu().numpy())
        errs = {k: slice_err(grads[k][:, :, hi:hi + 1].double().cpu().numpy(), r[k], AXES[k])
                for k in ("x", "dt", "lam", "theta", "B", "C")}
        print(f"backward H={H} head {hi}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= BAR, f"head {hi}: gradient of {k}: error {v:.3e}"
    del inp, gy, grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("split", [False, True])
def test_backward_adjoint_through_borrowed_lds(R, split):
    """At N = 128, P = 64 the updated adjoint state reaches the second wave
    group through LDS areas the chunk no longer reads (no room for a buffer
    of its own): every rank, a carried state and final-state gradients, in
    one workgroup per sequence and cut into segments."""
    from mamba_selective_ssm_ssd_amd import capi, mixer
    N, P = 128, 64
    io = "bf16" if R % 2 else "f32"
    # without a split: three chunks (32 / R tokens each, 10 for R = 3) and a
    # ragged tail, too few to cut into segments of two chunks or more
    b, H, T = (1, 1, 700) if split else (2, 2, 3 * (32 // R) - 2)
    rc, S, L = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(b, T, H, P, N, R, torch_io(io)))
    assert rc == capi.M3_OK and (S > 1) == split, (S, L)
    errs = _run(b, T, H, P, N, R, io, seed=13 * R + T, with_init=True, with_gfinal=True)
    print(f"backward N{N} P{P} R{R} {io} T{T} ({S} segments): "
          + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= BAR, f"gradient of {k}: error {v:.3e} > {BAR}"
