"""A carried state h~ stored in bf16 (every store rounded to nearest even, all
arithmetic fp32), studied against the fp64 oracle.  Decode is bound by the
state's read-modify-write, so halving its bytes is the lever.  How
quantising the complex recurrent state affects it is left open by the
"20.2 Mamba and S6" page (sungeuns.github.io), section 7 (open questions),
so the bar here is a reading: 2e-2 per (b, h) slice, the bar of bf16 I/O,
for outputs and final states, over short and 1000-step runs, with the
measured errors printed.  The oracle starts from the bf16 values the GPU
state holds.
"""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import synth
from _helpers import TOL, oracle_init_from_rot, slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BAR = 2e-2


def _bf16_state(b, H, N, P, R, io, seed, std=0.1):
    """Random carried state with h~ in bf16 (GPU State, and fp64 copies)."""
    from mamba_selective_ssm_ssd_amd import mixer
    rng = np.random.default_rng(seed)
    h = synth.round_io(rng.standard_normal((b, H, N, P)) * std, "bf16")
    phi = rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32)
    pB = (rng.standard_normal((b, H, R, N)) * 0.5).astype(np.float32)
    px = synth.round_io(rng.standard_normal((b, H, R, P)), io)
    st = mixer.State(torch.from_numpy(h).to("cuda", torch.bfloat16), torch.from_numpy(phi).cuda(),
                     torch.from_numpy(pB).cuda(), torch.from_numpy(px).to("cuda", torch_io(io)))
    return st, dict(h=h.astype(np.float64), phi=phi.astype(np.float64), prev_B=pB.astype(np.float64),
                    prev_x=px.astype(np.float64))


def _decode(d, io, st, t0, t1):
    from mamba_selective_ssm_ssd_amd import mixer
    t = to_dev(d, io)
    ys = []
    for s in range(t0, t1):
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")), st)
        ys.append(y.double().cpu().numpy()[:, None])
    return np.concatenate(ys, axis=1)


def _state_err(st, hT, phiT):
    h = st.h.double().cpu().numpy()
    return slice_err(oracle.state_to_true(h, phiT), hT, (0, 1))


@pytest.mark.parametrize("N,P,R,io", [
    (64, 64, 4, "bf16"), (128, 64, 1, "bf16"), (16, 16, 2, "f32"), (32, 64, 3, "f32"), (128, 32, 2, "bf16"),
])
def test_bf16_state_decode(N, P, R, io):
    b, T, H = 2, 64, 3
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=N + R, cfg=80)
    st, init = _bf16_state(b, H, N, P, R, io, seed=800 + N)
    yg = _decode(d, io, st, 0, T)
    kw = oracle_init_from_rot(init["h"], init["phi"], init["prev_B"], init["prev_x"])
    yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], **kw)
    phiT = oracle.cumulative_angle(d["theta"], init["phi"])
    ey, eh = slice_err(yg, yr, (0, 2)), _state_err(st, hT, phiT)
    print(f"bf16 state decode N{N} P{P} R{R} {io}: y err {ey:.2e}, state err {eh:.2e}")
    assert st.h.dtype == torch.bfloat16
    assert ey <= BAR and eh <= BAR


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_bf16_state_prefill_then_decode(io):
    """Prefill from a bf16 carried state into a bf16 final state (one and
    several segments), then decode on from it."""
    from mamba_selective_ssm_ssd_amd import mixer
    for (b, H, T) in ((2, 3, 150), (1, 2, 700)):       # the second is cut into segments
        N, P, R = 64, 32, 2
        d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=T, cfg=81)
        d["A"] *= 0.05
        st, init = _bf16_state(b, H, N, P, R, io, seed=810 + T)
        T1 = T - 20
        t = to_dev({k: (v[:, :T1] if v.ndim >= 3 else v) for k, v in d.items()}, io)
        y1, st2 = mixer.prefill(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")), state=st)
        assert st2 is st and st.h.dtype == torch.bfloat16
        y2 = _decode(d, io, st, T1, T)
        kw = oracle_init_from_rot(init["h"], init["phi"], init["prev_B"], init["prev_x"])
        yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], **kw)
        phiT = oracle.cumulative_angle(d["theta"], init["phi"])
        ey = slice_err(np.concatenate([y1.double().cpu().numpy(), y2], axis=1), yr, (0, 2))
        eh = _state_err(st, hT, phiT)
        print(f"bf16 state prefill+decode b{b} H{H} T{T} {io}: y err {ey:.2e}, state err {eh:.2e}")
        assert ey <= BAR and eh <= BAR


def test_bf16_state_fresh_prefill_final():
    """A fresh prefill that writes its final state in bf16 equals the fp32
    final state rounded to bf16 (same kernel arithmetic, one rounding)."""
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R = 2, 200, 3, 64, 128, 1
    d = synth.prefill_inputs(b, T, H, P, N, R, io="bf16", seed=3, cfg=82)
    t = to_dev(d, "bf16")
    args = [t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")]
    y32, s32 = mixer.prefill(*args)
    y16, s16 = mixer.prefill(*args, state_dtype=torch.bfloat16)
    assert torch.equal(y32, y16)
    assert s16.h.dtype == torch.bfloat16
    assert torch.equal(s16.h, s32.h.to(torch.bfloat16))
    assert torch.equal(s16.phi, s32.phi) and torch.equal(s16.prev_B, s32.prev_B)


def test_bf16_state_long_decode_error_stays_bounded():
    """1000 decode steps of the MIMO decode shape (P64 N64 R4, bf16 I/O) on
    a few (b, h): the error of the bf16 state does not grow with the steps."""
    from mamba_selective_ssm_ssd_amd import mixer
    b, H, P, N, R, steps = 2, 4, 64, 64, 4, 1000
    d = synth.prefill_inputs(b, steps, H, P, N, R, io="bf16", seed=9, cfg=83)
    st, init = _bf16_state(b, H, N, P, R, "bf16", seed=830)
    yg = _decode(d, "bf16", st, 0, steps)
    kw = oracle_init_from_rot(init["h"], init["phi"], init["prev_B"], init["prev_x"])
    yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], **kw)
    errs = [slice_err(yg[:, s:s + 100], yr[:, s:s + 100], (0, 2)) for s in range(0, steps, 100)]
    eh = _state_err(st, hT, oracle.cumulative_angle(d["theta"], init["phi"]))
    print("bf16 state, 1000 steps: y err per 100 steps " + " ".join(f"{e:.1e}" for e in errs)
          + f"; final state err {eh:.2e}")
    assert max(errs) <= BAR and eh <= BAR
    assert max(errs[5:]) <= 2 * max(errs[:5])


def test_bf16_state_decode_with_block_and_groups():
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R, G = 2, 40, 4, 32, 64, 2, 2
    d = synth.prefill_inputs(b, T, H, P, N, R, io="bf16", seed=11, cfg=84, G=G)
    bp = synth.block_inputs(b, T, H, P, N, R, io="bf16", seed=11, cfg=84)
    st = mixer.State.zeros(b, H, N, P, R, torch.bfloat16, state_dtype=torch.bfloat16)
    t = to_dev(d, "bf16")
    dev = {k: torch.from_numpy(bp[k]).cuda() for k in ("B_weight", "B_bias", "C_weight", "C_bias")}
    z = torch.from_numpy(bp["z"]).to("cuda", torch.bfloat16)
    blk = mixer.Block(bc_norm=True, eps=1e-6, **dev)
    ys = []
    for s in range(T):
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")), st,
                              block=blk, z=z[:, s].clone())
        ys.append(y.double().cpu().numpy()[:, None])
    ob = dict(bc_norm=True, eps=1e-6, z=bp["z"], **{k: bp[k] for k in dev})
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=ob)
    ey = slice_err(np.concatenate(ys, axis=1), yr, (0, 2))
    eh = _state_err(st, hT, oracle.cumulative_angle(d["theta"]))
    assert ey <= BAR and eh <= BAR


def test_bf16_state_decode_full_size():
    """The MIMO decode workload (b256 H64 P64 N64 R4, bf16 I/O), 200 steps with
    a bf16 state from N(0, 0.1), sampled (b, h) against the oracle."""
    from mamba_selective_ssm_ssd_amd import mixer
    c = synth.CONFIGS[4]
    b, H, P, N, R = (c[k] for k in ("batch", "H", "P", "N", "R"))
    steps = 200
    inp = synth.torch_inputs(steps, b, H, P, N, R, io="bf16", seed=4)   # step-major
    st = mixer.State.zeros(b, H, N, P, R, torch.bfloat16, state_dtype=torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(41)
    st.h.copy_((torch.randn(st.h.shape, generator=g, device="cuda") * 0.1).to(torch.bfloat16))
    picks = [(0, 0), (129, 40), (255, 63)]
    h0 = {pk: st.h[pk[0]:pk[0] + 1, pk[1]:pk[1] + 1].double().cpu().numpy() for pk in picks}
    ys = {pk: [] for pk in picks}
    for t in range(steps):
        y = mixer.decode_step(inp["x"][t], inp["dt"][t], inp["A"], inp["lam"][t], inp["theta"][t],
                              inp["B"][t], inp["C"][t], st)
        for pk in picks:
            ys[pk].append(y[pk[0], pk[1]])
    torch.cuda.synchronize()
    for (bi, hi) in picks:
        d = {k: inp[k][:, bi:bi + 1, hi:hi + 1].transpose(0, 1).float().cpu().numpy()
             for k in ("x", "dt", "lam", "theta", "B", "C")}
        d["A"] = inp["A"][hi:hi + 1].cpu().numpy()
        yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], h0=h0[(bi, hi)])
        yg = torch.stack(ys[(bi, hi)]).double().cpu().numpy()[None, :, None]
        e = slice_err(yg, yr, (0, 2))
        eh = slice_err(oracle.state_to_true(st.h[bi:bi + 1, hi:hi + 1].double().cpu().numpy(),
                                            oracle.cumulative_angle(d["theta"])), hT, (0, 1))
        print(f"bf16 state decode full size (b={bi}, h={hi}): y err {e:.2e}, state err {eh:.2e}")
        assert e <= BAR and eh <= BAR
