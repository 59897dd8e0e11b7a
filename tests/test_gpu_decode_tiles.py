"""Decode step over the whole tile set: every (N, P, R) the library compiles,
with an fp32 and a bf16 carried state, from a random carried state (angle,
previous token and state all nonzero), a few steps against the fp64 oracle.

The decode kernel's work split depends on the shape (threads per workgroup,
state runs per thread and how they are grouped per LDS read of x and x_prev,
resident waves), so each shape exercises its own instantiation.  Bars: the
parity bar of the I/O type with an fp32 state; 2e-2 with a bf16 state (the
state's own rounding; the oracle starts from the bf16 values the GPU state
holds).  The recurrence is the rotated-frame decode step of the Mamba-3
review, section 3.2.2 (Prop. 3.2.3), with the coefficients of section 3.1.1,
eq. (6), and the rank-R update of section 3.3.
"""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import synth
from _helpers import TOL, check_final_state, oracle_init_from_rot, slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TILES = [(N, P) for N in (16, 32, 64, 128) for P in (16, 32, 64)]


def _carried(b, H, N, P, R, io, sbf16, seed):
    """Random carried state: GPU State and its fp64 values."""
    from mamba_selective_ssm_ssd_amd import mixer
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((b, H, N, P)) * 0.1
    h = synth.round_io(h, "bf16") if sbf16 else h.astype(np.float32)
    phi = rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32)
    pB = (rng.standard_normal((b, H, R, N)) * 0.5).astype(np.float32)
    px = synth.round_io(rng.standard_normal((b, H, R, P)), io)
    st = mixer.State(torch.from_numpy(np.ascontiguousarray(h)).to("cuda", torch.bfloat16 if sbf16 else torch.float32),
                     torch.from_numpy(phi).cuda(), torch.from_numpy(pB).cuda(),
                     torch.from_numpy(px).to("cuda", torch_io(io)))
    return st, dict(h=h.astype(np.float64), phi=phi.astype(np.float64), prev_B=pB.astype(np.float64),
                    prev_x=px.astype(np.float64))


@pytest.mark.parametrize("N,P", TILES)
@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_decode_tile_set(N, P, R, state):
    from mamba_selective_ssm_ssd_amd import mixer
    io = "f32" if (N // 16 + P // 16 + R) % 2 == 0 else "bf16"
    sbf16 = state == "bf16"
    b, T, H = 2, 5, 3
    seed = 7 * N + 3 * P + R + (1000 if sbf16 else 0)
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=81)
    st, init = _carried(b, H, N, P, R, io, sbf16, seed)
    t = to_dev(d, io)
    ys = []
    for s in range(T):
        # per-step slices are copied: a slice of a batch is not contiguous
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")), st)
        ys.append(y.double().cpu().numpy()[:, None])
    torch.cuda.synchronize()
    yg = np.concatenate(ys, axis=1)
    kw = oracle_init_from_rot(init["h"], init["phi"], init["prev_B"], init["prev_x"])
    yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], **kw)
    phiT = oracle.cumulative_angle(d["theta"], init["phi"])
    bar = 2e-2 if sbf16 else TOL[io]
    ey = slice_err(yg, yr, (0, 2))
    assert st.h.dtype == (torch.bfloat16 if sbf16 else torch.float32)
    eh, _, _ = check_final_state(st, d, hT, phiT, io, bar)
    print(f"decode N{N} P{P} R{R} io {io} state {state}: y err {ey:.2e}, state err {eh:.2e}")
    assert ey <= bar, f"y error {ey:.3e} > {bar}"
