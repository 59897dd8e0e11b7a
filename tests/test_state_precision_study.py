"""How the storage type of the carried state h~ affects decode, studied on the
CPU with the fp64 oracle (no GPU): 1000 decode steps of the MIMO decode
shape (P64 N64 R4) on 2 x 4 (b, h), with h~ rounded to the storage type after
every step and all arithmetic in fp64.  The error is that of the outputs and
the final state against the unrounded recurrence, max |a - r| / max |r| per
(b, h), the metric of the GPU tests.

Quantising the recurrent state is left open by the "20.2 Mamba and S6" page
(sungeuns.github.io), section 7 (open questions); the bar taken for a stored
state is that of bf16 I/O, 2e-2.  fp32 and bf16 are the two state types the
library builds; fp8 (e4m3 with one scale per state row, per column or per
(b, h), and e5m2 per row) is the study: it fails the bar even at the drawn
decode decay, and by an order of magnitude when the decay is slow, so it is
not built.  The decay matters because each step's rounding error is carried
forward by alpha = exp(dt A): with the drawn A (-16 .. -1) the state forgets
within a few steps, with A x 0.02 it keeps errors for hundreds.
"""
import numpy as np
import pytest

from oracle import backward as ob
from mamba_selective_ssm_ssd_amd import synth

torch = pytest.importorskip("torch")

BAR = 2e-2
STEPS = 1000


def _round_state(h, mode):
    """h~ (fp64) as stored in `mode` and read back."""
    if mode == "f32":
        return h.float().double()
    if mode == "bf16":
        return h.to(torch.bfloat16).double()
    kind, scaling = mode.split("_")
    fmt, fmax = {"e4m3": (torch.float8_e4m3fn, 448.0), "e5m2": (torch.float8_e5m2, 57344.0)}[kind]
    dims = {"row": (-1,), "col": (-2,), "tensor": (-2, -1)}[scaling]   # rows are n, columns p
    s = h.abs().amax(dim=dims, keepdim=True) / fmax
    s = torch.where(s > 0, s, torch.ones_like(s))
    return (h / s).to(fmt).double() * s


def _decode(d, mode):
    """STEPS single-token calls of the rotated-frame recurrence, the state
    rounded after each; returns y [b, T, H, R, P] and the final h~."""
    t = {k: torch.tensor(np.asarray(d[k], dtype=np.float64)) for k in ob.NAMES}
    b, T, H, R, P = t["x"].shape
    N = t["B"].shape[-1]
    z = lambda *s: torch.zeros(*s, dtype=torch.float64)
    h, phi, Bp, xp = z(b, H, N, P), z(b, H, N // 2), z(b, H, R, N), z(b, H, R, P)
    ys = []
    for i in range(T):
        step = [t[k] if k == "A" else t[k][:, i:i + 1] for k in ob.NAMES]
        y, h, phi, Bp, xp = ob.forward_rot(*step, h0=h, phi0=phi, prevB0=Bp, prevx0=xp, final=True)
        if mode != "f64":
            h = _round_state(h, mode)
        ys.append(y)
    return torch.cat(ys, dim=1).numpy(), h.numpy()


def _err(a, r, head_axis):
    return max(float(np.max(np.abs(np.take(a, hh, head_axis)[bb] - np.take(r, hh, head_axis)[bb]))
                     / np.max(np.abs(np.take(r, hh, head_axis)[bb])))
               for bb in range(a.shape[0]) for hh in range(a.shape[head_axis]))


@pytest.fixture(scope="module", params=[1.0, 0.02], ids=["drawn_decay", "slow_decay"])
def study(request):
    d = synth.prefill_inputs(2, STEPS, 4, 64, 64, 4, io="bf16", seed=9, cfg=83)
    d["A"] = (d["A"] * request.param).astype(np.float32)
    yr, hr = _decode(d, "f64")
    out = {}
    for mode in ("f32", "bf16", "e4m3_row", "e4m3_col", "e4m3_tensor", "e5m2_row"):
        y, h = _decode(d, mode)
        out[mode] = (_err(y, yr, 2), _err(h, hr, 1))
    print(f"state storage study ({request.param} x A, {STEPS} steps): "
          + ", ".join(f"{m} y {ey:.1e} h {eh:.1e}" for m, (ey, eh) in out.items()))
    return request.param, out


def test_fp32_state_is_exact_to_fp32(study):
    _, out = study
    ey, eh = out["f32"]
    assert ey <= 1e-6 and eh <= 1e-6


def test_bf16_state_meets_the_bar_at_the_decode_decay(study):
    scale, out = study
    ey, eh = out["bf16"]
    if scale == 1.0:
        assert ey <= BAR and eh <= BAR
    else:
        # slow decay: outputs still within the bar, the stored state itself
        # drifts to about the bar (measured 1.2e-2 and 2.5e-2)
        assert ey <= BAR and eh <= 2 * BAR


def test_fp8_state_fails_the_bar(study):
    """Every fp8 variant misses the bar on the outputs or on the state; with
    slow decay by about 8x or more on the outputs."""
    scale, out = study
    for mode in ("e4m3_row", "e4m3_col", "e4m3_tensor", "e5m2_row"):
        ey, eh = out[mode]
        assert max(ey, eh) > BAR, mode
        if scale != 1.0:
            assert ey > 5 * BAR, mode
    # bf16 is at least 8x closer than the best fp8 scaling
    assert out["bf16"][0] * 8 <= min(out[m][0] for m in ("e4m3_row", "e4m3_col", "e4m3_tensor"))
