"""m3_ssm_prefill_noalloc (include/m3_ssm_noalloc.h), which takes its
workspace from the library's static per-device array, against m3_ssm_prefill
with a caller-provided workspace: two calls in a row, the second on a
smaller input, both cutting their sequences into segments (so the array is
used), the second from a carried state."""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import capi, synth
from _helpers import TOL, check_final_state, gpu_state, run_oracle, slice_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(t, io, init=None):
    from mamba_selective_ssm_ssd_amd import mixer
    x = t["x"]
    b, T, H, R, P = x.shape
    N = t["B"].shape[-1]
    tio = x.dtype
    shape = mixer.make_shape(b, T, H, P, N, R, tio)
    need = capi.m3_ssm_prefill_workspace_bytes(shape)
    assert 256 < need <= capi.M3_NOALLOC_SCRATCH_BYTES      # segments: the array is used
    y = torch.full_like(x, float("nan"))
    st = mixer.State.zeros(b, H, N, P, R, tio)
    st.h.fill_(float("nan"))
    rc = capi.m3_ssm_prefill_noalloc(shape, *(t[k].data_ptr() for k in ("x", "dt", "A", "lam", "theta", "B", "C")),
                                     init.c() if init is not None else None, st.c(), y.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == capi.M3_OK, capi.m3_status_string(rc)
    return y, st


def _reference(t, init=None):
    from mamba_selective_ssm_ssd_amd import mixer
    return mixer.prefill(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")),
                         state=init.clone() if init is not None else None,
                         final=None if init is not None else None)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_matches_prefill_two_calls(io):
    d1 = synth.prefill_inputs(1, 1500, 2, 64, 64, 4, io=io, seed=1, cfg=60)
    d1["A"] *= 0.05
    t1 = to_dev(d1, io)
    y1, st1 = _noalloc(t1, io)
    y1r, st1r = _reference(t1)
    torch.cuda.synchronize()
    # same kernels on the same inputs: identical results
    assert torch.equal(y1, y1r)
    assert torch.equal(st1.h, st1r.h) and torch.equal(st1.phi, st1r.phi)
    assert torch.equal(st1.prev_B, st1r.prev_B) and torch.equal(st1.prev_x, st1r.prev_x)
    # and both match the oracle
    yr, hT, phiT = run_oracle(d1)
    assert slice_err(y1.double().cpu().numpy(), yr, (0, 2)) <= TOL[io]
    check_final_state(st1, d1, hT, phiT, io, TOL[io])

    # second call: a smaller input (fewer tokens, more heads, N = 32), from a
    # carried state; the array still holds the first call's contents
    d2 = synth.prefill_inputs(1, 700, 3, 32, 32, 2, io=io, seed=2, cfg=60)
    d2["A"] *= 0.05
    t2 = to_dev(d2, io)
    from mamba_selective_ssm_ssd_amd import mixer
    rng = np.random.default_rng(61)
    init_np = dict(h=rng.standard_normal((1, 3, 32, 32)).astype(np.float32),
                   phi=rng.uniform(-np.pi, np.pi, size=(1, 3, 16)).astype(np.float32),
                   prev_B=rng.standard_normal((1, 3, 2, 32)).astype(np.float32),
                   prev_x=synth.round_io(rng.standard_normal((1, 3, 2, 32)), io))
    tio = torch.float32 if io == "f32" else torch.bfloat16
    init = mixer.State(*(torch.from_numpy(init_np[k]).cuda() for k in ("h", "phi", "prev_B")),
                       torch.from_numpy(init_np["prev_x"]).to("cuda", tio))
    y2, st2 = _noalloc(t2, io, init=init)
    y2r, st2r = _reference(t2, init=init)
    torch.cuda.synchronize()
    assert torch.equal(y2, y2r)
    assert torch.equal(st2.h, st2r.h) and torch.equal(st2.phi, st2r.phi)
    init_keep = {k: v.astype(np.float64) for k, v in init_np.items()}
    yr2, hT2, phiT2 = run_oracle(d2, init_keep)
    assert slice_err(y2.double().cpu().numpy(), yr2, (0, 2)) <= TOL[io]
    check_final_state(st2, d2, hT2, phiT2, io, TOL[io])
