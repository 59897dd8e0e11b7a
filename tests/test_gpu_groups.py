"""GPU parity of B/C shared by head groups (G groups of H/G consecutive heads;
the shared B, C projection of the Mamba-3 review, section 3.3) against the
oracle, which expands the groups to heads: prefill over several chunks with a
ragged tail, SISO and MIMO, both I/O types, one and several segments,
carried state, decode, and the block prologue on grouped B/C."""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import synth
from _helpers import TOL, check_final_state, run_gpu_prefill, run_oracle, slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _inputs(b, T, H, P, N, R, io, G, seed):
    return synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=70, G=G)


def _parity(d, io, init=None, init_np=None):
    y, st = run_gpu_prefill(d, io, init=init)
    yr, hT, phiT = run_oracle(d, init_np)
    e = slice_err(y, yr, (0, 2))
    assert e <= TOL[io], f"y error {e:.3e}"
    check_final_state(st, d, hT, phiT, io, TOL[io])


@pytest.mark.parametrize("N,P,R,io,H,G", [
    (128, 64, 1, "bf16", 4, 1),
    (64, 64, 4, "bf16", 4, 2),
    (128, 64, 1, "f32", 6, 3),
    (64, 64, 2, "f32", 4, 1),
    (32, 32, 3, "bf16", 6, 2),
    (16, 16, 1, "f32", 3, 1),
    (64, 32, 2, "bf16", 8, 8),
])
def test_groups_prefill(N, P, R, io, H, G):
    d = _inputs(2, 300, H, P, N, R, io, G, seed=N + P + R + G)
    _parity(d, io)


def test_groups_segmented_long_sequence():
    d = _inputs(1, 1500, 4, 32, 64, 4, "bf16", 2, seed=71)
    d["A"] *= 0.01
    _parity(d, "bf16")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_groups_split_prefill_then_decode(io):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R, G = 2, 150, 4, 64, 64, 2, 2
    d = _inputs(b, T, H, P, N, R, io, G, seed=72)
    d["A"] *= 0.05
    yr, hT, phiT = run_oracle(d)
    T1, T2 = 70, 131
    cut = lambda a, c: {k: (v[:, a:c] if v.ndim >= 3 else v) for k, v in d.items()}
    y1, st = run_gpu_prefill(cut(0, T1), io)
    y2, st = run_gpu_prefill(cut(T1, T2), io, init=st)
    t = to_dev(d, io)
    ys = [y1, y2]
    for s in range(T2, T):
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")), st)
        ys.append(y.double().cpu().numpy()[:, None])
    assert slice_err(np.concatenate(ys, axis=1), yr, (0, 2)) <= TOL[io]
    check_final_state(st, d, hT, phiT, io, TOL[io])


@pytest.mark.parametrize("N,P,R,io,H,G", [
    (16, 16, 1, "bf16", 4, 1), (64, 64, 4, "bf16", 8, 2), (128, 32, 2, "f32", 6, 3),
    (32, 64, 3, "f32", 5, 1),
])
def test_groups_decode(N, P, R, io, H, G):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T = 3, 10
    d = _inputs(b, T, H, P, N, R, io, G, seed=73 + N)
    t = to_dev(d, io)
    st = mixer.State.zeros(b, H, N, P, R, torch_io(io))
    ys = []
    for s in range(T):
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")), st)
        ys.append(y.double().cpu().numpy()[:, None])
    yr, hT, phiT = run_oracle(d)
    assert slice_err(np.concatenate(ys, axis=1), yr, (0, 2)) <= TOL[io]
    check_final_state(st, d, hT, phiT, io, TOL[io])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_groups_with_block(io):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R, G = 2, 200, 4, 32, 64, 2, 2
    d = _inputs(b, T, H, P, N, R, io, G, seed=74)
    bp = synth.block_inputs(b, T, H, P, N, R, io=io, seed=74, cfg=70)
    t = to_dev(d, io)
    dev = {k: torch.from_numpy(bp[k]).cuda() for k in ("B_weight", "B_bias", "C_weight", "C_bias")}
    z = torch.from_numpy(bp["z"]).to("cuda", torch_io(io))
    y, st = mixer.prefill(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")),
                          block=mixer.Block(bc_norm=True, eps=1e-6, **dev), z=z)
    blk = dict(bc_norm=True, eps=1e-6, z=bp["z"], **{k: bp[k] for k in dev})
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=blk)
    assert slice_err(y.double().cpu().numpy(), yr, (0, 2)) <= TOL[io]
    phiT = oracle.cumulative_angle(d["theta"])
    eh = slice_err(oracle.state_to_true(st.h.double().cpu().numpy(), phiT), hT, (0, 1))
    assert eh <= TOL[io]


def test_groups_siso_full_size_one_group():
    """The SISO workload (b4 T2048 H64 P64 N128, bf16) with one B/C group for
    all 64 heads, sampled (batch, head) instances against the oracle."""
    from mamba_selective_ssm_ssd_amd import mixer
    c = synth.CONFIGS[1]
    b, T, H, P, N, R = (c[k] for k in ("batch", "T", "H", "P", "N", "R"))
    inp = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0, G=1)
    y, st = mixer.prefill(*(inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")))
    torch.cuda.synchronize()
    for bi, hi in [(0, 0), (1, 33), (3, 63)]:
        d = {k: inp[k][bi:bi + 1, :, hi:hi + 1].float().cpu().numpy() for k in ("x", "dt", "lam", "theta")}
        for k in ("B", "C"):
            d[k] = inp[k][bi:bi + 1].float().cpu().numpy()          # the one group
        d["A"] = inp["A"][hi:hi + 1].cpu().numpy()
        yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"])
        e = slice_err(y[bi:bi + 1, :, hi:hi + 1].double().cpu().numpy(), yr, (0, 2))
        print(f"groups G=1 full size (b={bi}, h={hi}): y err {e:.2e}")
        assert e <= TOL["bf16"]
