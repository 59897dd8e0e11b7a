"""Seeded random configurations through the whole C ABI against the oracle:
shape (N, P, R, T, batch, heads), I/O type, B/C head groups, a random carried
state, block pieces, and a prefill split followed by decode steps.  Each case
is drawn from a fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import synth
from _helpers import TOL, oracle_init_from_rot, slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PIECES = ("bc_norm", "B_weight", "B_bias", "C_weight", "C_bias", "z")


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.choice([16, 32, 64, 128]))
    P = int(rng.choice([16, 32, 64]))
    R = int(rng.integers(1, 5))
    io = str(rng.choice(["f32", "bf16"]))
    H = int(rng.integers(1, 7))
    G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
    b = int(rng.integers(1, 4))
    T = int(rng.integers(1, 400))
    T1 = int(rng.integers(0, T))               # prefill T1 tokens (0: decode only) ...
    T2 = min(T - T1, int(rng.integers(0, 6)))   # ... then decode T2 steps, prefill the rest
    pieces = tuple(p for p in PIECES if rng.random() < 0.3)
    with_init = bool(rng.random() < 0.5)
    return dict(N=N, P=P, R=R, io=io, H=H, G=G, b=b, T=T, T1=T1, T2=T2, pieces=pieces,
                with_init=with_init)


def _supported(c):
    from mamba_selective_ssm_ssd_amd import capi, mixer
    sh = mixer.make_shape(c["b"], c["T"], c["H"], c["P"], c["N"], c["R"], torch_io(c["io"]), G=c["G"])
    if capi.m3_ssm_prefill_workspace_bytes(sh) == 0:
        return False
    if c["pieces"]:
        blk = capi.m3_block_t(1, 1e-6)
        F = 0x10000
        rc = capi.m3_ssm_prefill_block(sh, F, F, F, F, F, F, F, blk, None, None, F, F, 0, None)
        return rc == capi.M3_ERR_WORKSPACE
    return True


@pytest.mark.parametrize("seed", range(24))
def test_random_case(seed):
    from mamba_selective_ssm_ssd_amd import mixer
    c = _case(seed)
    print("case", seed, c)
    assert _supported(c), f"every shape of the tile set is compiled: {c}"
    N, P, R, io, H, G, b, T = (c[k] for k in ("N", "P", "R", "io", "H", "G", "b", "T"))
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=97, G=G)
    bp = synth.block_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=97)
    rng = np.random.default_rng(2000 + seed)
    init_np, st = None, None
    if c["with_init"]:
        init_np = dict(h=(rng.standard_normal((b, H, N, P)) * 0.3).astype(np.float32),
                       phi=rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32),
                       prev_B=rng.standard_normal((b, H, R, N)).astype(np.float32),
                       prev_x=synth.round_io(rng.standard_normal((b, H, R, P)), io))
        st = mixer.State(*(torch.from_numpy(init_np[k]).cuda() for k in ("h", "phi", "prev_B")),
                         torch.from_numpy(init_np["prev_x"]).to("cuda", torch_io(io)))
    else:
        st = mixer.State.zeros(b, H, N, P, R, torch_io(io))
    t = to_dev(d, io)
    dev = {k: torch.from_numpy(bp[k]).cuda() for k in ("B_weight", "B_bias", "C_weight", "C_bias")
           if k in c["pieces"]}
    block = mixer.Block(bc_norm="bc_norm" in c["pieces"], eps=1e-6, **dev) if c["pieces"] else None
    zfull = torch.from_numpy(bp["z"]).to("cuda", torch_io(io)) if "z" in c["pieces"] else None
    names = ("x", "dt", "A", "lam", "theta", "B", "C")
    ys = []
    T1, T2 = c["T1"], c["T2"]
    spans = [("p", 0, T1), ("d", T1, T1 + T2), ("p", T1 + T2, T)]
    for kind, a, e in spans:
        if e <= a:
            continue
        if kind == "p":
            # slices are copied: a batch-1 slice is contiguous but may be misaligned
            y, st = mixer.prefill(*(t[k][:, a:e].clone() if k != "A" else t[k] for k in names),
                                  state=st, block=block,
                                  z=zfull[:, a:e].clone() if zfull is not None else None)
            ys.append(y.double().cpu().numpy())
        else:
            for s in range(a, e):
                y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k] for k in names), st,
                                      block=block, z=zfull[:, s].clone() if zfull is not None else None)
                ys.append(y.double().cpu().numpy()[:, None])
    yg = np.concatenate(ys, axis=1)
    blk = dict(bc_norm="bc_norm" in c["pieces"], eps=1e-6)
    for k in ("B_weight", "B_bias", "C_weight", "C_bias", "z"):
        if k in c["pieces"]:
            blk[k] = bp[k]
    kw, phi0 = {}, None
    if init_np is not None:
        kw = oracle_init_from_rot(init_np["h"], init_np["phi"], init_np["prev_B"], init_np["prev_x"])
        phi0 = init_np["phi"]
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                                 block=blk, **kw)
    phiT = oracle.cumulative_angle(d["theta"], phi0)
    ey = slice_err(yg, yr, (0, 2))
    eh = slice_err(oracle.state_to_true(st.h.double().cpu().numpy(), phiT), hT, (0, 1))
    print(f"case {seed}: y err {ey:.2e}, state err {eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io], f"case {seed} {c}: y {ey:.3e}, state {eh:.3e}"
