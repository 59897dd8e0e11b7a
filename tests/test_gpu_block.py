"""GPU parity of the block prologue/epilogue (Mamba-3 review, section 3.4:
BC normalisation, per-head per-channel B/C biases, output gate) fused into the
mixer's kernels, against the oracle's ``run_block`` on the same seeded inputs:
every piece alone and all together, SISO and MIMO, both I/O dtypes, several
chunks with a ragged tail, segmented sequences, carried state, prefill then
decode, decode over the (N, P, R) tile set, and a full-size sampled check.
"""
import numpy as np
import pytest

import oracle
from mamba_selective_ssm_ssd_amd import synth
from _helpers import TOL, gpu_state, oracle_init_from_rot, slice_err, to_dev, torch_io

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALL = ("bc_norm", "B_weight", "B_bias", "C_weight", "C_bias", "z")
EPS = 1e-6


def _draw(b, T, H, P, N, R, io, seed):
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=60)
    bp = synth.block_inputs(b, T, H, P, N, R, io=io, seed=seed, cfg=60)
    return d, bp


def _oracle_block(bp, pieces):
    blk = dict(bc_norm="bc_norm" in pieces, eps=EPS)
    for k in ("B_weight", "B_bias", "C_weight", "C_bias", "z"):
        if k in pieces:
            blk[k] = bp[k]
    return blk


def _gpu_block(bp, pieces, io):
    from mamba_selective_ssm_ssd_amd import mixer
    dev = {k: torch.from_numpy(np.ascontiguousarray(bp[k])).cuda()
           for k in ("B_weight", "B_bias", "C_weight", "C_bias") if k in pieces}
    block = mixer.Block(bc_norm="bc_norm" in pieces, eps=EPS, **dev)
    z = (torch.from_numpy(np.ascontiguousarray(bp["z"])).to("cuda", torch_io(io))
         if "z" in pieces else None)
    return block, z


def _check_state(st, d, bp, blk, hT, phiT, io):
    g = gpu_state(st)
    e_h = slice_err(oracle.state_to_true(g["h"], phiT), hT, (0, 1))
    e_phi = float(np.max(np.abs(oracle.wrap_angle(g["phi"] - phiT))))
    B_last = oracle.bc_norm(oracle.heads_from_groups(d["B"][:, -1], d["x"].shape[2], axis=1),
                            blk.get("B_weight"), blk.get("B_bias"), EPS, blk["bc_norm"])
    e_B = slice_err(oracle.prevB_to_true(g["prev_B"], phiT), B_last, (0, 1))
    assert np.array_equal(g["prev_x"], d["x"][:, -1].astype(np.float64))
    assert e_h <= TOL[io], f"final state error {e_h:.3e}"
    assert e_phi <= 1e-4, f"final angle error {e_phi:.3e}"
    assert e_B <= (1e-4 if io == "f32" else 1e-3), f"prev_B error {e_B:.3e}"


def _parity(d, bp, pieces, io, init=None, init_np=None):
    from mamba_selective_ssm_ssd_amd import mixer
    t = to_dev(d, io)
    block, z = _gpu_block(bp, pieces, io)
    y, st = mixer.prefill(t["x"], t["dt"], t["A"], t["lam"], t["theta"], t["B"], t["C"],
                          state=init, block=block, z=z)
    yg = y.double().cpu().numpy()
    blk = _oracle_block(bp, pieces)
    kw, phi0 = {}, None
    if init_np is not None:
        kw = oracle_init_from_rot(init_np["h"], init_np["phi"], init_np["prev_B"], init_np["prev_x"])
        phi0 = init_np["phi"]
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                                 block=blk, **kw)
    phiT = oracle.cumulative_angle(d["theta"], phi0)
    e_y = slice_err(yg, yr, (0, 2))
    assert e_y <= TOL[io], f"y error {e_y:.3e} > {TOL[io]}"
    _check_state(st, d, bp, blk, hT, phiT, io)
    return e_y


@pytest.mark.parametrize("N,P,R,io", [
    (128, 64, 1, "bf16"),   # SISO workload shape
    (64, 64, 4, "bf16"),    # MIMO workload shape
    (128, 64, 1, "f32"),
    (64, 64, 2, "f32"),
    (32, 32, 3, "f32"),
    (16, 16, 2, "bf16"),
    (128, 32, 2, "bf16"),
])
def test_block_all_pieces(N, P, R, io):
    d, bp = _draw(2, 300, 3, P, N, R, io, seed=N + P + R)   # 5 chunks, ragged tail of 44
    _parity(d, bp, ALL, io)


@pytest.mark.parametrize("piece", ALL)
@pytest.mark.parametrize("R", [1, 3])
def test_block_each_piece(piece, R):
    d, bp = _draw(1, 150, 2, 32, 64, R, "f32", seed=20 + R)
    _parity(d, bp, (piece,), "f32")


def test_block_norm_scale_invariance():
    """With the normalisation on, scaling B and C by a per-row factor leaves
    the output unchanged up to eps: checked on the GPU against the oracle of
    the unscaled inputs."""
    d, bp = _draw(1, 130, 2, 32, 32, 2, "f32", seed=31)
    rng = np.random.default_rng(310)
    ds = dict(d)
    for k in ("B", "C"):
        ds[k] = (d[k] * rng.uniform(0.5, 4.0, size=d[k].shape[:-1] + (1,))).astype(np.float32)
    from mamba_selective_ssm_ssd_amd import mixer
    t = to_dev(ds, "f32")
    block, z = _gpu_block(bp, ("bc_norm", "C_bias"), "f32")
    y, _ = mixer.prefill(t["x"], t["dt"], t["A"], t["lam"], t["theta"], t["B"], t["C"], block=block, z=z)
    yr, _, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                                block=_oracle_block(bp, ("bc_norm", "C_bias")))
    assert slice_err(y.double().cpu().numpy(), yr, (0, 2)) <= TOL["f32"]


def test_block_segmented_long_sequence():
    """One long sequence over few heads: segments, the pre-pass and the block."""
    d, bp = _draw(1, 1500, 2, 32, 64, 4, "bf16", seed=32)
    d["A"] *= 0.01
    _parity(d, bp, ALL, "bf16")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_carried_state_split(io):
    """A sequence cut in two: the second call starts from the first's state."""
    from mamba_selective_ssm_ssd_amd import mixer
    d, bp = _draw(2, 230, 3, 32, 64, 3, io, seed=33)
    d["A"] *= 0.01
    T1 = 100
    cut = lambda v, a, b: v[:, a:b] if v.ndim >= 3 else v
    first = {k: cut(v, 0, T1) for k, v in d.items()}
    second = {k: cut(v, T1, None) for k, v in d.items()}
    bp1 = dict(bp, z=bp["z"][:, :T1])
    bp2 = dict(bp, z=bp["z"][:, T1:])
    ys = []
    st = None
    for part, bpp in ((first, bp1), (second, bp2)):
        t = to_dev(part, io)
        block, z = _gpu_block(bpp, ALL, io)
        y, st = mixer.prefill(t["x"], t["dt"], t["A"], t["lam"], t["theta"], t["B"], t["C"],
                              state=st, block=block, z=z)
        ys.append(y.double().cpu().numpy())
    blk = _oracle_block(bp, ALL)
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=blk)
    assert slice_err(np.concatenate(ys, axis=1), yr, (0, 2)) <= TOL[io]
    _check_state(st, d, bp, blk, hT, oracle.cumulative_angle(d["theta"]), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_random_carried_state(io):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R = 2, 97, 2, 32, 32, 2
    d, bp = _draw(b, T, H, P, N, R, io, seed=34)
    rng = np.random.default_rng(340)
    init_np = dict(h=rng.standard_normal((b, H, N, P)).astype(np.float32),
                   phi=rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)).astype(np.float32),
                   prev_B=rng.standard_normal((b, H, R, N)).astype(np.float32),
                   prev_x=synth.round_io(rng.standard_normal((b, H, R, P)), io))
    init = mixer.State(*(torch.from_numpy(init_np[k]).cuda() for k in ("h", "phi", "prev_B")),
                       torch.from_numpy(init_np["prev_x"]).to("cuda", torch_io(io)))
    _parity(d, bp, ALL, io, init=init, init_np={k: v.astype(np.float64) for k, v in init_np.items()})


def _decode_run(d, bp, pieces, io, st, t0, t1):
    """Decode tokens t0..t1-1 of d one step at a time; returns y [b,t1-t0,H,R,P]."""
    from mamba_selective_ssm_ssd_amd import mixer
    t = to_dev(d, io)
    block, z = _gpu_block(bp, pieces, io)
    ys = []
    for s in range(t0, t1):
        zs = z[:, s].clone() if z is not None else None
        y = mixer.decode_step(*(t[k][:, s].clone() if k != "A" else t[k]
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")),
                              st, block=block, z=zs)
        ys.append(y.double().cpu().numpy()[:, None])
    return np.concatenate(ys, axis=1)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_prefill_then_decode(io):
    b, T, H, P, N = 2, 150, 3, 64, 64
    R = 4 if io == "bf16" else 3
    d, bp = _draw(b, T, H, P, N, R, io, seed=35)
    d["A"] *= 0.05
    T1 = 131
    from mamba_selective_ssm_ssd_amd import mixer
    first = {k: (v[:, :T1] if v.ndim >= 3 else v) for k, v in d.items()}
    t = to_dev(first, io)
    block, z = _gpu_block(dict(bp, z=bp["z"][:, :T1]), ALL, io)
    y1, st = mixer.prefill(t["x"], t["dt"], t["A"], t["lam"], t["theta"], t["B"], t["C"],
                           block=block, z=z)
    y2 = _decode_run(d, bp, ALL, io, st, T1, T)
    blk = _oracle_block(bp, ALL)
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=blk)
    assert slice_err(np.concatenate([y1.double().cpu().numpy(), y2], axis=1), yr, (0, 2)) <= TOL[io]
    _check_state(st, d, bp, blk, hT, oracle.cumulative_angle(d["theta"]), io)


@pytest.mark.parametrize("N,P,R,io", [
    (16, 16, 1, "bf16"), (16, 64, 4, "f32"), (32, 32, 2, "bf16"), (64, 16, 3, "f32"),
    (64, 64, 4, "bf16"), (128, 32, 2, "f32"), (128, 64, 1, "bf16"), (128, 64, 4, "f32"),
])
def test_block_decode_tile_set(N, P, R, io):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H = 3, 12, 5
    d, bp = _draw(b, T, H, P, N, R, io, seed=N + 3 * P + R)
    st = mixer.State.zeros(b, H, N, P, R, torch_io(io))
    yg = _decode_run(d, bp, ALL, io, st, 0, T)
    blk = _oracle_block(bp, ALL)
    yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=blk)
    assert slice_err(yg, yr, (0, 2)) <= TOL[io]
    _check_state(st, d, bp, blk, hT, oracle.cumulative_angle(d["theta"]), io)


@pytest.mark.parametrize("piece", ALL)
def test_block_decode_each_piece(piece):
    from mamba_selective_ssm_ssd_amd import mixer
    b, T, H, P, N, R = 2, 9, 3, 32, 64, 2
    d, bp = _draw(b, T, H, P, N, R, "f32", seed=36)
    st = mixer.State.zeros(b, H, N, P, R, torch.float32)
    yg = _decode_run(d, bp, (piece,), "f32", st, 0, T)
    yr, _, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                                block=_oracle_block(bp, (piece,)))
    assert slice_err(yg, yr, (0, 2)) <= TOL["f32"]


def test_block_empty_is_plain_path():
    """A block with no piece present is the plain mixer, bit for bit; identity
    weights and zero biases without the normalisation give the plain output."""
    from mamba_selective_ssm_ssd_amd import mixer
    d, _ = _draw(2, 200, 3, 32, 64, 2, "bf16", seed=37)
    t = to_dev(d, "bf16")
    args = [t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")]
    y0, s0 = mixer.prefill(*args)
    y1, s1 = mixer.prefill(*args, block=mixer.Block(bc_norm=False))
    assert torch.equal(y0, y1) and torch.equal(s0.h, s1.h)
    H, R, N = 3, 2, 64
    ones = torch.ones(H, R, N, device="cuda")
    zeros = torch.zeros(H, R, N, device="cuda")
    blk = mixer.Block(bc_norm=False, B_weight=ones, B_bias=zeros, C_weight=ones, C_bias=zeros)
    y2, s2 = mixer.prefill(*args, block=blk)
    assert slice_err(y2.double().cpu().numpy(), y0.double().cpu().numpy(), (0, 2)) <= 1e-6
    assert slice_err(s2.h.double().cpu().numpy(), s0.h.double().cpu().numpy(), (0, 1)) <= 1e-6


def test_block_siso_prefill_full_size():
    """SISO workload at full size (b4 T2048 H64 P64 N128, bf16) with every
    block piece; sampled (batch, head) instances recomputed by the oracle."""
    from mamba_selective_ssm_ssd_amd import mixer
    c = synth.CONFIGS[1]
    b, T, H, P, N, R = (c[k] for k in ("batch", "T", "H", "P", "N", "R"))
    inp = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    bw, cw = (1.0 + 0.25 * torch.randn(H, R, N, generator=g, device="cuda") for _ in range(2))
    bb, cb = (0.5 * torch.randn(H, R, N, generator=g, device="cuda") for _ in range(2))
    z = torch.randn(inp["x"].shape, generator=g, device="cuda").to(torch.bfloat16)
    block = mixer.Block(bc_norm=True, eps=EPS, B_weight=bw, B_bias=bb, C_weight=cw, C_bias=cb)
    y, st = mixer.prefill(*(inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")), block=block, z=z)
    torch.cuda.synchronize()
    for bi, hi in [(0, 0), (1, 17), (3, 63)]:
        d = {k: inp[k][bi:bi + 1, :, hi:hi + 1].float().cpu().numpy() for k in ("x", "dt", "lam", "theta", "B", "C")}
        d["A"] = inp["A"][hi:hi + 1].cpu().numpy()
        blk = dict(bc_norm=True, eps=EPS, z=z[bi:bi + 1, :, hi:hi + 1].float().cpu().numpy())
        for k, v in (("B_weight", bw), ("B_bias", bb), ("C_weight", cw), ("C_bias", cb)):
            blk[k] = v[hi:hi + 1].cpu().numpy()
        yr, hT, _ = oracle.run_block(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"], block=blk)
        e = slice_err(y[bi:bi + 1, :, hi:hi + 1].double().cpu().numpy(), yr, (0, 2))
        phiT = oracle.cumulative_angle(d["theta"])
        eh = slice_err(oracle.state_to_true(st.h[bi:bi + 1, hi:hi + 1].double().cpu().numpy(), phiT), hT, (0, 1))
        print(f"block SISO full size (b={bi}, h={hi}): y err {e:.2e}, state err {eh:.2e}")
        assert e <= TOL["bf16"] and eh <= TOL["bf16"]
