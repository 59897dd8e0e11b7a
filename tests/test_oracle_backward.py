"""Pins of the oracle's gradients (oracle/backward.py), CPU only.

The gradient oracle is torch autograd through a rotated-frame formulation of
the mixer.  It is pinned to things other than itself: the forward agrees with
the complex true-frame recurrence of m3_oracle.c, every gradient agrees with
central finite differences of m3_oracle.c, and the gradients of the inputs the
output is linear in reproduce the loss exactly (Euler's identity for linear
maps).
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob
from mamba_selective_ssm_ssd_amd import synth

torch = pytest.importorskip("torch")


def _case(b=2, T=23, H=2, P=4, N=8, R=2, seed=0):
    d = synth.prefill_inputs(b, T, H, P, N, R, io="f32", seed=seed, cfg=95)
    d = {k: v.astype(np.float64) for k, v in d.items()}
    rng = np.random.default_rng(950 + seed)
    init = dict(h0=rng.standard_normal((b, H, N, P)) * 0.5,
                phi0=rng.uniform(-np.pi, np.pi, size=(b, H, N // 2)),
                prevB0=rng.standard_normal((b, H, R, N)),
                prevx0=rng.standard_normal((b, H, R, P)))
    gy = rng.standard_normal((b, T, H, R, P))
    return d, init, gy


def _loss_c(d, init, gy):
    """L = sum(gy * y) with y from m3_oracle.c (carried state converted to the
    state's own frame)."""
    h0 = oracle.state_to_true(init["h0"], init["phi0"])
    pB = oracle.prevB_to_true(init["prevB0"], init["phi0"])
    # Phi_{-1} enters the true-frame recurrence only through the carried
    # state's conversion; B_t and C_t are raw inputs there
    y, _, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                         h0=h0, prevB0=pB, prevx0=init["prevx0"])
    return float(np.sum(gy * y))


def test_rotated_forward_matches_complex_oracle():
    d, init, _ = _case()
    t = {k: torch.tensor(v) for k, v in d.items()}
    ti = {k: torch.tensor(v) for k, v in init.items()}
    y, hT = ob.forward_rot(*(t[k] for k in ob.NAMES), **ti)
    yc, hTc, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                            h0=oracle.state_to_true(init["h0"], init["phi0"]),
                            prevB0=oracle.prevB_to_true(init["prevB0"], init["phi0"]),
                            prevx0=init["prevx0"])
    assert np.max(np.abs(y.numpy() - yc)) <= 1e-12 * max(1.0, np.max(np.abs(yc)))
    phiT = oracle.cumulative_angle(d["theta"], init["phi0"])
    assert np.max(np.abs(oracle.state_to_true(hT.numpy(), phiT) - hTc)) <= 1e-12 * np.max(np.abs(hTc))


@pytest.mark.parametrize("R", [1, 2])
def test_gradients_match_finite_differences(R):
    d, init, gy = _case(R=R, seed=R)
    _, g = ob.grad(d, gy, init)
    rng = np.random.default_rng(7 + R)
    for name in ob.NAMES + ob.INIT:
        src = d if name in d else init
        gname = name if name in d else "g_" + name
        arr = src[name]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            eps = 1e-5 * max(1.0, abs(arr[idx]))
            plus, minus = {k: v.copy() for k, v in src.items()}, {k: v.copy() for k, v in src.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            if name in d:
                fd = (_loss_c(plus, init, gy) - _loss_c(minus, init, gy)) / (2 * eps)
            else:
                fd = (_loss_c(d, plus, gy) - _loss_c(d, minus, gy)) / (2 * eps)
            an = g[gname][idx]
            assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, an, fd)


def test_linear_inputs_reproduce_the_loss():
    """y is linear in C (everything else fixed), and linear in the pair
    (x, carried state) jointly: sum(g * v) over those inputs equals L."""
    d, init, gy = _case(seed=3)
    y, g = ob.grad(d, gy, init)
    L = float(np.sum(gy * y))
    assert abs(np.sum(g["C"] * d["C"]) - L) <= 1e-10 * max(1.0, abs(L))
    lin = (np.sum(g["x"] * d["x"]) + np.sum(g["g_h0"] * init["h0"]) + np.sum(g["g_prevx0"] * init["prevx0"]))
    assert abs(lin - L) <= 1e-10 * max(1.0, abs(L))


def test_fresh_sequence_has_no_previous_token_gradient_path():
    """With a zero carried state, the previous token's x still receives a
    gradient through beta_0 only via prev_B (zero here): it must be zero."""
    d, init, gy = _case(seed=4)
    zero = {k: np.zeros_like(v) for k, v in init.items()}
    _, g = ob.grad(d, gy, zero)
    assert np.max(np.abs(g["g_prevx0"])) == 0.0


@pytest.mark.parametrize("R,T1", [(1, 9), (2, 14), (3, 1)])
def test_final_state_gradients_chain_over_split_calls(R, T1):
    """The incoming final-state gradients (h~_T, Phi_T, B~_{T-1}, x_{T-1}) by
    the chain rule over a split: the gradients of a sequence split into two
    calls -- the second call's gradients of its initial carried state fed to
    the first call as gradients of its final state -- equal those of the whole
    sequence in one call (for every input; dA summed over the calls)."""
    d, init, gy = _case(T=23, R=R, seed=10 + R)
    _, g_full = ob.grad(d, gy, init)
    first = {k: (v[:, :T1] if v.ndim >= 3 else v) for k, v in d.items()}
    second = {k: (v[:, T1:] if v.ndim >= 3 else v) for k, v in d.items()}
    # the first call's final state, in the rotated frame, starts the second
    t = {k: torch.tensor(v) for k, v in first.items()}
    ti = {k: torch.tensor(v) for k, v in init.items()}
    _, hT, phiT, bT, xT = ob.forward_rot(*(t[k] for k in ob.NAMES), **ti, final=True)
    init2 = dict(h0=hT.numpy(), phi0=phiT.numpy(), prevB0=bT.numpy(), prevx0=xT.numpy())
    _, g2 = ob.grad(second, gy[:, T1:], init2)
    gfinal = dict(h=g2["g_h0"], phi=g2["g_phi0"], prev_B=g2["g_prevB0"], prev_x=g2["g_prevx0"])
    _, g1 = ob.grad(first, gy[:, :T1], init, gfinal)
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        got = np.concatenate([g1[k], g2[k]], axis=1)
        assert np.max(np.abs(got - g_full[k])) <= 1e-10 * max(1.0, np.max(np.abs(g_full[k]))), k
    assert np.max(np.abs(g1["A"] + g2["A"] - g_full["A"])) <= 1e-10 * max(1.0, np.max(np.abs(g_full["A"])))
    for k in ("g_h0", "g_phi0", "g_prevB0", "g_prevx0"):
        assert np.max(np.abs(g1[k] - g_full[k])) <= 1e-10 * max(1.0, np.max(np.abs(g_full[k]))), k


def test_final_state_gradient_of_h_matches_finite_differences():
    """<g, h~_T> through the complex true-frame oracle (h~_T = R(-Phi_T) h_T):
    its gradients with respect to x, dt and theta by central differences."""
    d, init, _ = _case(b=1, T=11, H=1, P=3, N=4, R=2, seed=21)
    rng = np.random.default_rng(2100)
    gh = rng.standard_normal((1, 1, 4, 3))
    gy0 = np.zeros((1, 11, 1, 2, 3))

    def loss(dd):
        h0 = oracle.state_to_true(init["h0"], init["phi0"])
        pB = oracle.prevB_to_true(init["prevB0"], init["phi0"])
        _, hT, _ = oracle.run(dd["x"], dd["dt"], dd["A"], dd["lam"], dd["theta"], dd["B"], dd["C"],
                              h0=h0, prevB0=pB, prevx0=init["prevx0"])
        phiT = oracle.cumulative_angle(dd["theta"], init["phi0"])
        h_rot = oracle.rotate_pairs(hT, -np.asarray(phiT)[..., None], axis=2)
        return float(np.sum(gh * h_rot))

    _, g = ob.grad(d, gy0, init, dict(h=gh))
    eps = 1e-6
    for k, idx in (("x", (0, 4, 0, 1, 2)), ("dt", (0, 7, 0)), ("theta", (0, 3, 0, 1)), ("B", (0, 10, 0, 0, 3))):
        dp = {kk: vv.copy() for kk, vv in d.items()}
        dm = {kk: vv.copy() for kk, vv in d.items()}
        dp[k][idx] += eps
        dm[k][idx] -= eps
        fd = (loss(dp) - loss(dm)) / (2 * eps)
        assert abs(fd - g[k][idx]) <= 1e-6 * max(1.0, abs(fd)), (k, fd, g[k][idx])
