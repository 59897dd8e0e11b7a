"""Causality and isolation on the GPU, through the C ABI.

A finite perturbation of token s's inputs (x and B scaled up, C and theta
changed) of one (batch, head) leaves every output of the earlier tokens of
that instance, and every output and final state of every other instance,
bit for bit unchanged: the masked entries of the intra-chunk products are
exact zeros, so the products of later tokens add exact zeros to earlier
rows.  A NaN planted at token s stays inside its own instance; inside it, it
reaches the head-dim column it was planted in, for every token from the
start of the chunk holding s on (a masked entry multiplies the NaN,
0 x NaN = NaN, in the intra-chunk product), and nothing before that chunk
nor any other column.
"""
import numpy as np
import pytest

from mamba_selective_ssm_ssd_amd import synth
from _helpers import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # (b, T, H, P, N, R, io, chunk): one segment per sequence, 64-token chunks
    (2, 300, 128, 32, 64, 1, "bf16", 64),
    # segmented sequences (pre-pass), the 64-token pre-pass and 16-token output pass
    (1, 1000, 2, 64, 64, 4, "bf16", 64),
    # fp32, small chunks in both passes, segmented
    (1, 700, 3, 32, 128, 2, "f32", 64),
    (2, 333, 2, 16, 32, 3, "f32", 32),
]


def _run(t, chunk):
    from mamba_selective_ssm_ssd_amd import mixer
    y, st = mixer.prefill(*(t[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")), chunk=chunk)
    torch.cuda.synchronize()
    return y, st


def _chunk_out(t, chunk):
    from mamba_selective_ssm_ssd_amd import capi, mixer
    x = t["x"]
    b, T, H, R, P = x.shape
    rc, qpre, qout, S, L, kp = capi.m3_ssm_prefill_plan(mixer.make_shape(b, T, H, P, t["B"].shape[-1], R, x.dtype,
                                                                      chunk=chunk))
    assert rc == 0
    return qout


@pytest.mark.parametrize("case", CASES)
def test_finite_perturbation_is_causal_and_isolated(case):
    b, T, H, P, N, R, io, chunk = case
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=5, cfg=70)
    t = to_dev(d, io)
    y0, st0 = _run(t, chunk)
    bi, hi = b - 1, H // 2
    for s in (0, 17, T // 2 + 3, T - 1):
        tp = {k: v.clone() for k, v in t.items()}
        tp["x"][bi, s, hi] *= 1000.0
        tp["B"][bi, s, hi] *= 100.0
        tp["C"][bi, s, hi] = -tp["C"][bi, s, hi]
        tp["theta"][bi, s, hi] += 1.0
        y1, st1 = _run(tp, chunk)
        # the instance's tokens before s: bit for bit
        assert torch.equal(y1[bi, :s, hi], y0[bi, :s, hi]), f"token {s} changed an earlier output"
        # tokens from s on do change
        assert not torch.equal(y1[bi, s:, hi], y0[bi, s:, hi])
        # every other instance: outputs and final states bit for bit
        mask = torch.ones(b, H, dtype=torch.bool, device="cuda")
        mask[bi, hi] = False
        yy0, yy1 = y0.permute(0, 2, 1, 3, 4)[mask], y1.permute(0, 2, 1, 3, 4)[mask]
        assert torch.equal(yy0, yy1), "another instance's output changed"
        for a0, a1 in ((st0.h, st1.h), (st0.phi, st1.phi), (st0.prev_B, st1.prev_B), (st0.prev_x, st1.prev_x)):
            assert torch.equal(a0[mask], a1[mask]), "another instance's final state changed"


@pytest.mark.parametrize("case", CASES)
def test_nan_stays_in_its_instance_and_chunk(case):
    b, T, H, P, N, R, io, chunk = case
    d = synth.prefill_inputs(b, T, H, P, N, R, io=io, seed=6, cfg=71)
    t = to_dev(d, io)
    y0, st0 = _run(t, chunk)
    q = _chunk_out(t, chunk)
    bi, hi = 0, H - 1
    for s in (5, T // 3, T - 2):
        tp = {k: v.clone() for k, v in t.items()}
        tp["x"][bi, s, hi, 0, 0] = float("nan")
        y1, st1 = _run(tp, chunk)
        c0 = (s // q) * q                                 # first token of the chunk holding s
        assert torch.equal(y1[bi, :c0, hi], y0[bi, :c0, hi]), "the NaN reached an earlier chunk"
        # head-dim column 0 of every output row from s on (all R output
        # channels), and of the final state, is NaN; the other columns of the
        # state and the output never meet it
        assert torch.isnan(y1[bi, s:, hi, :, 0].float()).all(), "outputs from s on must be NaN in column 0"
        assert torch.equal(y1[bi, :, hi, :, 1:], y0[bi, :, hi, :, 1:])
        assert torch.isnan(st1.h[bi, hi, :, 0].float()).all()
        assert torch.equal(st1.h[bi, hi, :, 1:], st0.h[bi, hi, :, 1:])
        mask = torch.ones(b, H, dtype=torch.bool, device="cuda")
        mask[bi, hi] = False
        assert torch.equal(y0.permute(0, 2, 1, 3, 4)[mask], y1.permute(0, 2, 1, 3, 4)[mask])
        assert torch.equal(st0.h[mask], st1.h[mask]) and torch.equal(st0.phi[mask], st1.phi[mask])
