"""Benchmark of the Mamba-3 SSM mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  ``value`` is the prefill throughput (tokens/s) of the
long-context MIMO prefill workload b1 T65536 H64 P64 N64 R4 (bf16 I/O, fp32
state, chunk 64), the largest single-GPU workload, with inputs resident in HBM;
one step is one whole prefill (the segment pre-pass and the output pass,
enqueued by the same stage entry points m3_ssm_prefill runs), timed with HIP
events on the stream the kernels run on.  Events between the two stages give
each kernel's average duration inside the same timed steps.

The same line carries the other workloads, each with its own roofline:
the tiny fp32 prefill (absolute time only), the SISO and MIMO prefill
workloads (b4 T2048 H64), the MIMO decode workload (b256, 1000 steps), the
block prologue/epilogue, head-group, bf16-state and backward variants; the
on-box ceilings (an MFMA-only loop, a streaming copy and read-modify-write);
the fp64 CPU oracle timed on a bounded sample of the headline workload; and
each workload's error against the oracle on sampled (batch, head) instances,
computed after the timed regions.  Inputs are synthetic and seeded
(mamba_selective_ssm_ssd_amd/synth.py).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA
METRIC = "Mamba-3 SSM prefill tokens/s + decode µs/step; % of MFMA / HBM peak"
TOL = {"f32": 1e-4, "bf16": 2e-2}
KERNEL_SOURCES = {"output": ["k_prefill.hpp", "m3_device.hpp", "m3_internal.hpp"],
                  "segment_state": ["k_prefill.hpp", "m3_device.hpp", "m3_internal.hpp"],
                  "decode_step": ["k_decode.hpp", "k_decode_bf16.hip", "m3_device.hpp", "m3_internal.hpp"]}


# ---------------------------------------------------------------------------
# Algorithmic bytes and flops (what each kernel must move / compute).
# s = bytes of the I/O dtype; one token-head = one (batch, token, head).
# ---------------------------------------------------------------------------
def token_head_bytes(P, N, R, s):
    """x, B, C, theta, dt, lam in and y out, per token-head."""
    return 2 * R * P * s + 2 * R * N * s + (N // 2) * s + 2 * s


def final_state_bytes(b, H, P, N, R, s, state_bytes=4):
    """h~, Phi, B~_prev, x_prev of every (batch, head)."""
    return b * H * (N * P * state_bytes + (N // 2) * 4 + R * N * 4 + R * P * s)


def path_min_bytes(b, T, H, P, N, R, s=2):
    """The whole prefill: inputs once, y once, the final state once."""
    return b * T * H * token_head_bytes(P, N, R, s) + final_state_bytes(b, H, P, N, R, s)


def aggregate_bytes(N, P):
    """One segment aggregate: N x P fp32 state, summed log decay, K fp64 angles."""
    return N * P * 4 + 4 + (N // 2) * 8


def kernel_bytes(kernel, b, T, H, P, N, R, plan, s=2):
    """Bytes each prefill kernel must move.  plan = (chunk_pre, chunk_out,
    segments S, tokens per segment, pre-pass pieces per segment k)."""
    _, _, S, L, k = plan
    if kernel == "output":
        # everything once, plus the aggregates of the pieces before each segment
        return path_min_bytes(b, T, H, P, N, R, s) + b * H * aggregate_bytes(N, P) * k * S * (S - 1) // 2
    if kernel == "segment_state":
        if S == 1:
            return 0
        toks = min(T, (S - 1) * L)
        per = R * P * s + R * N * s + (N // 2) * s + 2 * s  # x, B, theta, dt, lam
        return b * H * (toks * per + (S - 1) * k * aggregate_bytes(N, P))
    raise KeyError(kernel)


def output_useful_flops(b, T, H, P, N, R, Q):
    """Useful MFMA flops of the output pass with Q-token chunks: C B^T and
    M x over the causal (s <= t) token pairs of each chunk (R x R virtual
    rows per pair), C H for the incoming state and B^T x for the state
    update."""
    total = 0
    full, tail = divmod(T, Q)
    for q, n in ((Q, full), (tail, 1 if tail else 0)):
        pairs = q * (q + 1) // 2
        total += n * (pairs * R * R * 2 * (N + P) + q * R * 2 * N * P * 2)
    return total * b * H


def backward_bytes(b, T, H, P, N, R, s=2):
    """Inputs (x, gy, B, C, theta, dt, lam) read once, fp32 gradients written once."""
    K = N // 2
    rd = 2 * R * P * s + 2 * R * N * s + K * s + 2 * s
    wr = 4 * (R * P + 2 * R * N + K + 2)
    return b * T * H * (rd + wr)


def backward_flops(b, T, H, P, N, R, rows=32):
    """Algorithmic flops of the chunked backward's products, chunks of
    rows // R tokens: per chunk, the five masked products over token pairs
    i >= j (S = C~ B~^T, D = gy x^T, (W.S)^T gy, (W.D) B~, (W.D)^T C~) and the
    five state-sized ones (B~ G, gy H^T, x G^T, the update of G, and the
    forward sweep's update of H), each counted once."""
    Q = rows // R
    total = 0
    for c in range(math.ceil(T / Q)):
        q = min(Q, T - Q * c)
        pairs = q * (q + 1) // 2
        total += pairs * R * R * 2 * (3 * N + 2 * P) + 5 * q * R * N * P * 2
    return total * b * H


def decode_bytes_per_step(b, H, P, N, R, s=2, state_bytes=4):
    K = N // 2
    per = (2 * N * P * state_bytes + 2 * R * N * 4 + 2 * R * P * s + 2 * K * 4
           + R * P * s + 2 * R * N * s + K * s + 2 * s + R * P * s)
    return b * H * per


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mamba_selective_ssm_ssd_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel, workload):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters,
    recorded under profiles/ for the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != sources_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def record_traffic(fetch_csv, write_csv, copy_mib, workload):
    """Per-launch HBM bytes of the kernels of one workload from two rocprofv3
    --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch) made with --workloads <that one> --copy-calibration-mib COPY_MIB:
    each counter is scaled by what it reads for that plain device copy
    (COPY_MIB read and COPY_MIB written).  Writes
    profiles/<kernel>_<workload>_traffic.json for each kernel the runs hold,
    tagged with the sha256 of the kernel sources."""
    import csv
    from mamba_selective_ssm_ssd_amd import synth
    c = synth.CONFIGS[workload]
    kinds = {"decode": {"decode_step": "k_decode_step<"},
             "prefill": {"output": "k_prefill<", "segment_state": "k_prefill<"}}[c["kind"]]

    def rows(path, counter):
        out = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0, r.get("Dispatch_Id")))
        return out

    nbytes = copy_mib * (1 << 20)
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rs = rows(path, counter)
        copy = [v for k, v, _ in rs if "copyBuffer" in k]
        if not copy:
            raise SystemExit(f"{path}: no {counter} rows for the calibration copy")
        scale = nbytes / max(copy)
        for key, tag in kinds.items():
            # the pre-pass instance has OUT = false, the output pass OUT = true
            want = {"output": "true,", "segment_state": "false,", "decode_step": ""}[key]
            vals = [v for k, v, _ in rs if tag in k and (not want or want in k.replace(" ", ""))]
            if vals:
                per.setdefault(key, {})[counter] = (sum(vals) / len(vals), scale,
                                                    next(k for k, v, _ in rs if tag in k and (not want or want in k.replace(" ", ""))))
    for key, d in per.items():
        if "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        (fk, fs, name), (wk, ws, _) = d["FETCH_SIZE"], d["WRITE_SIZE"]
        rec = {"kernel": name, "workload": c["name"],
               "fetch_bytes_raw": fk, "write_bytes_raw": wk,
               "calibration_copy_bytes": nbytes, "fetch_scale": fs, "write_scale": ws,
               "hbm_read_bytes_per_launch": round(fk * fs), "hbm_write_bytes_per_launch": round(wk * ws),
               "hbm_bytes_per_launch": round(fk * fs + wk * ws),
               "sources_sha256": sources_digest(KERNEL_SOURCES[key])}
        out = os.path.join(ROOT, "profiles", f"{key}_{c['name']}_traffic.json")
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


# ---------------------------------------------------------------------------
# Timing helpers.  Every timed region is bracketed by HIP events recorded on
# the stream the kernels are enqueued on (torch's current stream, which the
# binding passes to the library).
# ---------------------------------------------------------------------------
def warm_for(torch, fn, seconds):
    """Calls fn until `seconds` of wall time have passed (the GPU raises its
    clocks only after about 100 ms of sustained work); returns the calls made."""
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(4):
            fn()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


class Prefill:
    """One prefill workload's buffers and its two stages as prepared C calls."""

    def __init__(self, torch, capi, mixer, inp, chunk=64):
        self.torch = torch
        x, B = inp["x"], inp["B"]
        b, T, H, R, P = x.shape
        N = B.shape[-1]
        self.dims = (b, T, H, P, N, R)
        self.io = "f32" if x.dtype == torch.float32 else "bf16"
        self.shape = mixer.make_shape(b, T, H, P, N, R, x.dtype, chunk=chunk, G=B.shape[2])
        rc, *plan = capi.m3_ssm_prefill_plan(self.shape)
        assert rc == capi.M3_OK, capi.m3_status_string(rc)
        self.plan = tuple(plan)
        self.y = torch.empty_like(x)
        self.st = mixer.State.zeros(b, H, N, P, R, x.dtype)
        self.ws = torch.empty(capi.m3_ssm_prefill_workspace_bytes(self.shape), device="cuda", dtype=torch.uint8)
        self.inp = inp
        stream = torch.cuda.current_stream().cuda_stream
        ptrs = [inp[k].data_ptr() for k in ("x", "dt", "A", "lam", "theta", "B", "C")]
        self._c_final = self.st.c()
        tail = (None, self._c_final, self.y.data_ptr(), self.ws.data_ptr(), self.ws.numel(), stream)

        def stage(sid):
            def go():
                rc = capi.m3_ssm_prefill_stage(sid, self.shape, *ptrs, *tail)
                if rc != capi.M3_OK:
                    raise capi.M3Error(rc, "m3_ssm_prefill_stage")
            return go

        def whole():
            rc = capi.m3_ssm_prefill(self.shape, *ptrs, *tail)
            if rc != capi.M3_OK:
                raise capi.M3Error(rc, "m3_ssm_prefill")

        self.pre, self.out, self.whole = stage(0), stage(1), whole
        self.segmented = self.plan[2] > 1

    def step(self):
        if self.segmented:
            self.pre()
        self.out()

    def time(self, steps, warmup, warm_s):
        """warm_s seconds of calls, `warmup` more, then `steps` timed steps.
        A segmented call (two kernels) has events before, between and after
        its two stages in every step; a call of one kernel (one segment per
        sequence) has one event before the first step and one after the
        last, so its kernel's average is the step's (an event between
        back-to-back launches costs a few microseconds).  Returns (ms per
        step, ms of the pre-pass, ms of the output pass, calls spent
        warming)."""
        torch = self.torch
        n = warm_for(torch, self.step, warm_s)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        if not self.segmented:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                self.out()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            return ms, 0.0, ms, n + warmup
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(steps):
            ev[k][0].record()
            self.pre()
            ev[k][1].record()
            self.out()
            ev[k][2].record()
        torch.cuda.synchronize()
        ms = ev[0][0].elapsed_time(ev[-1][2]) / steps
        pre = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        out = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
        return ms, pre, out, n + warmup


def roofline_hbm(kernel, alg_bytes, ms, traffic=None, stream_ceiling_gbs=None, extra=None):
    ach = alg_bytes / (ms / 1000) / 1e9
    r = {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "alg_bytes": alg_bytes,
         "avg_us": round(ms * 1000, 2)}
    if stream_ceiling_gbs:
        r["frac_of_measured_stream_ceiling"] = round(ach / stream_ceiling_gbs, 4)
    if extra:
        r.update(extra)
    return r


def prefill_entry(pf, ms, pre, out, name, kname, ceil):
    """The JSON entry of one prefill workload."""
    b, T, H, P, N, R = pf.dims
    s = 4 if pf.io == "f32" else 2
    qpre, qout, S, L, kp = pf.plan
    ob = kernel_bytes("output", b, T, H, P, N, R, pf.plan, s)
    pb = kernel_bytes("segment_state", b, T, H, P, N, R, pf.plan, s)
    flops = output_useful_flops(b, T, H, P, N, R, qout)
    mf = flops / (out / 1000) / 1e12
    roof = roofline_hbm(kname, ob, out, load_traffic("output", name) if pf.io == "bf16" else None,
                        ceil.get("stream_rmw_best_gbs"),
                        {"mfma_useful_tflops": round(mf, 2),
                         "mfma_frac_of_bf16_peak": round(mf / BF16_MFMA_PEAK_TFLOPS, 4)})
    pm = path_min_bytes(b, T, H, P, N, R, s)
    e = {"workload": name, "tokens_per_s": round(b * T / (ms / 1000), 1), "ms_per_step": round(ms, 4),
         "plan": {"chunk_pre": qpre, "chunk_out": qout, "segments": S, "segment_tokens": L,
                  "prepass_pieces": kp},
         "roofline": roof,
         "path": {"min_bytes": pm, "frac_of_hbm_peak_at_min_bytes": round(pm / (ms / 1000) / 1e9 / HBM_PEAK_GBS, 4)},
         "kernels": {"output": {"avg_us": round(out * 1000, 2), "alg_bytes": ob,
                                "gb_per_s": round(ob / (out / 1000) / 1e9, 1)}}}
    if S > 1:
        e["kernels"]["segment_state"] = {"avg_us": round(pre * 1000, 2), "alg_bytes": pb,
                                         "gb_per_s": round(pb / (pre / 1000) / 1e9, 1),
                                         "traffic": load_traffic("segment_state", name)}
    return e


def time_whole(torch, fn, steps, warmup, warm_s):
    warm_for(torch, fn, warm_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def block_params(torch, H, R, N, shape, seed=5):
    """Block prologue/epilogue parameters of the synthetic distributions
    (weight 1 + 0.25 N(0,1), bias 0.5 N(0,1), z ~ N(0,1) shaped like x)."""
    from mamba_selective_ssm_ssd_amd import mixer
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bw, cw = (1.0 + 0.25 * torch.randn(H, R, N, generator=g, device="cuda") for _ in range(2))
    bb, cb = (0.5 * torch.randn(H, R, N, generator=g, device="cuda") for _ in range(2))
    z = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    return mixer.Block(bc_norm=True, eps=1e-6, B_weight=bw, B_bias=bb, C_weight=cw, C_bias=cb), z


def time_backward(torch, mixer, inp, steps, warm_s):
    args = [inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    gy = torch.randn(inp["x"].shape, generator=g, device="cuda").to(inp["x"].dtype)
    return time_whole(torch, lambda: mixer.backward(*args, gy), steps, 2, warm_s)


def backward_entry(capi, mixer, torch, name, dims, msw, ceil):
    """The JSON entry of one backward workload timed at msw ms per call."""
    b, T, H, P, N, R = dims
    bb, bfl = backward_bytes(b, T, H, P, N, R), backward_flops(b, T, H, P, N, R)
    tf = bfl / (msw / 1000) / 1e12
    _, S, L = capi.m3_ssm_prefill_backward_plan(mixer.make_shape(b, T, H, P, N, R, torch.bfloat16))
    e = {"workload": name, "ms_per_step": round(msw, 3), "tokens_per_s": round(b * T / (msw / 1000), 1),
         "segments": S, "segment_tokens": L,
         "roofline": {"kernel": "k_backward", "bound": "mfma", "achieved": round(tf, 2),
                      "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                      "alg_flops": bfl, "avg_us": round(msw * 1000, 1)},
         "alg_bytes": bb, "frac_of_hbm_peak_at_alg_bytes": round(bb / (msw / 1000) / 1e9 / HBM_PEAK_GBS, 4),
         "note": "chunked, 32 (token, rank) rows per chunk, products on fp32 MFMA"}
    if ceil.get("mfma_fp32_tflops"):
        e["roofline"]["frac_of_measured_mfma_ceiling"] = round(tf / ceil["mfma_fp32_tflops"], 4)
    return e


def time_decode(torch, mixer, synth, b, H, P, N, R, steps, warmup, seed=0, with_block=False,
                state_dtype=None, warm_s=0.2, sample=None):
    """`steps` decode steps on step-major inputs after `warmup` steps and
    warm_s seconds of steps on other inputs.  With ``sample`` (a list of
    (batch, head)), also returns what the oracle needs to check those
    instances over the timed steps: the state before them, their per-step
    inputs and outputs (copied out after the timed region, by a replay of the
    same steps from the same state)."""
    inp = synth.torch_inputs(steps + warmup, b, H, P, N, R, io="bf16", seed=seed + 4)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 40)
    st = mixer.State.zeros(b, H, N, P, R, torch.bfloat16, state_dtype=state_dtype or torch.float32)
    st.h.copy_(torch.randn(st.h.shape, generator=g, device="cuda") * 0.1)
    y = torch.empty(b, H, R, P, device="cuda", dtype=torch.bfloat16)
    A = inp["A"]
    block, z = block_params(torch, H, R, N, (steps + warmup, b, H, R, P)) if with_block else (None, None)

    def step(t):
        mixer.decode_step(inp["x"][t], inp["dt"][t], A, inp["lam"][t], inp["theta"][t],
                          inp["B"][t], inp["C"][t], st, y=y, block=block,
                          z=z[t] if z is not None else None)

    # warm-up on the extra steps' inputs (the state keeps evolving from them)
    k = [0]

    def warm_step():
        step(steps + (k[0] % warmup))
        k[0] += 1

    warm_for(torch, warm_step, warm_s)
    torch.cuda.synchronize()
    saved = st.clone() if sample else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        step(t)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    check = None
    if sample:
        end = st.clone()
        # replay from the saved state, keeping the sampled outputs
        st.h.copy_(saved.h); st.phi.copy_(saved.phi); st.prev_B.copy_(saved.prev_B); st.prev_x.copy_(saved.prev_x)
        ys = []
        for t in range(steps):
            step(t)
            ys.append(torch.stack([y[bi, hi] for bi, hi in sample]).clone())
        torch.cuda.synchronize()
        assert torch.equal(st.h, end.h), "decode replay differs from the timed run"
        check = {"sample": sample, "h0": saved.h, "phi0": saved.phi, "prevB0": saved.prev_B,
                 "prevx0": saved.prev_x, "hT": end.h, "phiT": end.phi, "y": torch.stack(ys, 1),
                 "inputs": {k2: torch.stack([inp[k2][:steps, bi, hi] for bi, hi in sample]).float().cpu()
                            for k2 in ("x", "dt", "lam", "theta", "B", "C")},
                 "A": A.cpu()}
        check = {k2: (v.float().cpu() if hasattr(v, "cpu") and k2 not in ("inputs",) else v) for k2, v in check.items()}
    del inp
    return us, check


# ---------------------------------------------------------------------------
# On-box ceilings (include/m3_ssm_ceilings.h).
# ---------------------------------------------------------------------------
def ceilings(torch, capi):
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    nb = 4096
    sink = torch.empty(nb * 256, device="cuda")
    for kind, iters, fl, key in ((0, 1000, 16384, "mfma_bf16_tflops"), (1, 400, 2048, "mfma_fp32_tflops")):
        def go():
            rc = capi.m3_ceiling_mfma(kind, nb, iters, sink.data_ptr(), stream)
            assert rc == capi.M3_OK, capi.m3_status_string(rc)
        for _ in range(3):
            go()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(); go(); e1.record(); torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out[key] = round(nb * 4 * iters * 8 * fl / (best / 1000) / 1e12, 1)
    del sink
    # float4 streams of 1 GiB (beyond the 256 MB last-level cache) and of the
    # decode state's size (268 MB); best over grid sizes
    for nbytes, suffix in ((1 << 30, ""), (256 * 64 * 64 * 64 * 4, "_268MB")):
        n = nbytes // 16
        src = torch.ones(n * 4, device="cuda")
        dst = torch.ones_like(src)
        for mode, key in ((0, "stream_copy_gbs"), (1, "stream_rmw_gbs"), (2, "stream_copy_nt_gbs"),
                          (3, "stream_rmw_nt_gbs")):
            best = 1e9
            for nblk in (1024, 2048, 4096, 8192):
                def go():
                    rc = capi.m3_ceiling_stream(mode, src.data_ptr(), dst.data_ptr(), n, nblk, stream)
                    assert rc == capi.M3_OK, capi.m3_status_string(rc)
                for _ in range(3):
                    go()
                torch.cuda.synchronize()
                for _ in range(5):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(); go(); e1.record(); torch.cuda.synchronize()
                    best = min(best, e0.elapsed_time(e1))
            out[key + suffix] = round(2 * n * 16 / (best / 1000) / 1e9, 1)
        # the read-modify-write ceiling a kernel is compared with: the better
        # of the plain and the non-temporal stream
        out["stream_rmw_best_gbs" + suffix] = max(out["stream_rmw_gbs" + suffix], out["stream_rmw_nt_gbs" + suffix])
        del src, dst
    out["note"] = ("best of repeated launches: a v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32 loop on "
                   "8 accumulators over 4096 workgroups of 4 waves; a float4 copy and an in-place float4 "
                   "read-modify-write (bytes read + written) of 1 GiB and of 268 MB, plain and with "
                   "non-temporal loads and stores (_nt), best over 1024-8192 workgroups; "
                   "stream_rmw_best is the better of the two read-modify-writes")
    return out


# ---------------------------------------------------------------------------
# Oracle leg: CPU baseline and parity on sampled instances (after the timed
# regions; test infrastructure, fp64).
# ---------------------------------------------------------------------------
def slice_of(inp, bi, hi, t0=0, t1=None):
    """numpy fp64 inputs of one (batch, head) instance, shaped [1, T, 1, ...]."""
    import numpy as np
    out = {}
    for k in ("x", "dt", "lam", "theta", "B", "C"):
        v = inp[k][bi:bi + 1, t0:t1, hi:hi + 1]
        out[k] = v.float().cpu().numpy().astype(np.float64)
    out["A"] = inp["A"][hi:hi + 1].cpu().numpy().astype(np.float64)
    return out


def rel_err(g, r):
    import numpy as np
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))


def prefill_parity(samples, io):
    """samples: list of (inputs of one instance, GPU y [1,T,1,R,P], GPU final h~
    [1,1,N,P], GPU Phi [1,1,K]).  Errors per the metric of the tests: max over
    the instances of max|g - r| / max|r|, y and the final state in the true
    frame."""
    import numpy as np
    import oracle
    ey, eh = 0.0, 0.0
    for d, yg, hg, phig in samples:
        yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"])
        ey = max(ey, rel_err(yg, yr))
        phiT = oracle.cumulative_angle(d["theta"])
        eh = max(eh, rel_err(oracle.state_to_true(hg, phiT), hT))
    return {"y_max_rel_err": ey, "final_state_max_rel_err": eh, "tol": TOL[io],
            "pass": bool(ey <= TOL[io] and eh <= TOL[io])}


def cpu_baseline_and_parity(inp, pf, budget_s, nsample):
    """The fp64 oracle on the first `nsample` (batch, head) instances of the
    workload (all tokens), repeated until about budget_s CPU-seconds are
    spent; its throughput scaled to the whole workload's tokens/s, and the
    GPU's y and final state against it on those instances."""
    import numpy as np
    import oracle
    b, T, H, P, N, R = pf.dims
    hs = list(range(min(nsample, H)))
    d = {k: inp[k][0:1, :, 0:len(hs)].float().cpu().numpy().astype(np.float64)
         for k in ("x", "dt", "lam", "theta", "B", "C")}
    d["A"] = inp["A"][0:len(hs)].cpu().numpy().astype(np.float64)
    nthreads = oracle.default_threads()
    passes, wall, used, yr, hT = 0, 0.0, 1, None, None
    while True:
        t0 = time.perf_counter()
        yr, hT, used = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                                  nthreads=nthreads)
        wall += time.perf_counter() - t0
        passes += 1
        if wall * min(used, len(hs)) >= budget_s or passes >= 20:
            break
    yg = pf.y[0:1, :, 0:len(hs)].double().cpu().numpy()
    hg = pf.st.h[0:1, 0:len(hs)].double().cpu().numpy()
    phiT = oracle.cumulative_angle(d["theta"])
    ey = max(rel_err(yg[:, :, i], yr[:, :, i]) for i in range(len(hs)))
    eh = max(rel_err(oracle.state_to_true(hg, phiT)[:, i], hT[:, i]) for i in range(len(hs)))
    tok_heads = passes * len(hs) * T
    base = {"value": round(tok_heads / wall / H, 1), "unit": "tokens/s", "cores": int(min(used, len(hs))),
            "kind": "oracle",
            "sample": f"{len(hs)} of the {b * H} (batch, head) instances of the workload (batch 0, heads "
                      f"0..{len(hs) - 1}), all {T} tokens each, {passes} pass(es), {wall:.1f} s wall on "
                      f"{min(used, len(hs))} threads; tokens/s of the whole workload = token-heads/s / {H}"}
    par = {"y_max_rel_err": ey, "final_state_max_rel_err": eh, "tol": TOL[pf.io],
           "pass": bool(ey <= TOL[pf.io] and eh <= TOL[pf.io]),
           "sample": f"the same {len(hs)} instances"}
    return base, par


def decode_parity(chk):
    """The timed decode steps of the sampled instances against the oracle from
    the state they started from (true frame)."""
    import numpy as np
    import oracle
    ey, eh = 0.0, 0.0
    for i, (bi, hi) in enumerate(chk["sample"]):
        d = {k: chk["inputs"][k][i:i + 1, :, None].numpy().astype(np.float64) for k in chk["inputs"]}
        d["A"] = chk["A"][hi:hi + 1].numpy().astype(np.float64)
        phi0 = chk["phi0"][bi:bi + 1, hi:hi + 1].numpy().astype(np.float64)
        h0 = oracle.state_to_true(chk["h0"][bi:bi + 1, hi:hi + 1].numpy().astype(np.float64), phi0)
        pB = oracle.prevB_to_true(chk["prevB0"][bi:bi + 1, hi:hi + 1].numpy().astype(np.float64), phi0)
        px = chk["prevx0"][bi:bi + 1, hi:hi + 1].numpy().astype(np.float64)
        yr, hT, _ = oracle.run(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                               h0=h0, prevB0=pB, prevx0=px)
        yg = chk["y"][i].numpy().astype(np.float64)[None, :, None]
        ey = max(ey, rel_err(yg, yr))
        phiT = oracle.cumulative_angle(d["theta"], phi0)
        hg = chk["hT"][bi:bi + 1, hi:hi + 1].numpy().astype(np.float64)
        eh = max(eh, rel_err(oracle.state_to_true(hg, phiT), hT))
    return {"y_max_rel_err": ey, "final_state_max_rel_err": eh, "tol": TOL["bf16"],
            "pass": bool(ey <= TOL["bf16"] and eh <= TOL["bf16"]),
            "sample": f"(batch, head) {chk['sample']}, every timed step"}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps after the timed pre-warm")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed calls before the first timed region (clock ramp)")
    ap.add_argument("--warm-s", type=float, default=0.25,
                    help="seconds of untimed calls before each further timed region")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--workloads", default="0,1,2,3,4",
                    help="comma-separated workload numbers to run (the headline is 3)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline and parity leg")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the block, head-group, bf16-state and backward variants")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the on-box ceilings")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="CPU-seconds of oracle work")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "WORKLOAD"),
                    help="write the HBM traffic of one workload's kernels from two rocprofv3 counter "
                         "runs (no GPU needed) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        f, w, wl = args.record_traffic
        record_traffic(f, w, args.copy_calibration_mib or 512, int(wl))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer would shard over (batch, head) with no communication between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_selective_ssm_ssd_amd import capi, mixer, synth
    capi.load()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    wl = {int(v) for v in args.workloads.split(",") if v.strip()}

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + written")

    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic"}
    ceil = {}
    if not args.no_ceilings:
        ceil = ceilings(torch, capi)
        result["ceilings"] = ceil
        log(f"[ceilings] {ceil}")

    oracle_jobs = []   # work for the oracle leg, run after every timed region

    # --- headline: long-context MIMO prefill (configuration 3) -------------
    if 3 in wl:
        c = synth.CONFIGS[3]
        inp = synth.torch_inputs(c["batch"], c["T"], c["H"], c["P"], c["N"], c["R"], io="bf16", seed=0)
        pf = Prefill(torch, capi, mixer, inp)
        pre_t0 = time.perf_counter()
        warm_for(torch, pf.step, args.prewarm_s)
        prewarm = time.perf_counter() - pre_t0
        ms, pre, out, nw = pf.time(args.steps, args.warmup, 0.0)
        e = prefill_entry(pf, ms, pre, out, c["name"], "k_prefill output pass", ceil)
        b, T, H, P, N, R = pf.dims
        result.update(value=e["tokens_per_s"], ms_per_step=e["ms_per_step"])
        result["config"] = {"workload": c["name"], "batch": b, "seq_len": T, "heads": H, "headdim": P,
                            "dstate": N, "rank": R, "chunk": 64, "io": "bf16", "state": "fp32"}
        result["roofline"] = e["roofline"]
        result["path"] = e["path"]
        result["plan"] = e["plan"]
        result["kernels"] = e["kernels"]
        result["prewarm_s"] = round(prewarm, 3)
        log(f"[long mimo prefill] {ms:.3f} ms/step (pre-pass {pre:.3f}, output {out:.3f})  "
            f"{e['tokens_per_s']:.3e} tokens/s  output {e['roofline']['frac']:.3f} of HBM")
        if not args.no_variants:
            # its backward: 64 sequences, each cut into segments to fill the chip
            msw = time_backward(torch, mixer, inp, 3, args.warm_s)
            result["backward_long_mimo_prefill"] = backward_entry(capi, mixer, torch, c["name"], pf.dims, msw, ceil)
            log(f"[long mimo prefill backward] {msw:.3f} ms/step")
            torch.cuda.empty_cache()
        if not args.no_cpu:
            oracle_jobs.append(("cpu_baseline", inp, pf))
        else:
            del inp, pf
        torch.cuda.empty_cache()

    # --- the other prefill workloads ----------------------------------------
    for cfg in (0, 1, 2):
        if cfg not in wl:
            continue
        c = synth.CONFIGS[cfg]
        inp = synth.torch_inputs(c["batch"], c["T"], c["H"], c["P"], c["N"], c["R"], io=c["io"], seed=0)
        pf = Prefill(torch, capi, mixer, inp)
        steps = 200 if cfg else 500
        ms, pre, out, _ = pf.time(steps, 10, args.warm_s if result.get("prewarm_s") else args.prewarm_s)
        result.setdefault("prewarm_s", args.prewarm_s)
        e = prefill_entry(pf, ms, pre, out, c["name"], "k_prefill output pass", ceil)
        e["steps"] = steps
        if cfg == 0:
            e["note"] = "launch-bound tiny case: absolute time only"
        key = {0: "tiny_prefill", 1: "siso_prefill", 2: "mimo_prefill"}[cfg]
        result[key] = e
        log(f"[{key}] {ms * 1000:.1f} us/step  {e['tokens_per_s']:.3e} tokens/s  "
            f"output {e['roofline']['frac']:.3f} of HBM")
        if not args.no_cpu:
            b, T, H, P, N, R = pf.dims
            smp = [(0, 0)] if cfg == 0 else [(0, 5), (b - 1, H - 3)]
            if cfg == 0:
                smp = [(0, h) for h in range(H)]
            samples = [(slice_of(inp, bi, hi), pf.y[bi:bi + 1, :, hi:hi + 1].double().cpu().numpy(),
                        pf.st.h[bi:bi + 1, hi:hi + 1].double().cpu().numpy(), None) for bi, hi in smp]
            oracle_jobs.append((f"parity_{key}", samples, pf.io, smp))
        if not args.no_variants and cfg in (1, 2):
            b, T, H, P, N, R = pf.dims
            x, dt, A, lam, theta, B, C = (inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C"))
            blk, z = block_params(torch, H, R, N, x.shape)
            wsb = torch.empty(mixer.workspace_bytes(b, T, H, P, N, R, x.dtype), device="cuda", dtype=torch.uint8)
            msb = time_whole(torch, lambda: mixer.prefill(x, dt, A, lam, theta, B, C, final=pf.st, y=pf.y,
                                                          workspace=wsb, block=blk, z=z),
                             steps, 10, args.warm_s)
            zb = b * T * H * R * P * 2
            pm = path_min_bytes(b, T, H, P, N, R)
            result[f"block_{key}"] = {
                "workload": c["name"] + "+bcnorm_bias_gate", "tokens_per_s": round(b * T / (msb / 1000), 1),
                "ms_per_step": round(msb, 4), "vs_plain": round(ms / msb, 4), "path_min_bytes": pm + zb,
                "frac_of_hbm_peak_at_min_bytes": round((pm + zb) / (msb / 1000) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[{key} + block] {msb * 1000:.1f} us/step")
            del blk, z, wsb
            msw = time_backward(torch, mixer, inp, 10, args.warm_s)
            result[f"backward_{key}"] = backward_entry(capi, mixer, torch, c["name"], pf.dims, msw, ceil)
            log(f"[{key} backward] {msw:.3f} ms/step")
            if cfg == 1:
                del inp, pf
                torch.cuda.empty_cache()
                inpg = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0, G=1)
                pg = Prefill(torch, capi, mixer, inpg)
                msg, _, _, _ = pg.time(steps, 10, args.warm_s)
                gb = path_min_bytes(b, T, H, P, N, R) - b * T * (H - 1) * 2 * R * N * 2
                result["groups_siso_prefill"] = {
                    "workload": c["name"] + "_G1", "ngroups": 1, "tokens_per_s": round(b * T / (msg / 1000), 1),
                    "ms_per_step": round(msg, 4), "vs_per_head_bc": round(ms / msg, 4), "path_min_bytes": gb,
                    "frac_of_hbm_peak_at_min_bytes": round(gb / (msg / 1000) / 1e9 / HBM_PEAK_GBS, 4)}
                log(f"[siso prefill, one B/C group] {msg * 1000:.1f} us/step")
                del inpg, pg
        torch.cuda.empty_cache()

    # --- MIMO decode workload (configuration 4) -----------------------------
    if 4 in wl:
        c = synth.CONFIGS[4]
        b, H, P, N, R = (c[k] for k in ("batch", "H", "P", "N", "R"))
        sample = None if args.no_cpu else [(0, 0), (b - 1, H - 1)]
        us, chk = time_decode(torch, mixer, synth, b, H, P, N, R, args.decode_steps, 16,
                              warm_s=args.warm_s, sample=sample)
        db = decode_bytes_per_step(b, H, P, N, R)
        result["decode"] = {"workload": c["name"], "us_per_step": round(us, 2), "steps": args.decode_steps,
                            "roofline": roofline_hbm("k_decode_step", db, us / 1000,
                                                     load_traffic("decode_step", c["name"]),
                                                     ceil.get("stream_rmw_best_gbs_268MB"))}
        log(f"[mimo decode] {us:.1f} us/step  {result['decode']['roofline']['frac']:.3f} of HBM")
        if chk is not None:
            oracle_jobs.append(("parity_decode", chk))
        if not args.no_variants:
            usb, _ = time_decode(torch, mixer, synth, b, H, P, N, R, args.decode_steps, 16, with_block=True,
                                 warm_s=args.warm_s)
            dbb = db + b * H * R * P * 2
            result["block_decode"] = {
                "workload": c["name"] + "+bcnorm_bias_gate", "us_per_step": round(usb, 2),
                "vs_plain": round(us / usb, 4), "alg_bytes_per_step": dbb,
                "frac_of_hbm_peak": round(dbb / (usb * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[mimo decode + block] {usb:.1f} us/step")
            uss, _ = time_decode(torch, mixer, synth, b, H, P, N, R, args.decode_steps, 16,
                                 state_dtype=torch.bfloat16, warm_s=args.warm_s)
            dbs = decode_bytes_per_step(b, H, P, N, R, state_bytes=2)
            result["bf16_state_decode"] = {
                "workload": c["name"] + "_bf16_state", "us_per_step": round(uss, 2),
                "vs_fp32_state": round(us / uss, 4), "alg_bytes_per_step": dbs,
                "frac_of_hbm_peak": round(dbs / (uss * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[mimo decode, bf16 state] {uss:.1f} us/step")
        torch.cuda.empty_cache()

    # --- oracle leg (CPU; after every timed region) -------------------------
    if oracle_jobs:
        par = {}
        for job in oracle_jobs:
            if job[0] == "cpu_baseline":
                _, inp, pf = job
                log("[cpu baseline] timing the fp64 oracle on a sample of the headline workload ...")
                base, p3 = cpu_baseline_and_parity(inp, pf, args.cpu_budget, 16)
                result["cpu_baseline"] = base
                par["long_mimo_prefill"] = p3
                log(f"[cpu baseline] {base['value']:.3e} tokens/s on {base['cores']} threads")
                del inp, pf
                torch.cuda.empty_cache()
            elif job[0] == "parity_decode":
                par["decode"] = decode_parity(job[1])
            else:
                name, samples, io, smp = job
                p = prefill_parity(samples, io)
                p["sample"] = f"(batch, head) {smp}, all tokens"
                par[name[len("parity_"):]] = p
        result["parity"] = par
        log(f"[parity] " + ", ".join(f"{k}: y {v['y_max_rel_err']:.2e} h {v['final_state_max_rel_err']:.2e}"
                                     for k, v in par.items()))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
