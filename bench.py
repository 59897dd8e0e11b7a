"""Benchmark of the Mamba-3 SSM mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  ``value`` is the prefill throughput (tokens/s) of the
SISO prefill workload b4 T2048 H64 P64 N128 R1 (bf16 I/O, fp32 state, chunk
64) with inputs resident in HBM; one step is one m3_ssm_prefill call (the
whole chunked prefill).  The same line carries the MIMO prefill workload
(b4 T2048 H64 P64 N64 R4), the MIMO decode workload (b256 H64 P64 N64 R4,
1000 consecutive steps, us/step), each kernel's average time measured with
HIP events on the stream it runs on, the roofline of the dominant kernel, and
the fp64 CPU oracle timed on a bounded sample of the prefill workload.
Inputs are synthetic and seeded (see mamba_selective_ssm_ssd_amd/synth.py).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "Mamba-3 SSM prefill tokens/s + decode µs/step; % of MFMA / HBM peak"
KERNELS = ("segment_state", "output")
KERNEL_SOURCES = {"output": ["k_prefill.hpp", "m3_device.hpp", "m3_internal.hpp"],
                  "decode_step": ["k_decode.hpp", "k_decode_bf16.hip", "m3_device.hpp", "m3_internal.hpp"]}


# ---------------------------------------------------------------------------
# Algorithmic bytes and flops (what each kernel must move / compute).
# s = bytes of the I/O dtype.  "tok" = token-heads = b*T*H.
# ---------------------------------------------------------------------------
def segments(b, H, T, slots=256):
    """Segments per sequence chosen by the library for this shape."""
    nC = math.ceil(T / 64)
    s = 1 if b * H >= slots else slots // (b * H)
    s = max(1, min(s, nC))
    cps = math.ceil(nC / s)
    return math.ceil(nC / cps), cps


def kernel_bytes(kernel, b, T, H, P, N, R, s=2):
    """Bytes each prefill kernel must move: its inputs once, its outputs once."""
    S, cps = segments(b, H, T)
    K = N // 2
    state = b * H * N * P * 4
    if kernel == "output":
        # x, B, C, theta, dt, lam in, y out; aggregates of earlier segments in
        return path_min_bytes(b, T, H, P, N, R, s) + state * S * (S - 1) // 2
    if kernel == "segment_state":
        if S == 1:
            return 0
        toks = b * H * min(T, (S - 1) * cps * 64)
        return toks * (R * P * s + R * N * s + K * s + 2 * s) + state * (S - 1)
    raise KeyError(kernel)


def path_min_bytes(b, T, H, P, N, R, s=2):
    """Inputs + outputs of the whole prefill (x, B, C, theta, dt, lam, y)."""
    return b * T * H * (2 * R * P * s + 2 * R * N * s + (N // 2) * s + 2 * s)


def output_useful_flops(b, T, H, P, N, R):
    """Useful (causal) MFMA flops of the output pass: C B^T and M x over token
    pairs s <= t of a chunk, C H for the incoming state, and B^T x for the
    state update."""
    total = 0
    for c in range(math.ceil(T / 64)):
        q = min(64, T - 64 * c)
        pairs = q * (q + 1) // 2
        total += pairs * R * R * 2 * (N + P) + q * R * 2 * N * P * 2
    return total * b * H


def backward_bytes(b, T, H, P, N, R, s=2):
    """Inputs (x, gy, B, C, theta, dt, lam) read once, fp32 gradients written once."""
    K = N // 2
    rd = 2 * R * P * s + 2 * R * N * s + K * s + 2 * s
    wr = 4 * (R * P + 2 * R * N + K + 2)
    return b * T * H * (rd + wr)


FP32_MFMA_PEAK_TFLOPS = 157.3


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


def time_backward(torch, mixer, inp, reps=10, warmup=10):
    args = [inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C")]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    gy = torch.randn(inp["x"].shape, generator=g, device="cuda").to(inp["x"].dtype)
    for _ in range(warmup):
        mixer.backward(*args, gy)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mixer.backward(*args, gy)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


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


def record_traffic(fetch_csv, write_csv, copy_mib):
    """Per-launch HBM bytes of the prefill output pass (SISO workload) and of
    the decode step (MIMO decode workload) from two rocprofv3 --pmc runs of
    this script (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) that also
    ran --copy-calibration-mib COPY_MIB: each counter is scaled by what it
    reads for that plain device copy (COPY_MIB read and COPY_MIB written).
    Writes profiles/<kernel>_<workload>_traffic.json for each kernel the runs
    hold, tagged with the sha256 of the kernel sources."""
    import csv
    from mamba_selective_ssm_ssd_amd import synth
    c1, c4 = synth.CONFIGS[1], synth.CONFIGS[4]
    kernels = {
        "output": (f"k_prefill<m3::bf16, {c1['N']}, {c1['P']}, {c1['R']}, true, false>", c1["name"]),
        "decode_step": (f"k_decode_step<m3::bf16, {c4['N']}, {c4['P']}, {c4['R']}, false, false>", c4["name"]),
    }

    def avg(path, counter, tag):
        kern, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if tag in r["Kernel_Name"]:
                kern.append(v)
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
        if not copy:
            raise SystemExit(f"{path}: no {counter} rows for the calibration copy")
        # the calibration copy is the largest copy of the run (others, such as
        # filling the decode state, are smaller)
        return (sum(kern) / len(kern) if kern else None), max(copy)

    nbytes = copy_mib * (1 << 20)
    for key, (tag, workload) in kernels.items():
        fk, fc = avg(fetch_csv, "FETCH_SIZE", tag)
        wk, wc = avg(write_csv, "WRITE_SIZE", tag)
        if fk is None or wk is None:
            continue
        fs, ws = nbytes / fc, nbytes / wc
        rec = {"kernel": tag, "workload": workload,
               "fetch_bytes_raw": fk, "write_bytes_raw": wk,
               "calibration_copy_bytes": nbytes, "fetch_scale": fs, "write_scale": ws,
               "hbm_read_bytes_per_launch": round(fk * fs), "hbm_write_bytes_per_launch": round(wk * ws),
               "hbm_bytes_per_launch": round(fk * fs + wk * ws),
               "sources_sha256": sources_digest(KERNEL_SOURCES[key])}
        out = os.path.join(ROOT, "profiles", f"{key}_{workload}_traffic.json")
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


# ---------------------------------------------------------------------------
def time_prefill(torch, mixer, inp, steps, warmup, block=None, z=None):
    """Whole prefill calls back to back; then each kernel alone (plain path).
    With ``block``/``z`` only the whole calls are timed."""
    x, dt, A, lam, theta, B, C = (inp[k] for k in ("x", "dt", "A", "lam", "theta", "B", "C"))
    b, T, H, R, P = x.shape
    N = B.shape[-1]
    y = torch.empty_like(x)
    ws = torch.empty(mixer.workspace_bytes(b, T, H, P, N, R, x.dtype), device="cuda", dtype=torch.uint8)
    st = mixer.State.zeros(b, H, N, P, R, x.dtype)
    args = (x, dt, A, lam, theta, B, C)
    kw = dict(final=st, y=y, workspace=ws, block=block, z=z)
    for _ in range(warmup):
        mixer.prefill(*args, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        mixer.prefill(*args, **kw)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    if block is not None or z is not None:
        return ms, wall, {}
    # each kernel alone on the same stream (after a full prefill filled the
    # workspace): `steps` launches back to back between one event pair (an
    # event pair costs a few microseconds; per-launch pairs would add that to
    # every launch), right after the timed calls, so at the same clocks
    per_kernel = {}
    for name in KERNELS:
        if name == "segment_state" and segments(b, H, T)[0] == 1:
            per_kernel[name] = 0.0       # one segment per sequence: no pre-pass launch
            continue
        stage = mixer.capi.STAGES[name]
        reps = max(steps, 10)
        for _ in range(3):
            mixer.prefill_stage(stage, *args, None, st, y, ws)
        torch.cuda.synchronize()
        ks, ke = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ks.record()
        for _ in range(reps):
            mixer.prefill_stage(stage, *args, None, st, y, ws)
        ke.record()
        torch.cuda.synchronize()
        per_kernel[name] = ks.elapsed_time(ke) / reps
    mixer.prefill(*args, final=st, y=y, workspace=ws)   # leave a consistent state behind
    torch.cuda.synchronize()
    return ms, wall, per_kernel


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


def time_decode(torch, mixer, synth, b, H, P, N, R, steps, warmup, seed=0, with_block=False,
                state_dtype=None):
    # per-step inputs, step-major so that every step's slice is contiguous
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

    for t in range(warmup):
        step(steps + t)                  # (clocks up: the prefill ran just before)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        step(t)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    del inp
    return us


def cpu_baseline(torch, inp, budget_s):
    """The fp64 oracle over the whole prefill workload (every (batch, head)
    instance, all tokens), repeated until about budget_s seconds of CPU time
    (wall time x threads) are spent.  Returns the cpu_baseline object."""
    import numpy as np
    import oracle

    x = inp["x"]
    b, T, H, R, P = x.shape
    nthreads = oracle.default_threads()

    def batch(bi):
        sl = {k: inp[k][bi:bi + 1].float().cpu().numpy().astype(np.float64)
              for k in ("x", "dt", "lam", "theta", "B", "C")}
        sl["A"] = inp["A"].cpu().numpy().astype(np.float64)
        return sl

    passes, wall, used = 0, 0.0, 1
    while True:
        for bi in range(b):
            sl = batch(bi)
            t0 = time.perf_counter()
            _, _, used = oracle.run(sl["x"], sl["dt"], sl["A"], sl["lam"], sl["theta"], sl["B"], sl["C"],
                                    nthreads=nthreads)
            wall += time.perf_counter() - t0
        passes += 1
        if wall * used >= budget_s or passes >= 100:
            break
    return {"value": passes * b * T / wall, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"the whole workload ({b * H} (batch, head) instances x {T} tokens), "
                      f"{passes} pass(es), {wall:.1f} s wall on {used} threads "
                      f"({wall * used:.0f} CPU-seconds)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU raises its clocks only after about 100 ms of sustained work: a
    # short run measures the ramp (5-15% slower per call), so the defaults
    # time 200 calls after 800 untimed ones (about 0.1 s of SISO prefill).
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=800)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-mimo", action="store_true", help="skip the MIMO prefill workload")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the workloads with the block prologue/epilogue")
    ap.add_argument("--no-bf16-state", action="store_true",
                    help="skip the decode workload with a bf16 carried state")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass")
    ap.add_argument("--no-groups", action="store_true",
                    help="skip the SISO workload with B/C shared by all heads")
    ap.add_argument("--long", action="store_true", help="also run the T=65536 MIMO prefill")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="CPU-seconds of oracle work")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the output pass's HBM traffic from two rocprofv3 counter "
                         "runs (no GPU needed) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic, copy_mib=args.copy_calibration_mib or 512)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer shards over (batch, head) with no communication; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_selective_ssm_ssd_amd import mixer, synth
    mixer.capi.load()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {args.copy_calibration_mib} MiB read + written")

    # --- SISO prefill workload (the headline value) ----------------------------
    c1 = synth.CONFIGS[1]
    b, T, H, P, N, R = (c1[k] for k in ("batch", "T", "H", "P", "N", "R"))
    inp = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0)
    ms, wall, pk = time_prefill(torch, mixer, inp, args.steps, args.warmup)
    tok_s = b * T / (ms / 1000.0)
    log(f"[siso prefill] {ms * 1000:.1f} us/call  {tok_s:.3e} tokens/s  per kernel (us): "
        + ", ".join(f"{k} {v * 1000:.1f}" for k, v in pk.items()))
    kern = {}
    for k, v in pk.items():
        nb = kernel_bytes(k, b, T, H, P, N, R)
        kern[k] = {"avg_us": round(v * 1000, 2), "alg_bytes": nb,
                   "gb_per_s": round(nb / (v / 1000) / 1e9, 1) if nb else None}
    dom = max(pk, key=pk.get)
    dom_bytes = kernel_bytes(dom, b, T, H, P, N, R)
    achieved = dom_bytes / (pk[dom] / 1000) / 1e9
    traffic = load_traffic(dom, c1["name"]) if dom in KERNEL_SOURCES else None
    flops = output_useful_flops(b, T, H, P, N, R)
    roofline = {"kernel": f"k_{dom}", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "mfma_useful_tflops": round(flops / (pk["output"] / 1000) / 1e12, 2)}
    path_bytes = path_min_bytes(b, T, H, P, N, R)

    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": c1["name"], "batch": b, "seq_len": T, "heads": H, "headdim": P,
                   "dstate": N, "rank": R, "chunk": 64, "state": "fp32"},
        "roofline": roofline,
        "path": {"min_bytes": path_bytes,
                 "frac_of_hbm_peak_at_min_bytes": round(path_bytes / (ms / 1000) / 1e9 / HBM_PEAK_GBS, 4),
                 "wall_s": round(wall, 3)},
        "kernels": kern,
    }

    if not args.no_block:
        # the same SISO workload with BC norm, B/C weight and bias and the gate
        blk, z = block_params(torch, H, R, N, inp["x"].shape)
        msb, _, _ = time_prefill(torch, mixer, inp, args.steps, args.warmup, block=blk, z=z)
        zb = b * T * H * R * P * 2
        result["block_siso_prefill"] = {
            "workload": c1["name"] + "+bcnorm_bias_gate", "tokens_per_s": round(b * T / (msb / 1000), 1),
            "ms_per_call": round(msb, 4), "vs_plain": round(ms / msb, 4),
            "path_min_bytes": path_bytes + zb,
            "frac_of_hbm_peak_at_min_bytes": round((path_bytes + zb) / (msb / 1000) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[siso prefill + block] {msb * 1000:.1f} us/call")
        del blk, z

    if not args.no_groups:
        # the same SISO workload with one B/C group shared by all heads
        del inp
        torch.cuda.empty_cache()
        inp = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0, G=1)
        msg, _, _ = time_prefill(torch, mixer, inp, args.steps, args.warmup)
        gb = path_min_bytes(b, T, H, P, N, R) - b * T * (H - 1) * 2 * R * N * 2
        result["groups_siso_prefill"] = {
            "workload": c1["name"] + "_G1", "ngroups": 1,
            "tokens_per_s": round(b * T / (msg / 1000), 1), "ms_per_call": round(msg / 1, 4),
            "vs_per_head_bc": round(ms / msg, 4), "path_min_bytes": gb,
            "frac_of_hbm_peak_at_min_bytes": round(gb / (msg / 1000) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[siso prefill, one B/C group] {msg * 1000:.1f} us/call")
        del inp
        torch.cuda.empty_cache()
        inp = synth.torch_inputs(b, T, H, P, N, R, io="bf16", seed=0)

    if not args.no_backward:
        msb = time_backward(torch, mixer, inp)
        bb = backward_bytes(b, T, H, P, N, R)
        bf = backward_flops(b, T, H, P, N, R)
        result["backward_siso_prefill"] = {
            "workload": c1["name"], "ms_per_call": round(msb, 3),
            "tokens_per_s": round(b * T / (msb / 1000), 1), "alg_bytes": bb,
            "frac_of_hbm_peak_at_alg_bytes": round(bb / (msb / 1000) / 1e9 / HBM_PEAK_GBS, 4),
            "alg_flops": bf, "tflops_at_alg_flops": round(bf / (msb / 1000) / 1e12, 2),
            "frac_of_fp32_mfma_peak": round(bf / (msb / 1000) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            "note": "chunked, 32 (token, rank) rows per chunk, products on fp32 MFMA"}
        log(f"[siso backward] {msb:.3f} ms/call")

    if not args.no_cpu:
        log("[cpu baseline] timing the fp64 oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(torch, inp, args.cpu_budget)
        log(f"[cpu baseline] {result['cpu_baseline']['value']:.3e} tokens/s on "
            f"{result['cpu_baseline']['cores']} threads")
    del inp
    torch.cuda.empty_cache()

    # --- MIMO prefill workload ------------------------------------------------
    if not args.no_mimo:
        c2 = synth.CONFIGS[2]
        b2, T2, H2, P2, N2, R2 = (c2[k] for k in ("batch", "T", "H", "P", "N", "R"))
        inp = synth.torch_inputs(b2, T2, H2, P2, N2, R2, io="bf16", seed=0)
        ms2, _, pk2 = time_prefill(torch, mixer, inp, args.steps, args.warmup)
        ms2b = None
        if not args.no_backward:
            msw = time_backward(torch, mixer, inp)
            bf2 = backward_flops(b2, T2, H2, P2, N2, R2)
            bb2 = backward_bytes(b2, T2, H2, P2, N2, R2)
            result["backward_mimo_prefill"] = {
                "workload": c2["name"], "ms_per_call": round(msw, 3),
                "tokens_per_s": round(b2 * T2 / (msw / 1000), 1), "alg_bytes": bb2,
                "frac_of_hbm_peak_at_alg_bytes": round(bb2 / (msw / 1000) / 1e9 / HBM_PEAK_GBS, 4),
                "alg_flops": bf2, "tflops_at_alg_flops": round(bf2 / (msw / 1000) / 1e12, 2),
                "frac_of_fp32_mfma_peak": round(bf2 / (msw / 1000) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)}
            log(f"[mimo backward] {msw:.3f} ms/call")
        if not args.no_block:
            blk, z = block_params(torch, H2, R2, N2, inp["x"].shape)
            ms2b, _, _ = time_prefill(torch, mixer, inp, args.steps, args.warmup, block=blk, z=z)
            del blk, z
        del inp
        torch.cuda.empty_cache()
        f2 = output_useful_flops(b2, T2, H2, P2, N2, R2)
        result["mimo_prefill"] = {
            "workload": c2["name"], "tokens_per_s": round(b2 * T2 / (ms2 / 1000), 1),
            "ms_per_call": round(ms2, 4),
            "kernels": {k: {"avg_us": round(v * 1000, 2),
                            "gb_per_s": (round(kernel_bytes(k, b2, T2, H2, P2, N2, R2) / (v / 1000) / 1e9, 1)
                                         if kernel_bytes(k, b2, T2, H2, P2, N2, R2) else None)}
                        for k, v in pk2.items()},
            "output_mfma_useful_tflops": round(f2 / (pk2["output"] / 1000) / 1e12, 2),
            "output_mfma_frac_of_peak": round(f2 / (pk2["output"] / 1000) / 1e12
                                              / BF16_MFMA_PEAK_TFLOPS, 4),
            "path_frac_of_hbm_peak_at_min_bytes": round(
                path_min_bytes(b2, T2, H2, P2, N2, R2) / (ms2 / 1000) / 1e9 / HBM_PEAK_GBS, 4),
        }
        log(f"[mimo prefill] {ms2 * 1000:.1f} us/call  {b2 * T2 / (ms2 / 1000):.3e} tokens/s")
        if ms2b is not None:
            result["block_mimo_prefill"] = {
                "workload": c2["name"] + "+bcnorm_bias_gate",
                "tokens_per_s": round(b2 * T2 / (ms2b / 1000), 1), "ms_per_call": round(ms2b, 4),
                "vs_plain": round(ms2 / ms2b, 4)}
            log(f"[mimo prefill + block] {ms2b * 1000:.1f} us/call")

    if args.long:
        c3 = synth.CONFIGS[3]
        b3, T3, H3, P3, N3, R3 = (c3[k] for k in ("batch", "T", "H", "P", "N", "R"))
        inp = synth.torch_inputs(b3, T3, H3, P3, N3, R3, io="bf16", seed=0)
        ms3, _, pk3 = time_prefill(torch, mixer, inp, max(3, args.steps // 4), 1)
        del inp
        torch.cuda.empty_cache()
        result["long_mimo_prefill"] = {
            "workload": c3["name"], "tokens_per_s": round(b3 * T3 / (ms3 / 1000), 1),
            "ms_per_call": round(ms3, 4),
            "kernels": {k: {"avg_us": round(v * 1000, 2)} for k, v in pk3.items()}}
        log(f"[long mimo prefill] {ms3:.3f} ms/call")

    # --- MIMO decode workload -------------------------------------------------
    if not args.no_decode:
        c4 = synth.CONFIGS[4]
        b4, H4, P4, N4, R4 = (c4[k] for k in ("batch", "H", "P", "N", "R"))
        us = time_decode(torch, mixer, synth, b4, H4, P4, N4, R4, args.decode_steps, 10)
        db = decode_bytes_per_step(b4, H4, P4, N4, R4)
        ach = db / (us * 1e-6) / 1e9
        result["decode"] = {
            "workload": c4["name"], "us_per_step": round(us, 2), "steps": args.decode_steps,
            "roofline": {"kernel": "k_decode_step", "bound": "hbm", "achieved": round(ach, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic("decode_step", c4["name"]),
                         "alg_bytes_per_step": db}}
        log(f"[mimo decode] {us:.1f} us/step  {ach:.0f} GB/s")
        if not args.no_block:
            usb = time_decode(torch, mixer, synth, b4, H4, P4, N4, R4, args.decode_steps, 10,
                              with_block=True)
            dbb = db + b4 * H4 * R4 * P4 * 2         # + the gate input z
            result["block_decode"] = {
                "workload": c4["name"] + "+bcnorm_bias_gate", "us_per_step": round(usb, 2),
                "vs_plain": round(us / usb, 4), "alg_bytes_per_step": dbb,
                "frac_of_hbm_peak": round(dbb / (usb * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[mimo decode + block] {usb:.1f} us/step")
        if not args.no_bf16_state:
            uss = time_decode(torch, mixer, synth, b4, H4, P4, N4, R4, args.decode_steps, 10,
                              state_dtype=torch.bfloat16)
            dbs = decode_bytes_per_step(b4, H4, P4, N4, R4, state_bytes=2)
            result["bf16_state_decode"] = {
                "workload": c4["name"] + "_bf16_state", "us_per_step": round(uss, 2),
                "vs_fp32_state": round(us / uss, 4), "alg_bytes_per_step": dbs,
                "frac_of_hbm_peak": round(dbs / (uss * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[mimo decode, bf16 state] {uss:.1f} us/step")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
