"""Benchmark of the MALA hot path on one MI355X.

A step is one MALA training pass - forward then backward - over one batch of
the MHA workload (batch 2, 32 heads, N = 4096, d = 128, B_q = B_k = 128,
bf16, tau = 0.05, dO ~ N(0, 1)), with every input resident in HBM before the
timed region. ``value`` is dense-equivalent TFLOP/s: the FLOPs FullAttn would
execute for the same pass (4 d per legal (q, k) pair forward, 10 d
backward) divided by the measured time. The JSON line also carries executed
FLOPs, the skip rates, post-score slots per query, the roofline of the
dominant kernel (timed with HIP events on the stream it runs on) and the CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def legal_pairs(nq, nk, off):
    # sum over rows of the number of visible keys, L_q = q + off + 1
    return sum(min(q + off + 1, nk) for q in range(nq))


def tile_counts(nq, nk, bq, bk, off):
    nqb = (nq + bq - 1) // bq
    legal = 0
    for i in range(nqb):
        last = min((i + 1) * bq, nq) - 1 + off
        legal += last // bk + 1
    return legal


def timed(fn, steps, warmup, stream_events=None):
    """Run fn() warmup times, then time `steps` calls; returns ms per call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(wl, tau, bq, bk, seconds, with_bwd):
    """The oracle (as it stands) on whole heads of the same workload until
    about ``seconds`` of CPU work; dense-equivalent TFLOP/s of that sample."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    q = wl.q.float().cpu().double().numpy()
    k = wl.k.float().cpu().double().numpy()
    v = wl.v.float().cpu().double().numpy()
    do = wl.do.float().cpu().double().numpy() if with_bwd else None
    B, nq, hq, d = q.shape
    nqb = (nq + bq - 1) // bq
    nkb = (k.shape[1] + bk - 1) // bk
    pairs_head = legal_pairs(nq, k.shape[1], k.shape[1] - nq)
    t0 = time.perf_counter()
    heads = 0
    flops = 0.0
    while True:
        b, h = divmod(heads, hq)
        sl = slice(h, h + 1)
        qs, ks, vs = q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl]
        r = oracle.mala_forward(qs, ks, vs, tau, bq, bk)
        flops += pairs_head * 4 * d
        if with_bwd:
            oracle.mala_backward(qs, ks, vs, r["o"], do[b:b + 1, :, sl], r["z"], tau, bq, bk)
            flops += pairs_head * 10 * d
        heads += 1
        el = time.perf_counter() - t0
        log(f"cpu oracle: {heads} head(s) in {el:.1f}s")
        if el >= seconds or heads >= B * hq:
            break
    el = time.perf_counter() - t0
    what = "forward + backward" if with_bwd else "forward"
    return {"value": flops / el / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads} whole (batch, head) unit(s) of the same workload, {what}, "
                      f"numpy float64 on the host, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tau", type=float, default=0.05)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MALA operator here runs on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_causal_tile_amd as mala
    import workloads

    if not os.path.exists(mala.lib_path()):
        from block_sparse_causal_tile_amd import build
        build.build()
    mala.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    tau, bq, bk = args.tau, 128, 128
    wl = workloads.mha_temperature(device=dev, tau=tau, with_grad=True)
    B, nq, hq, d = wl.q.shape
    nk = wl.k.shape[1]
    off = nk - nq
    log(f"workload {wl.name}: q {tuple(wl.q.shape)} bf16, tau {tau}")

    has_bwd = True
    o = torch.empty_like(wl.q)
    z = torch.empty((B, hq, nq), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(wl.q), torch.empty_like(wl.k), torch.empty_like(wl.v)
    prob = mala.make_problem(wl.q, wl.k, tau, bq, bk)
    ws = torch.empty(max(mala.mala_bwd_workspace_size(prob), 16), device=dev, dtype=torch.uint8)

    # untimed pass with the debug counters on: skip rates and slots
    st_f = torch.zeros(4, dtype=torch.int64, device=dev)
    st_b = torch.zeros(4, dtype=torch.int64, device=dev)
    mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z, stats=st_f)
    try:
        mala.mala_bwd(wl.q, wl.k, wl.v, o, wl.do, z, tau, bq, bk, dq=dq, dk=dk, dv=dv,
                      workspace=ws, stats=st_b)
    except mala.MalaError as e:
        if e.status != mala.MALA_EUNSUPPORTED:
            raise
        has_bwd = False
        log("backward not available: timing the forward only")
    torch.cuda.synchronize()
    sf = st_f.cpu().tolist()
    sb = st_b.cpu().tolist()

    def fwd():
        mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z)

    def bwd():
        mala.mala_bwd(wl.q, wl.k, wl.v, o, wl.do, z, tau, bq, bk, dq=dq, dk=dk, dv=dv, workspace=ws)

    def step():
        fwd()
        if has_bwd:
            bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-kernel events on the stream the library launches on (torch's current stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        fwd()
        e1.record()
        if has_bwd:
            bwd()
        e2.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps if has_bwd else 0.0
    step_ms = sum(a.elapsed_time(c) for a, _, c in ev) / args.steps
    log(f"step {step_ms:.3f} ms (fwd {fwd_ms:.3f}, bwd {bwd_ms:.3f}), wall {wall_ms:.3f} ms")

    pairs = B * hq * legal_pairs(nq, nk, off)
    tile_flops = 2.0 * bq * bk * d
    dense_f = pairs * 4.0 * d
    dense_b = pairs * 10.0 * d if has_bwd else 0.0
    exec_f = sf[0] * tile_flops + sf[1] * tile_flops
    exec_b = (sb[0] * tile_flops + sb[1] * 4 * tile_flops) if has_bwd else 0.0
    value = (dense_f + dense_b) / (step_ms * 1e-3) / 1e12
    kern = {"mala_fwd": (fwd_ms, exec_f)}
    if has_bwd:
        kern["mala_bwd"] = (bwd_ms, exec_b)
    dom = max(kern, key=lambda n: kern[n][0])
    achieved = kern[dom][1] / (kern[dom][0] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "kernel": dom, "algorithmic_flops_per_launch": kern[dom][1],
            "avg_launch_ms": round(kern[dom][0], 4)}

    out = {
        "metric": "MALA fwd/bwd dense-equiv TFLOP/s + skip rate + % MFMA peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + (" fwd+bwd" if has_bwd else " fwd"),
                   "batch": B, "heads": hq, "seq_len": nq, "head_dim": d,
                   "block_q": bq, "block_k": bk, "tau": tau, "parallelism": "none (1 GPU)"},
        "fwd": {"ms": round(fwd_ms, 4), "dense_equiv_tflops": round(dense_f / fwd_ms / 1e9, 2),
                "executed_tflops": round(exec_f / fwd_ms / 1e9, 2),
                "skip_rate": round(1 - sf[1] / sf[0], 4),
                "slots_per_query": round(sf[2] / (B * hq * nq), 2),
                "pct_mfma_peak_executed": round(100 * exec_f / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 2)},
        "roofline": roof,
    }
    if has_bwd:
        out["bwd"] = {"ms": round(bwd_ms, 4), "dense_equiv_tflops": round(dense_b / bwd_ms / 1e9, 2),
                      "executed_tflops": round(exec_b / bwd_ms / 1e9, 2),
                      "skip_rate": round(1 - sb[1] / sb[0], 4),
                      "slots_per_query": round(sb[2] / (B * hq * nq), 2),
                      "pct_mfma_peak_executed": round(100 * exec_b / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, tau, bq, bk, args.cpu_seconds, has_bwd)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
