"""Benchmark of the MALA hot path on one MI355X.

A step is one MALA training pass - forward, then backward - over one batch
of the backward workload (batch 1, 16 heads, N = 8192, d = 128,
B_q = B_k = 64, bf16, tau = 0.05, forward inputs as the MHA recipe with
temperature 2, dO ~ N(0, 1)); every input is resident in HBM before the
timed region. ``value`` is dense-equivalent TFLOP/s: the FLOPs FullAttn
would execute for the same pass (4 d per legal (q, k) pair forward, 10 d
backward, one multiply-add = 2 FLOPs) over the measured step time.

The JSON line also reports executed FLOPs, skip rates and post-score slots
per query of each pass, the roofline of the dominant kernel (HIP events on
the stream the library launches on), sub-benchmarks of the other workloads
(MHA forward at four tolerances, GQA sink/window forward, split-KV decode
against the HBM roofline), and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-sub]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_DECODE_SPLITS = "4,8,16,32,64"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def legal_pairs(nq, nk, off):
    return sum(min(q + off + 1, nk) for q in range(nq))


class Timer:
    """Events on torch's current stream - the stream the binding hands to
    the library - around each call."""

    def __init__(self, n):
        import torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]

    def ms(self):
        return sum(a.elapsed_time(b) for a, b in self.ev) / len(self.ev)

    def median_ms(self):
        t = sorted(a.elapsed_time(b) for a, b in self.ev)
        n = len(t)
        return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])


def time_calls(fn, steps, warmup):
    """Median launch time (ms) over ``steps`` timed calls of a sub-benchmark.
    The timed calls follow the warmup without a synchronization, so the
    queue is never empty when a call's first event is recorded; the median
    keeps a host stall between two calls (which lets the queue drain and the
    GPU idle inside one call's events) out of the figure."""
    import torch
    for _ in range(warmup):
        fn()
    t = Timer(steps)
    for a, b in t.ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return t.median_ms()


def library_source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_sparse_causal_tile_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernels):
    """HBM bytes per launch of the given kernels from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs summarized in profiles/ (scaled by the copy calibration),
    or None when the library sources changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != library_source_hash():
        return None
    try:
        return sum(t["kernels"][k]["read_bytes"] + t["kernels"][k]["write_bytes"] for k in kernels)
    except KeyError:
        return None


_ORACLE_INPUTS = None  # host copies of the workload, shared with the forked oracle workers


def _oracle_head(job):
    """One (batch, head) unit of the oracle, forward + backward, on one BLAS
    thread; returns its wall time."""
    import oracle
    from threadpoolctl import threadpool_limits
    b, h, tau, bq, bk = job
    q, k, v, do = _ORACLE_INPUTS
    sl = slice(h, h + 1)
    qs, ks, vs, dos = q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl], do[b:b + 1, :, sl]
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        r = oracle.mala_forward(qs, ks, vs, tau, bq, bk)
        oracle.mala_backward(qs, ks, vs, r["o"], dos, r["z"], tau, bq, bk)
        return time.perf_counter() - t


def host_workload(tau):
    """The training-pass workload drawn on the host: the GPU step and the
    oracle baseline both run on exactly these numbers (the GPU gets a copy)."""
    import workloads
    return workloads.mha_backward(device="cpu", tau=tau)


def start_oracle_pool(wl):
    """Fork one oracle worker per host core - up to 16, the CPU share of one
    GPU - over the host copy of the training-pass workload, before anything
    touches the GPU, so no process that holds the device is ever forked."""
    global _ORACLE_INPUTS
    import multiprocessing as mp
    _ORACLE_INPUTS = tuple(t.float().double().numpy() for t in (wl.q, wl.k, wl.v, wl.do))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(n, 16))
    return mp.get_context("fork").Pool(processes=n), n, tuple(wl.q.shape), wl.k.shape[1]


def cpu_baseline(pool, n_workers, shape, nk, tau, bq, bk, seconds):
    """The oracle as it stands, forward + backward on whole (batch, head)
    units of the training-pass workload, one unit per worker process at a
    time, in rounds until about ``seconds`` of wall time or every unit is
    done; dense-equivalent TFLOP/s of the whole pool, and of one core."""
    B, nq, hq, d = shape
    pairs_head = legal_pairs(nq, nk, nk - nq)
    jobs = [(b, h, tau, bq, bk) for b in range(B) for h in range(hq)]
    t0 = time.perf_counter()
    times = []
    while jobs and time.perf_counter() - t0 < seconds:
        batch, jobs = jobs[:n_workers], jobs[n_workers:]
        times += pool.map(_oracle_head, batch)
        log(f"cpu oracle: {len(times)} head(s) fwd+bwd on {n_workers} worker(s) in {time.perf_counter() - t0:.1f}s")
    el = time.perf_counter() - t0
    flops = len(times) * pairs_head * 14.0 * d
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s (dense-equivalent)",
            "cores": n_workers, "kind": "oracle", "cpu_model": model,
            "per_core_value": round(pairs_head * 14.0 * d / (sum(times) / len(times)) / 1e12, 6),
            "sample": f"{len(times)} whole (batch, head) unit(s) of the training-pass workload "
                      f"(the very tensors the GPU step times), forward + backward, "
                      f"numpy float64, {n_workers} worker process(es) with one BLAS thread each, "
                      f"{el:.1f} s wall"}


def attainable_peaks(dev, steps=10, warmup=3):
    """What plain library kernels reach on this machine: a bf16 GEMM (8192^3,
    hipBLASLt through torch) for the matrix cores and a 1 GiB device copy for
    HBM. Context for the fractions of the published peaks, not a target."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    gemm_ms = time_calls(lambda: torch.matmul(a, b, out=c), steps, warmup)
    del a, b, c
    src = torch.empty(512 * 1024 * 1024, device=dev, dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    copy_ms = time_calls(lambda: dst.copy_(src), steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_8192_tflops": round(2.0 * n ** 3 / gemm_ms / 1e9, 1),
            "device_copy_1gib_gbs": round(2.0 * 1024 ** 3 / copy_ms / 1e6, 1)}


def fwd_sub(mala, wl, taus, steps, warmup):
    import torch
    B, nq, hq, d = wl.q.shape
    nk = wl.k.shape[1]
    bq, bk = wl.block_q, wl.block_k
    o = torch.empty_like(wl.q)
    z = torch.empty((B, hq, nq), device=wl.q.device, dtype=torch.float32)
    pairs = B * hq * legal_pairs(nq, nk, nk - nq)
    out = {}
    for tau in taus:
        st = torch.zeros(4, dtype=torch.int64, device=wl.q.device)
        mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z, stats=st)
        s = st.cpu().tolist()
        ms = time_calls(lambda: mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z), steps, warmup)
        ex = (s[0] + s[1]) * 2.0 * bq * bk * d
        out[str(tau)] = {"ms": round(ms, 4), "dense_equiv_tflops": round(pairs * 4.0 * d / ms / 1e9, 1),
                         "executed_tflops": round(ex / ms / 1e9, 1),
                         "pct_mfma_peak_executed": round(100 * ex / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                         "skip_rate": round(1 - s[1] / s[0], 4),
                         "slots_per_query": round(s[2] / (B * hq * nq), 1)}
        log(f"{wl.name} tau={tau}: {out[str(tau)]}")
    return out


def skip_fidelity_sub(mala, wl, tau, steps, warmup, settings=None):
    """The screened operator against the screening-disabled one (tau = 0) on
    one input: forward and backward times, skip rates, and the fidelity
    measures of the page's operator study from the library's instrumentation
    kernels (omitted mass per query row; per-head relative L2 of O, and of
    dQ, dK, dV under a Rademacher dO). ``settings`` (a subset of
    (tau, 0.0)) runs only those, e.g. to profile one setting alone; the
    fidelity measures and speedups need both."""
    settings = (tau, 0.0) if settings is None else tuple(settings)
    import torch
    B, nq, hq, d = wl.q.shape
    bq, bk = wl.block_q, wl.block_k
    dev = wl.q.device
    do = mala.mala_rademacher(wl.q.shape, 2024, device=dev)
    prob = mala.make_problem(wl.q, wl.k, tau, bq, bk)
    ws = torch.empty(mala.mala_bwd_workspace_size(prob), device=dev, dtype=torch.uint8)
    def hist_summary(hist):
        # post-score slots per query at the 50th / 90th / 99th percentile and max
        h = torch.tensor(hist, dtype=torch.float64)
        cdf = h.cumsum(0) / h.sum()
        pick = lambda p: int(torch.searchsorted(cdf, torch.tensor([p], dtype=torch.float64))[0]) * bk
        return {"p50": pick(0.5), "p90": pick(0.9), "p99": pick(0.99),
                "max": int(torch.nonzero(h).max()) * bk}

    res, runs, calls, counts = {}, {}, {}, {}
    pairs = B * hq * legal_pairs(nq, nq, 0)
    tile = 2.0 * bq * bk * d
    for t in settings:
        o = torch.empty_like(wl.q)
        z = torch.empty((B, hq, nq), device=dev, dtype=torch.float32)
        g = [torch.empty_like(wl.q), torch.empty_like(wl.k), torch.empty_like(wl.v)]
        sf = torch.zeros(4, dtype=torch.int64, device=dev)
        sb = torch.zeros(4, dtype=torch.int64, device=dev)
        fmask = mala.new_tile_mask(B, hq, nq, nq, bq, bk, dev)
        bmask = mala.new_tile_mask(B, hq, nq, nq, bq, bk, dev)
        mala.mala_fwd(wl.q, wl.k, wl.v, t, bq, bk, o=o, z=z, stats=sf, tile_mask=fmask)
        mala.mala_bwd(wl.q, wl.k, wl.v, o, do, z, t, bq, bk, dq=g[0], dk=g[1], dv=g[2], workspace=ws,
                      stats=sb, tile_mask=bmask)
        f, b = sf.cpu().tolist(), sb.cpu().tolist()
        counts[t] = (f, b)
        res[str(t)] = {"fwd_skip_rate": round(1 - f[1] / f[0], 4), "bwd_skip_rate": round(1 - b[1] / b[0], 4),
                       "fwd_slots_per_query_mean": round(f[2] / (B * hq * nq), 1),
                       "bwd_slots_per_query_mean": round(b[2] / (B * hq * nq), 1),
                       "fwd_slots_per_query": hist_summary(mala.mala_slot_histogram(fmask, nq, nq, bq, bk).cpu().tolist()),
                       "bwd_slots_per_query": hist_summary(mala.mala_slot_histogram(bmask, nq, nq, bq, bk).cpu().tolist()),
                       "fwd_ms": float("inf"), "bwd_ms": float("inf")}
        runs[t] = (o, z, g)
        calls[t] = (lambda t=t, o=o, z=z: mala.mala_fwd(wl.q, wl.k, wl.v, t, bq, bk, o=o, z=z),
                    lambda t=t, o=o, z=z, g=g: mala.mala_bwd(wl.q, wl.k, wl.v, o, do, z, t, bq, bk, dq=g[0],
                                                             dk=g[1], dv=g[2], workspace=ws))
    for _ in range(2):  # alternate the two settings; keep each one's best mean
        for t in settings:
            r = res[str(t)]
            r["fwd_ms"] = round(min(r["fwd_ms"], time_calls(calls[t][0], steps, warmup)), 4)
            r["bwd_ms"] = round(min(r["bwd_ms"], time_calls(calls[t][1], steps, warmup)), 4)
    for t in settings:
        # executed: S on every legal tile, P V per retained tile (forward);
        # S per legal tile, dP, dV, dK, dQ per retained tile (backward);
        # dense-equivalent: FullAttn's 4 d (forward) and 10 d (backward) per pair
        (f, b), r = counts[t], res[str(t)]
        ef, eb = (f[0] + f[1]) * tile, (b[0] + 4 * b[1]) * tile
        r["fwd_executed_tflops"] = round(ef / r["fwd_ms"] / 1e9, 1)
        r["fwd_dense_equiv_tflops"] = round(pairs * 4.0 * d / r["fwd_ms"] / 1e9, 1)
        r["fwd_pct_mfma_peak_executed"] = round(100 * ef / r["fwd_ms"] / 1e9 / PEAK_BF16_TFLOPS, 2)
        r["bwd_executed_tflops"] = round(eb / r["bwd_ms"] / 1e9, 1)
        r["bwd_dense_equiv_tflops"] = round(pairs * 10.0 * d / r["bwd_ms"] / 1e9, 1)
        r["bwd_pct_mfma_peak_executed"] = round(100 * eb / r["bwd_ms"] / 1e9 / PEAK_BF16_TFLOPS, 2)
    if settings != (tau, 0.0):
        out = {"workload": wl.name, "tau": tau, "by_tau": res}
        log(f"{wl.name}: {out}")
        return out
    (o_s, z_s, g_s), (o_r, z_r, g_r) = runs[tau], runs[0.0]
    om = mala.mala_omitted_mass(z_s, z_r).flatten()
    fid = {"omitted_mass_mean": float(om.mean()), "omitted_mass_p99": float(torch.quantile(om[:1 << 24], 0.99)),
           "omitted_mass_max": float(om.max())}
    for name, x, ref in (("o", o_s, o_r), ("dq", g_s[0], g_r[0]), ("dk", g_s[1], g_r[1]),
                         ("dv", g_s[2], g_r[2])):
        sd, sr = mala.mala_sq_err_heads(x, ref)
        rel = (sd / sr).sqrt()
        fid[f"rel_l2_{name}_head_mean"] = float(rel.mean())
        fid[f"rel_l2_{name}_head_max"] = float(rel.max())
    r0, rt = res["0.0"], res[str(tau)]
    out = {"workload": wl.name, "tau": tau, "by_tau": res, "fidelity": fid,
           "fwd_speedup_vs_tau0": round(r0["fwd_ms"] / rt["fwd_ms"], 3),
           "bwd_speedup_vs_tau0": round(r0["bwd_ms"] / rt["bwd_ms"], 3)}
    log(f"{wl.name}: {out}")
    return out


def latent_sub(mala, steps, warmup, taus=(0.0, 0.05, 1.0)):
    """Latent (MLA-shaped) forward and backward: batch 1, 16 query heads
    sharing one cached row per position, N = 4096, d_qk 576, d_v 512, 64 x 64
    tiles, banded latent scores, dO ~ N(0, 1).
    Forward: executed FLOPs = legal tiles x 2 B_q B_k d_qk + retained tiles x
    2 B_q B_k d_v; dense-equivalent = legal pairs x 2 (d_qk + d_v).
    Backward: executed = legal tiles x 2 B_q B_k d_qk (S recomputed) +
    retained tiles x 2 B_q B_k (d_v + d_v + d_qk + d_qk) (dP, dV, dK, dQ);
    dense-equivalent = legal pairs x 2 (3 d_qk + 2 d_v)."""
    import torch
    import workloads
    wl = workloads.latent_mqa(device="cuda")
    B, nq, hq, dqk = wl.q.shape
    dv = wl.v.shape[3]
    pairs = B * hq * legal_pairs(nq, nq, 0)
    g = torch.Generator(device="cuda").manual_seed(4242)
    do = torch.randn((B, nq, hq, dv), generator=g, device="cuda").to(wl.q.dtype)
    o = torch.empty((B, nq, hq, dv), device="cuda", dtype=wl.q.dtype)
    z = torch.empty((B, hq, nq), device="cuda", dtype=torch.float32)
    dq, dkv = torch.empty_like(wl.q), torch.empty_like(wl.k)
    prob = mala.make_problem(wl.q, wl.k, 0.05, 64, 64)
    ws = torch.empty(mala.mala_bwd_latent_workspace_size(prob), device="cuda", dtype=torch.uint8)
    res = {"workload": wl.name, "bwd_workspace_mb": round(ws.numel() / 1e6, 1)}
    for tau in taus:
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        sb = torch.zeros(4, dtype=torch.int64, device="cuda")
        mala.mala_fwd_latent(wl.q, wl.k, dv, tau, 64, 64, o=o, z=z, stats=st)
        mala.mala_bwd_latent(wl.q, wl.k, dv, o, do, z, tau, 64, 64, dq=dq, dkv=dkv, workspace=ws, stats=sb)
        s, t = st.cpu().tolist(), sb.cpu().tolist()
        ms = time_calls(lambda: mala.mala_fwd_latent(wl.q, wl.k, dv, tau, 64, 64, o=o, z=z), steps, warmup)
        msb = time_calls(lambda: mala.mala_bwd_latent(wl.q, wl.k, dv, o, do, z, tau, 64, 64, dq=dq, dkv=dkv,
                                                      workspace=ws), steps, warmup)
        ex = s[0] * 2.0 * 64 * 64 * dqk + s[1] * 2.0 * 64 * 64 * dv
        exb = t[0] * 2.0 * 64 * 64 * dqk + t[1] * 2.0 * 64 * 64 * (2 * dv + 2 * dqk)
        r = {"ms": round(ms, 4), "executed_tflops": round(ex / ms / 1e9, 2),
             "dense_equiv_tflops": round(pairs * 2.0 * (dqk + dv) / ms / 1e9, 2),
             "pct_mfma_peak_executed": round(100 * ex / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
             "skip_rate": round(1 - s[1] / s[0], 4),
             "slots_per_query": round(s[2] / (B * hq * nq), 2),
             "bwd": {"ms": round(msb, 4), "executed_tflops": round(exb / msb / 1e9, 2),
                     "dense_equiv_tflops": round(pairs * 2.0 * (3 * dqk + 2 * dv) / msb / 1e9, 2),
                     "pct_mfma_peak_executed": round(100 * exb / msb / 1e9 / PEAK_BF16_TFLOPS, 2),
                     "skip_rate": round(1 - t[1] / t[0], 4),
                     "slots_per_query": round(t[2] / (B * hq * nq), 2)}}
        res[str(tau)] = r
        log(f"latent tau={tau}: {r}")
    del wl
    torch.cuda.empty_cache()
    return res


def varlen_sub(mala, steps, warmup, tau=0.05, block=64):
    """Packed chunked prefill: 12 sequences of mixed lengths (new tokens
    N_q from 256 to 8192, each after a cached context of 0 to 8192 tokens),
    32 query / 8 KV heads, d 128, through mala_fwd_varlen."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(4242)
    hq, hkv, d = 32, 8, 128
    nq_list = [256, 512, 8192, 1024, 4096, 300, 2048, 777, 8192, 1500, 64, 3000]
    ctx = [0, 8192, 0, 4096, 2048, 1000, 0, 5000, 1024, 0, 8000, 512]
    nk_list = [a + b for a, b in zip(nq_list, ctx)]
    tq, tk = sum(nq_list), sum(nk_list)
    q = (torch.randn((tq, hq, d), generator=g, device="cuda") / d ** 0.5).bfloat16()
    k = torch.randn((tk, hkv, d), generator=g, device="cuda").bfloat16()
    v = torch.randn((tk, hkv, d), generator=g, device="cuda").bfloat16()
    cu_q = torch.tensor([0] + list(__import__("itertools").accumulate(nq_list)), dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0] + list(__import__("itertools").accumulate(nk_list)), dtype=torch.int32, device="cuda")
    mq, mk = max(nq_list), max(nk_list)
    o = torch.empty_like(q)
    z = torch.empty((hq, tq), device="cuda", dtype=torch.float32)
    st = torch.zeros(4, dtype=torch.int64, device="cuda")
    mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, mq, mk, tau, block, block, o=o, z=z, stats=st)
    s = st.cpu().tolist()
    ms = time_calls(lambda: mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, mq, mk, tau, block, block, o=o, z=z),
                    steps, warmup)
    pairs = hq * sum(legal_pairs(a, b, b - a) for a, b in zip(nq_list, nk_list))
    ex = (s[0] + s[1]) * 2.0 * block * block * d
    r = {"sequences": len(nq_list), "new_tokens": tq, "context_tokens": tk, "heads": f"{hq}q/{hkv}kv",
         "tau": tau, "ms": round(ms, 4), "dense_equiv_tflops": round(pairs * 4.0 * d / ms / 1e9, 1),
         "executed_tflops": round(ex / ms / 1e9, 1),
         "pct_mfma_peak_executed": round(100 * ex / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
         "skip_rate": round(1 - s[1] / s[0], 4)}
    log(f"varlen chunked prefill: {r}")
    return r


def decode_sub(mala, steps, warmup, splits_list=(4, 8, 16, 32, 64)):
    import torch
    import workloads
    wl = workloads.decode_cache(device="cuda")
    B, _, hq, d = wl.q.shape
    nk, hkv = wl.k.shape[1], wl.k.shape[2]
    bk = wl.block_k
    T = (nk + bk - 1) // bk
    kbytes = B * hkv * nk * d * 2
    res = {"workload": wl.name, "tau": wl.tau, "block_k": bk, "by_splits": {}}
    best = None
    for S in splits_list:
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        prob = mala.make_problem(wl.q, wl.k, wl.tau, 1, bk, nk - 1)
        ws = torch.empty(mala.mala_decode_workspace_size(prob, S), device="cuda", dtype=torch.uint8)
        o = torch.empty_like(wl.q)
        z = torch.empty((B, hq), device="cuda", dtype=torch.float32)
        mala.mala_decode(wl.q, wl.k, wl.v, wl.tau, bk, S, o=o, z=z, workspace=ws, stats=st)
        s = st.cpu().tolist()
        ms = time_calls(lambda: mala.mala_decode(wl.q, wl.k, wl.v, wl.tau, bk, S, o=o, z=z,
                                                 workspace=ws), steps, warmup)
        vbytes = s[3] * bk * d * 2
        gbs = (kbytes + vbytes) / (ms * 1e-3) / 1e9
        r = {"ms": round(ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
             "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
             "per_head_retain": round(s[1] / s[0], 4),
             "v_tile_load_fraction": round(s[3] / (B * hkv * T), 4),
             "bytes_per_launch": kbytes + vbytes}
        res["by_splits"][str(S)] = r
        log(f"decode splits={S}: {r}")
        if best is None or ms < res["by_splits"][str(best)]["ms"]:
            best = S
    res["best_splits"] = best
    # the same cache seen as pages (a zero-copy view: page i of sequence b is
    # rows [i P, (i + 1) P) of b's cache), decoded through the block table
    res["paged"] = {}
    for P in (16, 256):
        npb = nk // P
        kp = wl.k.view(B * npb, P, hkv, d)
        vp = wl.v.view(B * npb, P, hkv, d)
        table = torch.arange(B * npb, device="cuda", dtype=torch.int32).view(B, npb)
        seq = torch.full((B,), nk, device="cuda", dtype=torch.int32)
        S = best
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        mala.mala_decode_paged(wl.q, kp, vp, table, seq, wl.tau, bk, S, stats=st)
        s = st.cpu().tolist()
        ms = time_calls(lambda: mala.mala_decode_paged(wl.q, kp, vp, table, seq, wl.tau, bk, S), steps, warmup)
        gbs = (kbytes + s[3] * bk * d * 2) / (ms * 1e-3) / 1e9
        r = {"splits": S, "ms": round(ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
             "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
        res["paged"][f"page_size_{P}"] = r
        log(f"decode paged P={P}: {r}")
    del wl
    torch.cuda.empty_cache()
    return res


def decode_short_sub(mala, steps, warmup, nq=4, splits_list=(4, 16)):
    """Decode of a short query: the decode workload's shape (batch 64, GQA
    32/8, N_k = 131072, d 128, B_k 256, tau 0.05) with the nq newest tokens
    of every sequence as one query block per head (the G nq = 16 (head,
    token) pairs of a KV group are one MFMA's columns, so K is read once for
    all of them). Algorithmic bytes per launch = K + the V tiles loaded
    (q, o and the partials are below 0.1 percent of it)."""
    import torch
    import workloads
    wl = workloads.decode_cache(device="cuda", nq=nq)
    B, _, hq, d = wl.q.shape
    nk, hkv = wl.k.shape[1], wl.k.shape[2]
    bk = wl.block_k
    T = (nk + bk - 1) // bk
    kbytes = B * hkv * nk * d * 2
    res = {"workload": wl.name, "tau": wl.tau, "block_k": bk, "query_tokens": nq, "by_splits": {}}
    for S in splits_list:
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        o = torch.empty_like(wl.q)
        z = torch.empty((B, hq, nq), device="cuda", dtype=torch.float32)
        prob = mala.make_problem(wl.q, wl.k, wl.tau, 1, bk, nk - nq)
        ws = torch.empty(mala.mala_decode_workspace_size(prob, S), device="cuda", dtype=torch.uint8)
        mala.mala_decode(wl.q, wl.k, wl.v, wl.tau, bk, S, o=o, z=z, workspace=ws, stats=st)
        s = st.cpu().tolist()
        ms = time_calls(lambda: mala.mala_decode(wl.q, wl.k, wl.v, wl.tau, bk, S, o=o, z=z, workspace=ws),
                        steps, warmup)
        vbytes = s[3] * bk * d * 2
        gbs = (kbytes + vbytes) / (ms * 1e-3) / 1e9
        r = {"ms": round(ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
             "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
             "per_head_retain": round(s[1] / s[0], 4),
             "v_tile_load_fraction": round(s[3] / (B * hkv * T), 4),
             "bytes_per_launch": kbytes + vbytes,
             "query_rows_per_s": round(B * hq * nq / (ms * 1e-3), 1)}
        res["by_splits"][str(S)] = r
        log(f"decode short query ({nq} tokens) splits={S}: {r}")
    del wl
    torch.cuda.empty_cache()
    return res


def latent_decode_sub(mala, steps, warmup, splits_list=(2, 4, 8, 16), taus=(0.05, 1.0)):
    """Latent (MLA-shaped) decode: batch 64, 16 query heads sharing one
    cached row per position, N_k = 32768, d_qk 576, d_v 512, B_k 64. The
    value is part of the cached row, so every launch reads the whole cache
    (1152 bytes per key) whatever the decisions: algorithmic bytes =
    B N_k d_qk 2 (q, o and partials are below 0.1 percent of it)."""
    import torch
    import workloads
    wl = workloads.latent_decode(device="cuda")
    B, _, hq, dqk = wl.q.shape
    nk, dv, bk = wl.k.shape[1], wl.v.shape[3], wl.block_k
    cbytes = B * nk * dqk * 2
    res = {"workload": wl.name, "block_k": bk, "bytes_per_launch": cbytes}
    for tau in taus:
        by = {}
        best = None
        for S in splits_list:
            prob = mala.make_problem(wl.q, wl.k, tau, 1, bk, nk - 1)
            ws = torch.empty(mala.mala_decode_workspace_size(prob, S), device="cuda", dtype=torch.uint8)
            o = torch.empty((B, 1, hq, dv), device="cuda", dtype=wl.q.dtype)
            z = torch.empty((B, hq), device="cuda", dtype=torch.float32)
            st = torch.zeros(4, dtype=torch.int64, device="cuda")
            mala.mala_decode_latent(wl.q, wl.k, dv, tau, bk, S, o=o, z=z, workspace=ws, stats=st)
            s = st.cpu().tolist()
            ms = time_calls(lambda: mala.mala_decode_latent(wl.q, wl.k, dv, tau, bk, S, o=o, z=z,
                                                            workspace=ws), steps, warmup)
            gbs = cbytes / (ms * 1e-3) / 1e9
            r = {"ms": round(ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
                 "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                 "per_head_retain": round(s[1] / s[0], 4),
                 "pv_tile_fraction": round(s[3] / (s[0] / 16), 4),
                 "slots_per_query": round(s[2] / (B * hq), 1)}
            by[str(S)] = r
            log(f"latent decode tau={tau} splits={S}: {r}")
            if best is None or ms < by[str(best)]["ms"]:
                best = S
        res[str(tau)] = {"by_splits": by, "best_splits": best}
    del wl
    torch.cuda.empty_cache()
    # many heads (128 query heads per cached row, batch 16): the work per
    # byte of cache is 8x higher, so the executed FLOPs are reported too
    # (S on every tile, P V on each (tile, 16-head group) that retains)
    wl = workloads.latent_decode(device="cuda", batch=16, heads=128)
    B, _, hq, dqk = wl.q.shape
    nk, dv, bk = wl.k.shape[1], wl.v.shape[3], wl.block_k
    cbytes = B * nk * dqk * 2
    many = {"workload": wl.name, "tau": wl.tau, "by_splits": {}}
    for S in (4, 8, 16):
        prob = mala.make_problem(wl.q, wl.k, wl.tau, 1, bk, nk - 1)
        ws = torch.empty(mala.mala_decode_workspace_size(prob, S), device="cuda", dtype=torch.uint8)
        o = torch.empty((B, 1, hq, dv), device="cuda", dtype=wl.q.dtype)
        z = torch.empty((B, hq), device="cuda", dtype=torch.float32)
        st = torch.zeros(4, dtype=torch.int64, device="cuda")
        mala.mala_decode_latent(wl.q, wl.k, dv, wl.tau, bk, S, o=o, z=z, workspace=ws, stats=st)
        s = st.cpu().tolist()
        ms = time_calls(lambda: mala.mala_decode_latent(wl.q, wl.k, dv, wl.tau, bk, S, o=o, z=z, workspace=ws),
                        steps, warmup)
        ex = s[0] * 2.0 * bk * dqk + s[3] * 16 * 2.0 * bk * dv
        r = {"ms": round(ms, 4), "hbm_gbs_algorithmic": round(cbytes / (ms * 1e-3) / 1e9, 1),
             "executed_tflops": round(ex / ms / 1e9, 1),
             "pct_mfma_peak_executed": round(100 * ex / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
             "per_head_retain": round(s[1] / s[0], 4)}
        many["by_splits"][str(S)] = r
        log(f"latent decode 128 heads splits={S}: {r}")
    res["many_heads"] = many
    del wl
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tau", type=float, default=0.05)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true", help="skip the sub-benchmarks")
    ap.add_argument("--only", default="",
                    help="run only these sub-benchmarks (comma list of mha, gqa, local_band, page_band, "
                         "train_fidelity, varlen, latent, decode, decode_short, latent_decode), e.g. to "
                         "profile one "
                         "workload at a time")
    ap.add_argument("--decode-splits", default=DEFAULT_DECODE_SPLITS,
                    help="split counts of the decode sub-benchmarks (the short-query one runs 4 and 16 "
                         "unless this is given)")
    ap.add_argument("--sub-taus", default="",
                    help="run only these tau settings of the MHA, GQA, band, training-fidelity and latent "
                         "sub-benchmarks (comma list), e.g. to profile one setting alone")
    ap.add_argument("--no-step", action="store_true",
                    help="skip the timed training pass (profiling a sub-benchmark alone); the line then "
                         "carries no value")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 512 MiB device copy (untimed) so hardware byte "
                         "counters can be scaled against a transfer of known size")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this MALA build runs on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    # the training-pass workload is drawn on the host; the oracle's worker
    # processes are forked over it before anything touches the GPU, and the
    # GPU step runs on a device copy of the same tensors
    host_wl = host_workload(args.tau)
    oracle_pool = None
    if not args.no_cpu_baseline:
        oracle_pool = start_oracle_pool(host_wl)

    import torch
    import block_sparse_causal_tile_amd as mala
    import workloads

    if not os.path.exists(mala.lib_path()):
        from block_sparse_causal_tile_amd import build
        build.build()
    mala.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy:
        src = torch.ones(256 * 1024 * 1024, device=dev, dtype=torch.bfloat16)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 536870912 bytes read, 536870912 bytes written")
        del src, dst

    tau = args.tau
    wl = host_wl
    wl.q, wl.k, wl.v, wl.do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    bq, bk = wl.block_q, wl.block_k
    B, nq, hq, d = wl.q.shape
    nk = wl.k.shape[1]
    off = nk - nq
    log(f"workload {wl.name}: q {tuple(wl.q.shape)} bf16, B_q=B_k={bq}, tau {tau}")

    o = torch.empty_like(wl.q)
    z = torch.empty((B, hq, nq), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(wl.q), torch.empty_like(wl.k), torch.empty_like(wl.v)
    prob = mala.make_problem(wl.q, wl.k, tau, bq, bk)
    ws = torch.empty(mala.mala_bwd_workspace_size(prob), device=dev, dtype=torch.uint8)

    # untimed pass with the debug counters on: skip rates and slots
    st_f = torch.zeros(4, dtype=torch.int64, device=dev)
    st_b = torch.zeros(4, dtype=torch.int64, device=dev)
    if not args.no_step:
        mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z, stats=st_f)
        mala.mala_bwd(wl.q, wl.k, wl.v, o, wl.do, z, tau, bq, bk, dq=dq, dk=dk, dv=dv, workspace=ws,
                      stats=st_b)
        torch.cuda.synchronize()
    sf, sb = st_f.cpu().tolist(), st_b.cpu().tolist()

    def fwd():
        mala.mala_fwd(wl.q, wl.k, wl.v, tau, bq, bk, o=o, z=z)

    def bwd():
        mala.mala_bwd(wl.q, wl.k, wl.v, o, wl.do, z, tau, bq, bk, dq=dq, dk=dk, dv=dv, workspace=ws)

    achieved = None
    if args.no_step:
        out = {"metric": "MALA fwd/bwd dense-equiv TFLOP/s + skip rate + % MFMA peak, 1 MI355X",
               "value": None, "note": "--no-step: sub-benchmarks only (profiling)"}
    else:
        for _ in range(args.warmup):
            fwd()
            bwd()
        torch.cuda.synchronize()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        for e0, e1, e2 in ev:
            e0.record()
            fwd()
            e1.record()
            bwd()
            e2.record()
        torch.cuda.synchronize()
        fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
        bwd_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
        step_ms = sum(a.elapsed_time(c) for a, _, c in ev) / args.steps
        log(f"step {step_ms:.3f} ms (fwd {fwd_ms:.3f}, bwd {bwd_ms:.3f})")

        pairs = B * hq * legal_pairs(nq, nk, off)
        tile_flops = 2.0 * bq * bk * d
        dense_f, dense_b = pairs * 4.0 * d, pairs * 10.0 * d
        # executed: QK on every legal tile; forward PV per retained tile;
        # backward dP, dV, dK, dQ per retained tile
        exec_f = (sf[0] + sf[1]) * tile_flops
        exec_b = (sb[0] + 4 * sb[1]) * tile_flops
        value = (dense_f + dense_b) / (step_ms * 1e-3) / 1e12
        kern = {"mala_fwd (fwd_bf16_kernel<128, 128, 64, 64, false>)":
                    (fwd_ms, exec_f, ["fwd_bf16_kernel<128, 128, 64, 64, false>"]),
                "mala_bwd (bwd_absmax_kernel + bwd_prep_kernel + bwd_main_kernel<128>)":
                    (bwd_ms, exec_b, ["bwd_absmax_kernel", "bwd_prep_kernel", "bwd_main_kernel<128>"])}
        dom = max(kern, key=lambda n: kern[n][0])
        achieved = kern[dom][1] / (kern[dom][0] * 1e-3) / 1e12
        traffic = measured_traffic(kern[dom][2])
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": dom, "algorithmic_flops_per_launch": kern[dom][1],
                "avg_launch_ms": round(kern[dom][0], 4)}

        def pass_report(ms, dense, ex, s):
            return {"ms": round(ms, 4), "dense_equiv_tflops": round(dense / ms / 1e9, 2),
                    "executed_tflops": round(ex / ms / 1e9, 2),
                    "pct_mfma_peak_executed": round(100 * ex / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                    "skip_rate": round(1 - s[1] / s[0], 4),
                    "slots_per_query": round(s[2] / (B * hq * nq), 2),
                    "legal_tiles": s[0], "retained_tiles": s[1]}

        out = {
            "metric": "MALA fwd/bwd dense-equiv TFLOP/s + skip rate + % MFMA peak, 1 MI355X",
            "value": round(value, 2),
            "unit": "TFLOP/s (dense-equivalent)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(step_ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{wl.name} forward+backward (MALA training pass)",
                       "batch": B, "heads": hq, "seq_len": nq, "head_dim": d,
                       "block_q": bq, "block_k": bk, "tau": tau, "parallelism": "none (1 GPU)"},
            "fwd": pass_report(fwd_ms, dense_f, exec_f, sf),
            "bwd": pass_report(bwd_ms, dense_b, exec_b, sb),
            "roofline": roof,
        }
    if not args.no_sub:
        only = set(args.only.split(",")) if args.only else None
        splits = tuple(int(x) for x in args.decode_splits.split(","))

        def want(name):
            return only is None or name in only

        sub_taus = None if not args.sub_taus else [float(x) for x in args.sub_taus.split(",")]

        def pick(taus):
            # the sub-benchmark's tau settings, or those of them --sub-taus names
            return tuple(taus) if sub_taus is None else tuple(t for t in taus if t in sub_taus)

        subs = {}
        if want("mha"):
            w2 = workloads.mha_temperature(device=dev, with_grad=False)
            subs["fwd_" + w2.name] = fwd_sub(mala, w2, pick((0.01, 0.05, 0.2, 1.0)), args.steps, args.warmup)
            del w2
        if want("gqa"):
            w3 = workloads.gqa_sink_window(device=dev)
            subs["fwd_" + w3.name] = fwd_sub(mala, w3, pick((w3.tau,)), args.steps, args.warmup)
            del w3
        torch.cuda.empty_cache()
        if want("local_band"):
            w4 = workloads.local_band(device=dev, heads=hq, n=nq, d=d, block=bq)
            subs["skip_fidelity_" + w4.name] = skip_fidelity_sub(mala, w4, tau, args.steps, args.warmup,
                                                                 pick((tau, 0.0)))
            del w4
        if want("page_band"):
            # the page's allocation level: ~1,000 forward post-score slots per query
            w6 = workloads.page_band(device=dev, heads=hq, n=nq, d=d, block=bq)
            subs["skip_fidelity_" + w6.name] = skip_fidelity_sub(mala, w6, tau, args.steps, args.warmup,
                                                                 pick((tau, 0.0)))
            del w6
        if want("train_fidelity"):
            # the training-pass workload itself (its Gaussian scores retain ~every tile)
            w5 = workloads.Workload(wl.name, wl.q, wl.k, wl.v, tau, bq, bk, off)
            subs["skip_fidelity_" + wl.name] = skip_fidelity_sub(mala, w5, tau, args.steps, args.warmup,
                                                                 pick((tau, 0.0)))
            del w5
        torch.cuda.empty_cache()
        if want("varlen"):
            subs["fwd_varlen_chunked_prefill"] = varlen_sub(mala, args.steps, args.warmup)
            torch.cuda.empty_cache()
        if want("latent"):
            subs["latent_mla_shape"] = latent_sub(mala, args.steps, args.warmup, taus=pick((0.0, 0.05, 1.0)))
            torch.cuda.empty_cache()
        if want("decode"):
            subs["decode"] = decode_sub(mala, max(5, args.steps // 2), 2, splits_list=splits)
            torch.cuda.empty_cache()
        if want("decode_short"):
            subs["decode_short_query"] = decode_short_sub(
                mala, max(5, args.steps // 2), 2,
                splits_list=splits if args.decode_splits != DEFAULT_DECODE_SPLITS else (4, 16))
            torch.cuda.empty_cache()
        if want("latent_decode"):
            subs["decode_latent_mla_shape"] = latent_decode_sub(mala, max(5, args.steps // 2), 2)
        out["sub_benchmarks"] = subs
        if only is None:
            att = attainable_peaks(dev)
            if achieved is not None:
                att["step_kernel_frac_of_gemm"] = round(achieved / att["bf16_gemm_8192_tflops"], 4)
            dec = subs["decode"]
            best = dec["by_splits"][str(dec["best_splits"])]["hbm_gbs_algorithmic"]
            att["decode_frac_of_copy"] = round(best / att["device_copy_1gib_gbs"], 4)
            out["attainable"] = att
    if not args.no_cpu_baseline:
        pool, n_workers, shape, nk_h = oracle_pool
        out["cpu_baseline"] = cpu_baseline(pool, n_workers, shape, nk_h, tau, bq, bk, args.cpu_seconds)
        pool.close()
        pool.join()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
