"""Seeded synthetic inputs shaped like the MALA page's workloads.

This module builds input tensors only: it holds none of the attention method's
arithmetic, and both the HIP library's tests/bench and the CPU oracle read
what it produces (the oracle receives exact host copies of the device tensors,
so parity never depends on two RNGs agreeing).

The pages measure on activations of trained GQA models (8 KV heads, head
width 128, contexts of 1K-131K tokens) over language-modelling corpora; none
of that is available here, so each recipe below is a seeded stand-in with the
same shapes and the structure the pages name: sharp rows (temperature),
shared low-rank key structure, attention sinks, a local window bias and a few
heavy keys. Every tensor uses the BSHD layout [batch, seq, heads, head_dim]
with the softmax scale already folded into q.

Seeds: workload n uses ``BASE_SEED + n`` unless a seed is passed explicitly.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BASE_SEED = 42
SWEEP_SEEDS = (0, 42, 233, 666, 1234)


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    tau: float
    block_q: int
    block_k: int
    causal_offset: int
    do: torch.Tensor | None = None
    extra: dict = field(default_factory=dict)

    @property
    def dims(self):
        B, nq, hq, d = self.q.shape
        return dict(batch=B, seqlen_q=nq, heads_q=hq, head_dim=d,
                    seqlen_k=self.k.shape[1], heads_kv=self.k.shape[2])


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _rand(shape, g, device):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def _randint(hi, shape, g, device):
    return torch.randint(0, hi, shape, generator=g, device=device)


def _plant_heavy_keys(k, q_src, n_heavy, g, device, per_head_group=None):
    """Overwrite n_heavy key rows with 4x a random query row (per batch and
    KV head): the key then scores ~4|q|^2 against that query."""
    B, nk, hkv, d = k.shape
    hq = q_src.shape[2]
    group = hq // hkv
    for b in range(B):
        for g_ in range(hkv):
            pos = torch.randperm(nk, generator=g, device=device)[:n_heavy]
            rows = _randint(q_src.shape[1], (n_heavy,), g, device)
            heads = g_ * group + _randint(group, (n_heavy,), g, device)
            k[b, pos, g_] = 4.0 * q_src[b, rows, heads]
    return k


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def small_fp32(device="cpu", seed=None, n=512, d=64, block=64, tau=0.05, n_heavy=4):
    """Forward, 1 batch x 1 head, N=512, d=64, B_q=B_k=64, fp32, tau=0.05.

    q, k, v ~ N(0, 1); q <- 3 q / sqrt(d) (scale folded in, rows sharpened);
    4 heavy keys at distinct random positions are set to 4x a random
    (scaled) query row."""
    g = _gen(device, BASE_SEED + 1 if seed is None else seed)
    q = 3.0 * _randn((1, n, 1, d), g, device) / math.sqrt(d)
    k = _randn((1, n, 1, d), g, device)
    v = _randn((1, n, 1, d), g, device)
    k = _plant_heavy_keys(k, q, n_heavy, g, device)
    return Workload("mala-fwd-fp32-n512-d64", q, k, v, tau, block, block, 0)


def _lowrank_keys(B, n, h, d, g, device, struct_len=128, rank=8):
    """K = N(0,1) + Z_{floor(pos / 128)} R with Z ~ N(0,1) [n/128, 8] and
    R ~ N(0,1)/sqrt(8) [8, d], shared by the heads of a batch element."""
    k = _randn((B, n, h, d), g, device)
    nb = (n + struct_len - 1) // struct_len
    for b in range(B):
        zr = _randn((nb, rank), g, device) @ (_randn((rank, d), g, device) / math.sqrt(rank))
        k[b] += zr.repeat_interleave(struct_len, dim=0)[:n, None, :]
    return k


def mha_temperature(device="cpu", seed=None, batch=2, heads=32, n=4096, d=128,
                    block=128, tau=0.05, dtype=torch.bfloat16, with_grad=True,
                    temperature=None):
    """Forward, batch 2, 32 heads (MHA), N=4096, d=128, B_q=B_k=128, bf16.

    q, k, v ~ N(0, 1); each head h gets a temperature T_h ~ U[1, 4] (or the
    fixed ``temperature``) and q_h <- T_h q_h / sqrt(d); k receives a shared
    rank-8 component constant over runs of 128 positions (block structure).
    ``with_grad`` also draws dO ~ N(0, 1)."""
    g = _gen(device, BASE_SEED + 2 if seed is None else seed)
    if temperature is None:
        t = 1.0 + 3.0 * _rand((heads,), g, device)
    else:
        t = torch.full((heads,), float(temperature), device=device)
    q = _randn((batch, n, heads, d), g, device) * (t[None, None, :, None] / math.sqrt(d))
    k = _lowrank_keys(batch, n, heads, d, g, device)
    v = _randn((batch, n, heads, d), g, device)
    do = _randn((batch, n, heads, d), g, device) if with_grad else None
    cast = (lambda x: x.to(dtype)) if dtype is not None else (lambda x: x)
    return Workload(f"mala-mha-b{batch}-h{heads}-n{n}-d{d}", cast(q), cast(k), cast(v),
                    tau, block, block, 0, do=None if do is None else cast(do),
                    extra={"temperature": t.cpu()})


def gqa_sink_window(device="cpu", seed=None, heads_q=32, heads_kv=8, n=16384, d=128,
                    block_q=128, block_k=64, tau=0.05, dtype=torch.bfloat16,
                    window=512, window_bias=2.0, sink_score=6.0, n_sinks=4,
                    rope_pairs=16):
    """Forward, batch 1, GQA 32 query / 8 KV heads, N=16384, d=128, B_q=128,
    B_k=64, bf16, tau=0.05.

    * generic part: the last d - 2*rope_pairs dims of q, k are N(0,1) with q
      scaled by 1/sqrt(width), so generic scores are ~N(0, 1);
    * local window: the first 2*rope_pairs dims of q and k hold the same
      constant vector rotated by position (angle w_t * pos for pair t, random
      frequencies w_t in (0, pi/window)), so q.k gains
      a^2 sum_t cos(w_t (q - k)); a^2 is set so the mean bias over
      0 <= q - k < window is ``window_bias`` (beyond it the cosines
      decorrelate and the mean bias is near 0);
    * sinks: keys 0..3 get a large component 4*sqrt(width)*u_g along a
      per-KV-head unit direction u_g and every query of the group gets
      c*u_g, with c chosen so the sink score is ~``sink_score``;
    * v ~ N(0, 1).
    """
    g = _gen(device, BASE_SEED + 3 if seed is None else seed)
    rd = 2 * rope_pairs
    w = d - rd
    q = torch.zeros((1, n, heads_q, d), device=device)
    k = torch.zeros((1, n, heads_kv, d), device=device)
    q[..., rd:] = _randn((1, n, heads_q, w), g, device) / math.sqrt(w)
    k[..., rd:] = _randn((1, n, heads_kv, w), g, device)
    # local window through a rotation of a constant vector
    freqs = (math.pi / window) * _rand((rope_pairs,), g, device)
    delta = torch.arange(window, device=device, dtype=torch.float32)
    mean_cos = torch.cos(delta[:, None] * freqs[None, :]).sum(dim=1).mean()
    amp = math.sqrt(window_bias / float(mean_cos))
    pos = torch.arange(n, device=device, dtype=torch.float32)
    ang = pos[:, None] * freqs[None, :]
    rot = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).reshape(n, rd) * amp
    q[0, :, :, :rd] = rot[:, None, :]
    k[0, :, :, :rd] = rot[:, None, :]
    # sinks
    group = heads_q // heads_kv
    u = _randn((heads_kv, w), g, device)
    u = u / u.norm(dim=1, keepdim=True)
    ksink = 4.0 * math.sqrt(w)
    c = sink_score / ksink
    k[0, :n_sinks, :, rd:] += ksink * u[None, :, :]
    q[0, :, :, rd:] += c * u.repeat_interleave(group, dim=0)[None, :, :]
    v = _randn((1, n, heads_kv, d), g, device)
    return Workload(f"mala-gqa-h{heads_q}x{heads_kv}-n{n}-d{d}-sink-window",
                    q.to(dtype), k.to(dtype), v.to(dtype), tau, block_q, block_k, 0,
                    extra={"rope_amp": amp, "freqs": freqs.cpu()})


def mha_backward(device="cpu", seed=None, batch=1, heads=16, n=8192, d=128, block=64,
                 tau=0.05, dtype=torch.bfloat16):
    """Backward, batch 1, 16 heads, N=8192, d=128, B_q=B_k=64, bf16: the
    ``mha_temperature`` recipe with temperature 2 for every head, plus
    dO ~ N(0, 1)."""
    wl = mha_temperature(device=device, seed=BASE_SEED + 4 if seed is None else seed,
                         batch=batch, heads=heads, n=n, d=d, block=block, tau=tau,
                         dtype=dtype, with_grad=True, temperature=2.0)
    wl.name = f"mala-bwd-b{batch}-h{heads}-n{n}-d{d}"
    return wl


def decode_cache(device="cpu", seed=None, batch=64, heads_q=32, heads_kv=8, nk=131072,
                 d=128, block_k=256, tau=0.05, dtype=torch.bfloat16, n_sinks=4,
                 n_heavy=32, sink_norm=8.0, nq=1):
    """Single-token decode, batch 64, 32 query / 8 KV heads, N_k=131072,
    d=128, B_k=256, bf16 cache, L_0 = N_k, tau=0.05.

    q ~ 3 N(0,1) / sqrt(d); k, v ~ N(0, 1); per (batch, KV head) the first 4
    keys are sinks ``sink_norm * u_g`` along a unit direction u_g that every
    query of the group also leans on (q += u_g), and 32 uniformly drawn
    positions get k = 4x a random query of the group. Generated one batch
    row at a time to bound the fp32 staging memory. ``nq`` > 1 gives a short
    query of nq tokens (the newest nq positions of the cache, drawn the same
    way; nq = 1 draws exactly the single-token workload)."""
    g = _gen(device, BASE_SEED + 5 if seed is None else seed)
    group = heads_q // heads_kv
    q = 3.0 * _randn((batch, nq, heads_q, d), g, device) / math.sqrt(d)
    u = _randn((batch, heads_kv, d), g, device)
    u = u / u.norm(dim=-1, keepdim=True)
    q += u.repeat_interleave(group, dim=1)[:, None]
    k = torch.empty((batch, nk, heads_kv, d), device=device, dtype=dtype)
    v = torch.empty((batch, nk, heads_kv, d), device=device, dtype=dtype)
    for b in range(batch):
        kb = _randn((1, nk, heads_kv, d), g, device)
        kb[0, :n_sinks] = sink_norm * u[b][None, :, :]
        kb = _plant_heavy_keys(kb, q[b:b + 1], n_heavy, g, device)
        k[b] = kb[0].to(dtype)
        v[b] = _randn((nk, heads_kv, d), g, device).to(dtype)
    qc = q.to(dtype)
    name = f"mala-decode-b{batch}-h{heads_q}x{heads_kv}-nk{nk}-d{d}" + (f"-nq{nq}" if nq > 1 else "")
    return Workload(name, qc, k, v, tau, nq, block_k, nk - nq)


def uniform(device="cpu", seed=0, batch=1, heads_q=2, heads_kv=None, nq=256, nk=None,
            d=64, scale=1.0, dtype=torch.float32):
    """Plain N(0,1) tensors (q scaled by ``scale``/sqrt(d)) for edge-case and
    ragged-shape tests."""
    heads_kv = heads_q if heads_kv is None else heads_kv
    nk = nq if nk is None else nk
    g = _gen(device, seed)
    q = scale * _randn((batch, nq, heads_q, d), g, device) / math.sqrt(d)
    k = _randn((batch, nk, heads_kv, d), g, device)
    v = _randn((batch, nk, heads_kv, d), g, device)
    do = _randn((batch, nq, heads_q, d), g, device)
    cast = (lambda x: x.to(dtype))
    return cast(q), cast(k), cast(v), cast(do)


def late_sink(device="cpu", seed=0, batch=1, heads=2, n=700, d=128, gaps=(15.0, 4.0),
              dtype=torch.bfloat16):
    """Generic scores ~ N(0, 1) plus four sink keys (positions 0-3) that every
    query of head h scores about ``gaps[h] + 3.5`` (the generic maximum over a
    few hundred keys is about 3): the diagonal-first walk meets them last, so
    a row's largest score arrives at its final tile, by far (gap 15) or by
    a little less than the online softmax's rescale threshold of 8 / log2(e)
    (gap 4). q = N(0, 1) / d^(1/4) + u_h, k = N(0, 1) / d^(1/4) except
    k_sink = (gap_h + 3.5) u_h + N(0, 1) / d^(1/4), u_h a random unit vector;
    v, dO ~ N(0, 1). One KV head per query head."""
    assert len(gaps) == heads
    g = _gen(device, seed)
    r = d ** 0.25
    u = _randn((heads, d), g, device)
    u = u / u.norm(dim=-1, keepdim=True)
    q = _randn((batch, n, heads, d), g, device) / r + u[None, None]
    k = _randn((batch, n, heads, d), g, device) / r
    c = torch.tensor([x + 3.5 for x in gaps], device=device, dtype=torch.float32)
    k[:, :4] += (c[:, None] * u)[None, None]
    v = _randn((batch, n, heads, d), g, device)
    do = _randn((batch, n, heads, d), g, device)
    return q.to(dtype), k.to(dtype), v.to(dtype), do.to(dtype)


def local_band(device="cpu", seed=None, batch=1, heads=4, n=4096, d=128, block=64, tau=0.05,
               width=48.0, amplitude=24.0, noise=1.0, key_noise=1.0, dtype=torch.bfloat16):
    """Attention concentrated near the diagonal (the locality that makes the
    page visit tiles diagonal-first): q_t . k_s = amplitude * mean_j
    cos(w_j (t - s)) + noise, with random Fourier frequencies w_j ~
    N(0, 1 / width^2) per head (j < d/2), so the structured part is a
    Gaussian-kernel band of width ``width`` tokens and far tiles carry
    vanishing probability. k_s = [cos(w_j s), sin(w_j s)]_j + key_noise N(0, 1)
    (every key also carries content of its own, so neighbouring keys are not
    near-copies), q_t = amplitude / (d/2) [cos(w_j t), sin(w_j t)]_j
    + noise N(0,1) / sqrt(d / 2); v, dO ~ N(0, 1)."""
    g = _gen(device, BASE_SEED + 6 if seed is None else seed)
    half = d // 2
    w = _randn((heads, half), g, device) / width
    pos = torch.arange(n, device=device, dtype=torch.float32)
    ang = pos[:, None, None] * w[None, :, :]                      # [n, heads, half]
    feat = torch.stack((torch.cos(ang), torch.sin(ang)), dim=-1).reshape(n, heads, d)
    k = feat[None].expand(batch, n, heads, d) + key_noise * _randn((batch, n, heads, d), g, device)
    q = amplitude / half * feat[None].expand(batch, n, heads, d) \
        + noise * _randn((batch, n, heads, d), g, device) / math.sqrt(half)
    v = _randn((batch, n, heads, d), g, device)
    do = _randn((batch, n, heads, d), g, device)
    return Workload(f"mala-local-b{batch}-h{heads}-n{n}-d{d}", q.to(dtype), k.to(dtype), v.to(dtype),
                    tau, block, block, 0, do=do.to(dtype))


def page_band(device="cpu", seed=None, batch=1, heads=16, n=8192, d=128, block=64, tau=0.05,
              width=900.0, amplitude=24.0, dtype=torch.bfloat16):
    """The ``local_band`` recipe with a band wide enough that MALA's forward
    keeps about 1,000 post-score key slots per query at N = 8192, tau = 0.05
    (882 to 1,146 on four sampled heads in the oracle) - the allocation
    level of the MALA page's runs (about 1,024 forward slots per query in its
    operator benchmark; 906.78 forward / 896.74 backward in its 4K training
    run). Batch 1, 16 heads, d = 128, 64 x 64 tiles, bf16; dO ~ N(0, 1)."""
    wl = local_band(device=device, seed=BASE_SEED + 7 if seed is None else seed, batch=batch, heads=heads, n=n,
                    d=d, block=block, tau=tau, width=width, amplitude=amplitude, dtype=dtype)
    wl.name = f"mala-band1k-b{batch}-h{heads}-n{n}-d{d}"
    return wl


def latent_mqa(device="cpu", seed=None, batch=1, heads=16, n=4096, d_qk=576, d_v=512, block=64,
               tau=0.05, amplitude=24.0, width=48.0, dtype=torch.bfloat16):
    """Latent (MLA-shaped) attention: every query head scores one shared
    cached row per position, kv_s = [c_s, r_s] with a d_v-wide latent c_s and
    a (d_qk - d_v)-wide positional part r_s, and the value is the latent
    itself (v_s = c_s, the first d_v columns of the row). Defaults: batch 1,
    16 query heads, N = 4096, d_qk = 576, d_v = 512, 64 x 64 tiles, bf16.

    c ~ N(0,1) plus a shared rank-8 component constant over runs of 128
    positions; r_s = [cos(w_j s), sin(w_j s)]_j + N(0,1) with frequencies
    w_j ~ N(0, 1/width^2); per head h a temperature T_h ~ U[1, 4] and
    q_t = [T_h N(0,1) / sqrt(d_qk),
           amplitude / (r/2) [cos(w_j t), sin(w_j t)]_j + N(0,1) / sqrt(r/2)],
    so a score is a Gaussian content term plus ``amplitude`` times a
    Gaussian-kernel band around the diagonal (``amplitude`` 0: no band).
    At the defaults about half the legal tiles fall below tau = 0.05 (about
    1,000 post-score slots per query at N = 4096) and three quarters below
    tau = 1.
    ``v`` is the latent view of ``k`` (no copy)."""
    g = _gen(device, BASE_SEED + 7 if seed is None else seed)
    rdim = d_qk - d_v
    half = rdim // 2
    t = 1.0 + 3.0 * _rand((heads,), g, device)
    c = _lowrank_keys(batch, n, 1, d_v, g, device)
    w = _randn((half,), g, device) / width
    pos = torch.arange(n, device=device, dtype=torch.float32)
    ang = pos[:, None] * w[None, :]
    feat = torch.stack((torch.cos(ang), torch.sin(ang)), dim=-1).reshape(n, rdim)
    r = feat[None, :, None, :].expand(batch, n, 1, rdim) + _randn((batch, n, 1, rdim), g, device)
    kv = torch.cat((c, r), dim=-1).to(dtype)
    qc = _randn((batch, n, heads, d_v), g, device) * (t[None, None, :, None] / math.sqrt(d_qk))
    qr = amplitude / half * feat[None, :, None, :].expand(batch, n, heads, rdim) \
        + _randn((batch, n, heads, rdim), g, device) / math.sqrt(half)
    q = torch.cat((qc, qr), dim=-1).to(dtype)
    return Workload(f"mala-latent-b{batch}-h{heads}-n{n}-dqk{d_qk}-dv{d_v}", q, kv, kv[..., :d_v],
                    tau, block, block, 0, extra={"temperature": t.cpu(), "d_v": d_v})


def latent_decode(device="cpu", seed=None, batch=64, heads=16, nk=32768, d_qk=576, d_v=512,
                  block_k=64, tau=0.05, amplitude=24.0, width=48.0, n_sinks=4, sink_score=6.0,
                  dtype=torch.bfloat16):
    """Single-token decode on latent (MLA-shaped) attention. Defaults: batch
    64, 16 query heads sharing one cached row per position, N_k = 32768,
    d_qk = 576, d_v = 512, B_k = 64, bf16 cache, L_0 = N_k, tau = 0.05.

    Cached rows as in ``latent_mqa`` (a d_v-wide latent with shared rank-8
    structure and a positional part [cos(w_j s), sin(w_j s)] + N(0,1));
    the query is the token at position N_k - 1, drawn as there (content
    T_h N(0,1) / sqrt(d_qk) with T_h ~ U[1, 4], positional part centred on
    its own position, so recent keys gain up to ``amplitude``), plus
    attention sinks: the latent of the first ``n_sinks`` keys is
    8 u_b along a unit direction u_b of the batch row and every head's query
    content gains (sink_score / 8) u_b, so the sinks score about
    ``sink_score``. Generated one batch row at a time to bound the fp32
    staging memory. ``v`` is the latent view of ``k`` (no copy)."""
    g = _gen(device, BASE_SEED + 8 if seed is None else seed)
    rdim = d_qk - d_v
    half = rdim // 2
    t = 1.0 + 3.0 * _rand((heads,), g, device)
    w = _randn((half,), g, device) / width
    pos = torch.arange(nk, device=device, dtype=torch.float32)
    ang = pos[:, None] * w[None, :]
    feat = torch.stack((torch.cos(ang), torch.sin(ang)), dim=-1).reshape(nk, rdim)
    u = _randn((batch, d_v), g, device)
    u = u / u.norm(dim=-1, keepdim=True)
    kv = torch.empty((batch, nk, 1, d_qk), device=device, dtype=dtype)
    for b in range(batch):
        c = _lowrank_keys(1, nk, 1, d_v, g, device)
        c[0, :n_sinks, 0] = 8.0 * u[b]
        r = feat[None, :, None, :] + _randn((1, nk, 1, rdim), g, device)
        kv[b] = torch.cat((c, r), dim=-1)[0].to(dtype)
    qc = _randn((batch, 1, heads, d_v), g, device) * (t[None, None, :, None] / math.sqrt(d_qk))
    qc = qc + (sink_score / 8.0) * u[:, None, None, :]
    qr = amplitude / half * feat[nk - 1][None, None, None, :].expand(batch, 1, heads, rdim) \
        + _randn((batch, 1, heads, rdim), g, device) / math.sqrt(half)
    q = torch.cat((qc, qr), dim=-1).to(dtype)
    return Workload(f"mala-latent-decode-b{batch}-h{heads}-nk{nk}-dqk{d_qk}-dv{d_v}", q, kv,
                    kv[..., :d_v], tau, 1, block_k, nk - 1,
                    extra={"temperature": t.cpu(), "d_v": d_v})


WORKLOADS = {
    "small_fp32": small_fp32,
    "mha_temperature": mha_temperature,
    "gqa_sink_window": gqa_sink_window,
    "mha_backward": mha_backward,
    "decode_cache": decode_cache,
    "local_band": local_band,
    "latent_mqa": latent_mqa,
    "latent_decode": latent_decode,
}
