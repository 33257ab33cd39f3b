"""Seeded random sweep over problem shapes: forward, backward, packed
forward and split-KV decode against the oracle on configurations drawn from
the supported space (batch, GQA ratio, lengths, causal offset, tile sizes,
head dim, tau, input scale), a few dozen in total. Every case prints its
parameters before it runs."""

import numpy as np
import pytest
import torch

import workloads
from parity import (assert_decode, assert_forward, check_backward, decode_parity, decode_short_parity,
                    forward_parity, fresh_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def hip_bwd(mala, q, k, v, do, tau, off):
    """A launcher of the HIP backward (64 x 64 tiles) on given (o, z)."""
    B, nq, hq, _ = q.shape
    nk = k.shape[1]

    def run(o, z):
        mb = fresh_mask(B, hq, nq, nk, 64, 64)
        mq = fresh_mask(B, hq, nq, nk, 64, 64)
        sb = torch.zeros(4, dtype=torch.int64, device="cuda")
        dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, tau, 64, 64, causal_offset=off, stats=sb, tile_mask=mb,
                                   tile_mask_dq=mq)
        return dq, dk, dv, mb, mq, sb
    return run


def draw(rng):
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4]))
    nq = int(rng.integers(1, 420))
    nk = nq + int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    return dict(batch=int(rng.integers(1, 3)), hkv=hkv, hq=hkv * group, nq=nq, nk=nk,
                off=nk - nq - int(rng.integers(0, nk - nq + 1)) if nk > nq and rng.random() < 0.3 else nk - nq,
                d=int(rng.choice([64, 128])), bq=int(rng.choice([64, 128])), bk=int(rng.choice([64, 128])),
                tau=float(rng.choice([0.0, 0.01, 0.05, 0.3, 1.0, 3.0])), scale=float(rng.choice([1.0, 4.0, 8.0])),
                seed=int(rng.integers(1 << 30)))


def inputs(c):
    return workloads.uniform(device="cuda", seed=c["seed"], batch=c["batch"], heads_q=c["hq"], heads_kv=c["hkv"],
                             nq=c["nq"], nk=c["nk"], d=c["d"], scale=c["scale"], dtype=torch.bfloat16)


@pytest.mark.parametrize("case", range(12))
def test_sweep_forward_backward(mala, case):
    c = draw(np.random.default_rng(1000 + case))
    print("case", case, c, flush=True)
    q, k, v, do = inputs(c)
    B, nq, hq, nk = c["batch"], c["nq"], c["hq"], c["nk"]
    mf = fresh_mask(B, hq, nq, nk, c["bq"], c["bk"])
    o, z = mala.mala_fwd(q, k, v, c["tau"], c["bq"], c["bk"], causal_offset=c["off"], tile_mask=mf)
    torch.cuda.synchronize()
    rep = forward_parity(q, k, v, c["tau"], c["bq"], c["bk"], c["off"], o, z, mf)
    print(rep)
    assert_forward(rep, fp32=False)
    if c["bq"] == 64 and c["bk"] == 64:  # the backward's tile size
        mb = fresh_mask(B, hq, nq, nk, 64, 64)
        dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, c["tau"], 64, 64, causal_offset=c["off"], tile_mask=mb)
        torch.cuda.synchronize()
        check_backward(hip_bwd(mala, q, k, v, do, c["tau"], c["off"]), q, k, v, do, c["tau"], 64, 64, c["off"], mf,
                       e2e=(dq, dk, dv, mb))


@pytest.mark.parametrize("case", range(8))
def test_sweep_backward_tiles(mala, case):
    """Backward-focused draws (64 x 64 tiles, the backward's size)."""
    c = draw(np.random.default_rng(2000 + case))
    c.update(bq=64, bk=64)
    print("case", case, c, flush=True)
    q, k, v, do = inputs(c)
    B, nq, hq, nk = c["batch"], c["nq"], c["hq"], c["nk"]
    mf = fresh_mask(B, hq, nq, nk, 64, 64)
    mb = fresh_mask(B, hq, nq, nk, 64, 64)
    o, z = mala.mala_fwd(q, k, v, c["tau"], 64, 64, causal_offset=c["off"], tile_mask=mf)
    dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, c["tau"], 64, 64, causal_offset=c["off"], tile_mask=mb)
    torch.cuda.synchronize()
    check_backward(hip_bwd(mala, q, k, v, do, c["tau"], c["off"]), q, k, v, do, c["tau"], 64, 64, c["off"], mf,
                   e2e=(dq, dk, dv, mb))


@pytest.mark.parametrize("case", range(6))
def test_sweep_decode(mala, case):
    rng = np.random.default_rng(3000 + case)
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    nk = int(rng.integers(1, 3000))
    bk = int(rng.choice([64, 128, 256]))
    T = -(-nk // bk)
    splits = int(rng.integers(1, T + 1))
    tau = float(rng.choice([0.0, 0.05, 0.5, 2.0]))
    seed = int(rng.integers(1 << 30))
    print("case", case, dict(hkv=hkv, group=group, nk=nk, bk=bk, splits=splits, tau=tau, seed=seed), flush=True)
    q, k, v, _ = workloads.uniform(device="cuda", seed=seed, batch=2, heads_q=hkv * group, heads_kv=hkv, nq=1,
                                   nk=nk, d=128, scale=4.0, dtype=torch.bfloat16)
    mask = torch.full((2, hkv * group, T), 255, dtype=torch.uint8, device="cuda")
    o, z = mala.mala_decode(q, k, v, tau, bk, num_splits=splits, tile_mask=mask)
    torch.cuda.synchronize()
    rep = decode_parity(q, k, v, tau, bk, splits, o, z, mask)
    print(rep)
    assert_decode(rep)


@pytest.mark.parametrize("case", range(8))
def test_sweep_decode_short(mala, case):
    """Short queries: N_q newest tokens (G N_q <= 16), lengths down to N_k = N_q."""
    rng = np.random.default_rng(3500 + case)
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    nq = int(rng.integers(1, 16 // group + 1))
    nk = nq + int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(1, 3000))], p=[0.25, 0.25, 0.5]))
    bk = int(rng.choice([64, 128, 256]))
    T = -(-nk // bk)
    splits = int(rng.integers(1, T + 1))
    tau = float(rng.choice([0.0, 0.05, 0.5, 2.0]))
    seed = int(rng.integers(1 << 30))
    print("case", case, dict(hkv=hkv, group=group, nq=nq, nk=nk, bk=bk, splits=splits, tau=tau, seed=seed),
          flush=True)
    q, k, v, _ = workloads.uniform(device="cuda", seed=seed, batch=2, heads_q=hkv * group, heads_kv=hkv, nq=nq,
                                   nk=nk, d=128, scale=4.0, dtype=torch.bfloat16)
    mask = torch.full((2, hkv * group, T), 255, dtype=torch.uint8, device="cuda")
    o, z = mala.mala_decode(q, k, v, tau, bk, num_splits=splits, tile_mask=mask)
    torch.cuda.synchronize()
    rep = decode_short_parity(q, k, v, tau, bk, splits, o, z, mask)
    print(rep)
    assert_decode(rep)


@pytest.mark.parametrize("case", range(4))
def test_sweep_packed(mala, case):
    rng = np.random.default_rng(4000 + case)
    nseq = int(rng.integers(1, 6))
    nq_list = [int(rng.integers(1, 300)) for _ in range(nseq)]
    nk_list = [n + int(rng.choice([0, int(rng.integers(0, 400))])) for n in nq_list]
    bq, bk = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    tau = float(rng.choice([0.0, 0.05, 1.0]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 4]))
    print("case", case, dict(nq=nq_list, nk=nk_list, bq=bq, bk=bk, tau=tau, hq=hq, hkv=hkv), flush=True)
    g = torch.Generator(device="cuda").manual_seed(case)
    tq, tk = sum(nq_list), sum(nk_list)
    q = (4.0 * torch.randn((tq, hq, 128), generator=g, device="cuda") / 128 ** 0.5).bfloat16()
    k = torch.randn((tk, hkv, 128), generator=g, device="cuda").bfloat16()
    v = torch.randn((tk, hkv, 128), generator=g, device="cuda").bfloat16()
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(nq_list)]), dtype=torch.int32, device="cuda")
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(nk_list)]), dtype=torch.int32, device="cuda")
    mq, mk = max(nq_list), max(nk_list)
    mask = torch.full((nseq, hq, -(-mq // bq), -(-mk // bk)), 255, dtype=torch.uint8, device="cuda")
    o, z = mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, mq, mk, tau, bq, bk, tile_mask=mask)
    torch.cuda.synchronize()
    for b, (nq, nk) in enumerate(zip(nq_list, nk_list)):
        qs, ks = int(cu_q[b]), int(cu_k[b])
        m_b = mask[b:b + 1, :, :-(-nq // bq), :-(-nk // bk)].contiguous()
        rep = forward_parity(q[None, qs:qs + nq], k[None, ks:ks + nk], v[None, ks:ks + nk], tau, bq, bk,
                             nk - nq, o[None, qs:qs + nq].contiguous(), z[None, :, qs:qs + nq].contiguous(), m_b)
        assert_forward(rep, fp32=False)


@pytest.mark.parametrize("case", range(6))
def test_sweep_latent(mala, case):
    """Latent (MLA-shaped) forward: drawn batch, heads, lengths, offset, tau
    and band strength; every query block against the oracle."""
    rng = np.random.default_rng(5000 + case)
    nq = int(rng.integers(1, 260))
    nk = nq + int(rng.choice([0, int(rng.integers(1, 200))]))
    off = nk - nq - (int(rng.integers(0, nk - nq + 1)) if nk > nq and rng.random() < 0.3 else 0)
    c = dict(batch=int(rng.integers(1, 3)), hq=int(rng.choice([1, 3, 8])), nq=nq, nk=nk, off=off,
             tau=float(rng.choice([0.0, 0.05, 0.3, 1.0])), amplitude=float(rng.choice([0.0, 24.0, 40.0])),
             seed=int(rng.integers(1 << 30)))
    print("case", case, c, flush=True)
    wl = workloads.latent_mqa(device="cuda", seed=c["seed"], batch=c["batch"], heads=c["hq"], n=nk,
                              amplitude=c["amplitude"])
    q = wl.q[:, nk - nq:].contiguous()
    mask = fresh_mask(c["batch"], c["hq"], nq, nk, 64, 64)
    o, z = mala.mala_fwd_latent(q, wl.k, 512, c["tau"], 64, 64, causal_offset=off, tile_mask=mask)
    torch.cuda.synchronize()
    rep = forward_parity(q, wl.k, wl.v, c["tau"], 64, 64, off, o, z, mask)
    print(rep)
    assert_forward(rep, fp32=False)


@pytest.mark.parametrize("case", range(6))
def test_sweep_latent_backward(mala, case):
    """Latent (MLA-shaped) backward: drawn batch, heads, lengths, offset, tau
    and band strength; every dQ row and every row gradient dK + [dV, 0]
    against the oracle."""
    from parity import check_latent_backward, run_latent_pass
    rng = np.random.default_rng(6000 + case)
    nq = int(rng.integers(1, 200))
    nk = nq + int(rng.choice([0, int(rng.integers(1, 150))]))
    off = nk - nq - (int(rng.integers(0, nk - nq + 1)) if nk > nq and rng.random() < 0.3 else 0)
    c = dict(batch=int(rng.integers(1, 3)), hq=int(rng.choice([1, 3, 8])), nq=nq, nk=nk, off=off,
             tau=float(rng.choice([0.0, 0.05, 0.3, 1.0])), amplitude=float(rng.choice([0.0, 24.0, 40.0])),
             seed=int(rng.integers(1 << 30)))
    print("case", case, c, flush=True)
    wl = workloads.latent_mqa(device="cuda", seed=c["seed"], batch=c["batch"], heads=c["hq"], n=nk,
                              amplitude=c["amplitude"])
    q = wl.q[:, nk - nq:].contiguous()
    g = torch.Generator(device="cuda").manual_seed(c["seed"] % 1000)
    do = torch.randn((c["batch"], nq, c["hq"], 512), generator=g, device="cuda").to(q.dtype)
    r = run_latent_pass(mala, q, wl.k, do, c["tau"], off=off)
    check_latent_backward(mala, q, wl.k, do, c["tau"], r)


@pytest.mark.parametrize("case", range(6))
def test_sweep_latent_decode(mala, case):
    """Latent (MLA-shaped) decode: drawn batch, head count (16 to 128, so both
    the 16-head and the 64-head workgroup layouts run), cache length, split
    count, tau and band strength; sampled (batch, head) rows against the
    oracle with the same split count."""
    from parity import assert_decode, decode_parity
    rng = np.random.default_rng(7000 + case)
    hq = int(rng.choice([16, 32, 64, 128]))
    nk = int(rng.integers(1, 3000))
    T = (nk + 63) // 64
    c = dict(batch=int(rng.integers(1, 4)), hq=hq, nk=nk, splits=int(rng.integers(1, T + 1)),
             tau=float(rng.choice([0.0, 0.05, 0.3, 1.0])), amplitude=float(rng.choice([0.0, 12.0, 30.0])),
             seed=int(rng.integers(1 << 30)))
    print("case", case, c, flush=True)
    wl = workloads.latent_decode(device="cuda", seed=c["seed"], batch=c["batch"], heads=hq, nk=nk,
                                 amplitude=c["amplitude"])
    mask = torch.full((c["batch"], hq, T), 255, dtype=torch.uint8, device="cuda")
    o, z = mala.mala_decode_latent(wl.q, wl.k, 512, c["tau"], 64, c["splits"], tile_mask=mask)
    torch.cuda.synchronize()
    rows = sorted({(int(rng.integers(c["batch"])), int(rng.integers(hq))) for _ in range(6)})
    rep = decode_parity(wl.q, wl.k, wl.v, c["tau"], 64, c["splits"], o, z, mask, rows=rows)
    print(rep)
    assert_decode(rep)
