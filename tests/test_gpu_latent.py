"""GPU parity of the latent (MLA-shaped) forward and decode against the CPU oracle:
q [B, Nq, Hq, 576], one cached row per position kv [B, Nk, 1, 576], and the
value is the latent kv[..., :512] (mala_fwd_latent / mala_forward_latent and
mala_decode_latent / mala_decode_latent)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_forward, bf16_close, forward_parity, fresh_mask, legal_tile_count, sample_blocks

pytestmark = pytest.mark.gpu

DV = 512


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def run_latent(mala, q, kv, tau, off=None):
    B, nq, hq, _ = q.shape
    nk = kv.shape[1]
    off = nk - nq if off is None else off
    mask = fresh_mask(B, hq, nq, nk, 64, 64)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_fwd_latent B={B} nq={nq} nk={nk} hq={hq} tau={tau} off={off}", flush=True)
    o, z = mala.mala_fwd_latent(q, kv, DV, tau, 64, 64, causal_offset=off, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    return o, z, mask, stats, off


def check_stats(stats, mask, B, hq, nq, nk, off):
    s = stats.cpu().numpy()
    m = mask.cpu().numpy()
    assert s[0] == legal_tile_count(B, hq, nq, nk, 64, 64, off) == int((m != 255).sum())
    assert s[1] == int((m == 1).sum()) == s[3]
    assert s[2] == oracle.post_score_slots(m, 64, 64, nq)


@pytest.mark.parametrize("amplitude", [0.0, 24.0])
@pytest.mark.parametrize("tau", [0.05, 0.3])
def test_latent_all_blocks(mala, amplitude, tau):
    """Batch 2, 3 heads, N = 300 (a ragged last block), plain Gaussian scores
    and a strong diagonal band (tiles skipped): every query block."""
    wl = workloads.latent_mqa(device="cuda", seed=11, batch=2, heads=3, n=300, amplitude=amplitude)
    o, z, mask, stats, off = run_latent(mala, wl.q, wl.k, tau)
    assert o.shape == (2, 300, 3, DV)
    rep = forward_parity(wl.q, wl.k, wl.v, tau, 64, 64, off, o, z, mask)
    print(rep, "skipped", int((mask == 0).sum()))
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 2, 3, 300, 300, off)
    if amplitude > 0:
        assert int((mask == 0).sum()) > 0


def test_latent_tau_zero_is_dense(mala):
    wl = workloads.latent_mqa(device="cuda", seed=5, batch=1, heads=2, n=200)
    o, z, mask, _, _ = run_latent(mala, wl.q, wl.k, 0.0)
    m = mask.cpu().numpy()
    assert ((m == 1) | (m == 255)).all()
    od, zd = oracle.dense_attention(wl.q, wl.k, wl.v)
    ok, err = bf16_close(o.double().cpu().numpy(), od)
    assert ok, err
    assert np.abs(z.double().cpu().numpy() - zd).max() < 1e-4


def test_latent_offset_short_query(mala):
    """N_q = 100 new rows after 257 cached positions (offset 257)."""
    full = workloads.latent_mqa(device="cuda", seed=9, batch=1, heads=4, n=357, amplitude=12.0)
    q = full.q[:, 257:].contiguous()
    for tau in (0.05, 1.0):
        o, z, mask, stats, off = run_latent(mala, q, full.k, tau)
        assert off == 257
        rep = forward_parity(q, full.k, full.v, tau, 64, 64, off, o, z, mask)
        print(tau, rep)
        assert_forward(rep, fp32=False)
        check_stats(stats, mask, 1, 4, 100, 357, off)


def test_latent_deterministic(mala):
    wl = workloads.latent_mqa(device="cuda", seed=2, batch=1, heads=4, n=512, amplitude=12.0)
    o1, z1, m1, _, _ = run_latent(mala, wl.q, wl.k, 0.05)
    o2, z2, m2, _, _ = run_latent(mala, wl.q, wl.k, 0.05)
    assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(m1, m2)


def test_latent_full_size_sampled(mala):
    """The launch the bench times: batch 1, 16 heads, N = 4096, d_qk 576,
    d_v 512, tau 0.05, banded latent scores; sampled query blocks."""
    wl = workloads.latent_mqa(device="cuda")
    o, z, mask, stats, off = run_latent(mala, wl.q, wl.k, wl.tau)
    blocks = sample_blocks(1, 16, 64, 6, seed=5)
    rep = forward_parity(wl.q, wl.k, wl.v, wl.tau, 64, 64, off, o, z, mask, blocks=blocks)
    print(rep, "skip rate", float((mask == 0).sum()) / float((mask != 255).sum()))
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 1, 16, 4096, 4096, off)
    assert torch.isfinite(o.float()).all() and torch.isfinite(z).all()


# ---------------------------------------------------------------------------
# decode on the latent cache (mala_decode_latent / mala_decode_latent oracle)
# ---------------------------------------------------------------------------
from parity import assert_decode, decode_parity  # noqa: E402


def run_latent_decode(mala, q, kv, tau, splits):
    B, _, hq, _ = q.shape
    T = oracle.num_blocks(kv.shape[1], 64)
    mask = torch.full((B, hq, T), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_decode_latent B={B} hq={hq} nk={kv.shape[1]} tau={tau} splits={splits}", flush=True)
    o, z = mala.mala_decode_latent(q, kv, DV, tau, 64, num_splits=splits, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    return o, z, mask, stats


def check_decode_stats(stats, mask, B, hq):
    s = stats.cpu().numpy()
    m = mask.cpu().numpy()
    T = m.shape[2]
    assert s[0] == m.size and s[1] == int((m == 1).sum()) and s[2] == s[1] * 64
    # a tile's P V runs once per group of 16 heads in which some head retains it
    assert s[3] == int((m.reshape(B, hq // 16, 16, T) == 1).any(axis=2).sum())


@pytest.mark.parametrize("amplitude", [0.0, 30.0])
@pytest.mark.parametrize("tau", [0.05, 1.0])
def test_latent_decode_splits(mala, amplitude, tau):
    """Batch 2, 32 heads (two head groups), N_k = 1000 (a ragged last tile),
    with and without the positional band; 1, 3 and T splits."""
    wl = workloads.latent_decode(device="cuda", seed=21, batch=2, heads=32, nk=1000,
                                 amplitude=amplitude)
    T = oracle.num_blocks(1000, 64)
    skipped = 0
    for splits in (1, 3, T):
        o, z, mask, stats = run_latent_decode(mala, wl.q, wl.k, tau, splits)
        assert o.shape == (2, 1, 32, DV) and z.shape == (2, 32)
        rep = decode_parity(wl.q, wl.k, wl.v, tau, 64, splits, o, z, mask)
        print(splits, rep)
        assert_decode(rep)
        check_decode_stats(stats, mask, 2, 32)
        skipped += int((mask == 0).sum())
    if amplitude > 0:
        assert skipped > 0


def test_latent_decode_tau_zero_is_dense(mala):
    wl = workloads.latent_decode(device="cuda", seed=3, batch=2, heads=16, nk=777)
    od, zd = oracle.dense_attention(wl.q, wl.k, wl.v)
    for splits in (1, 4):
        o, z, mask, _ = run_latent_decode(mala, wl.q, wl.k, 0.0, splits)
        assert (mask.cpu().numpy() == 1).all()
        ok, err = bf16_close(o.double().cpu().numpy()[:, 0], od[:, 0])
        assert ok, err
        assert np.abs(z.double().cpu().numpy() - zd[:, :, 0]).max() < 1e-4


@pytest.mark.parametrize("nk", [1, 63, 64, 65, 130])
def test_latent_decode_short_caches(mala, nk):
    """One key, a partial single tile, exactly one tile, one key past it."""
    wl = workloads.latent_decode(device="cuda", seed=nk, batch=3, heads=16, nk=nk, amplitude=12.0)
    T = oracle.num_blocks(nk, 64)
    for splits in sorted({1, T}):
        o, z, mask, stats = run_latent_decode(mala, wl.q, wl.k, 0.05, splits)
        rep = decode_parity(wl.q, wl.k, wl.v, 0.05, 64, splits, o, z, mask)
        assert_decode(rep)
        check_decode_stats(stats, mask, 3, 16)


@pytest.mark.parametrize("amplitude,tau", [(0.0, 0.05), (30.0, 0.05), (30.0, 1.0)])
def test_latent_decode_64_heads(mala, amplitude, tau):
    """64 query heads: one workgroup per 64 heads, each wave owning 16 heads
    over whole tiles; batch 2, N_k = 1000 (a ragged last tile), 1, 3 and T
    splits."""
    wl = workloads.latent_decode(device="cuda", seed=64, batch=2, heads=64, nk=1000, amplitude=amplitude)
    T = oracle.num_blocks(1000, 64)
    for splits in (1, 3, T):
        o, z, mask, stats = run_latent_decode(mala, wl.q, wl.k, tau, splits)
        rows = [(b, h) for b in range(2) for h in (0, 5, 15, 16, 31, 32, 47, 48, 63)]
        rep = decode_parity(wl.q, wl.k, wl.v, tau, 64, splits, o, z, mask, rows=rows)
        print(splits, rep)
        assert_decode(rep)
        check_decode_stats(stats, mask, 2, 64)


def test_latent_decode_128_heads(mala):
    """128 query heads (eight head groups reading the same cache rows)."""
    wl = workloads.latent_decode(device="cuda", seed=8, batch=1, heads=128, nk=2000, amplitude=24.0)
    o, z, mask, stats = run_latent_decode(mala, wl.q, wl.k, 0.05, 5)
    rows = [(0, h) for h in (0, 1, 15, 16, 63, 64, 100, 127)]
    rep = decode_parity(wl.q, wl.k, wl.v, 0.05, 64, 5, o, z, mask, rows=rows)
    print(rep)
    assert_decode(rep)
    check_decode_stats(stats, mask, 1, 128)


def test_latent_decode_deterministic(mala):
    wl = workloads.latent_decode(device="cuda", seed=4, batch=2, heads=16, nk=3000)
    a = run_latent_decode(mala, wl.q, wl.k, 0.05, 7)
    b = run_latent_decode(mala, wl.q, wl.k, 0.05, 7)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("splits", [1, 8])
def test_latent_decode_full_size_sampled(mala, splits):
    """The launch the bench times: batch 64, 16 heads, N_k = 32768, d_qk 576,
    d_v 512, B_k 64, tau 0.05; sampled (batch, head) rows."""
    wl = workloads.latent_decode(device="cuda")
    o, z, mask, stats = run_latent_decode(mala, wl.q, wl.k, wl.tau, splits)
    rows = [(0, 0), (0, 15), (63, 7), (17, 12), (40, 3)]
    rep = decode_parity(wl.q, wl.k, wl.v, wl.tau, 64, splits, o, z, mask, rows=rows)
    print(rep)
    assert_decode(rep)
    check_decode_stats(stats, mask, 64, 16)
    assert torch.isfinite(o.float()).all() and torch.isfinite(z).all()


# ---------------------------------------------------------------------------
# backward on the latent cache (mala_bwd_latent / mala_backward_latent)
# ---------------------------------------------------------------------------
from parity import check_latent_backward, host64, rel_l2_only, run_latent_pass  # noqa: E402


def check_backward_stats(r, B, hq, nq, nk):
    sb, mb = r["sb"].cpu().numpy(), r["mb"].cpu().numpy()
    assert sb[0] == legal_tile_count(B, hq, nq, nk, 64, 64, r["off"]) == int((mb != 255).sum())
    assert sb[1] == int((mb == 1).sum()) == sb[3]
    assert sb[2] == oracle.post_score_slots(mb, 64, 64, nq)


def latent_do(seed, q):
    g = torch.Generator(device="cuda").manual_seed(seed)
    B, nq, hq, _ = q.shape
    return torch.randn((B, nq, hq, DV), generator=g, device="cuda").to(q.dtype)


@pytest.mark.parametrize("amplitude", [0.0, 24.0])
@pytest.mark.parametrize("tau", [0.05, 0.3])
def test_latent_backward_all_blocks(mala, amplitude, tau):
    """Batch 2, 3 heads, N = 300 (ragged last blocks), with and without the
    positional band (tiles skipped): every dQ row and every dKV row."""
    wl = workloads.latent_mqa(device="cuda", seed=31, batch=2, heads=3, n=300, amplitude=amplitude)
    do = latent_do(1, wl.q)
    r = run_latent_pass(mala, wl.q, wl.k, do, tau)
    assert r["dq"].shape == wl.q.shape and r["dkv"].shape == wl.k.shape
    check_latent_backward(mala, wl.q, wl.k, do, tau, r)
    check_backward_stats(r, 2, 3, 300, 300)
    if amplitude > 0:
        assert int((r["mb"] == 0).sum()) > 0


def test_latent_backward_offset_short_query(mala):
    """N_q = 100 new rows after 257 cached positions (offset 257): dKV of the
    cached rows gets only the new rows' gradients."""
    full = workloads.latent_mqa(device="cuda", seed=19, batch=1, heads=4, n=357, amplitude=12.0)
    q = full.q[:, 257:].contiguous()
    do = latent_do(2, q)
    r = run_latent_pass(mala, q, full.k, do, 0.05)
    assert r["off"] == 257
    check_latent_backward(mala, q, full.k, do, 0.05, r)
    check_backward_stats(r, 1, 4, 100, 357)


def test_latent_backward_tau_zero_is_dense(mala):
    """tau = 0 retains every tile: strict kernel parity on the oracle
    forward, and the end-to-end gradients against dense attention over the
    latent value by torch autograd in float64 on the host (relative L2: the
    bf16 rounding of the forward's O moves D = rowsum(dO O) and with it every
    gradient element, which the strict part isolates)."""
    wl = workloads.latent_mqa(device="cuda", seed=6, batch=1, heads=2, n=200, amplitude=0.0)
    do = latent_do(3, wl.q)
    r = run_latent_pass(mala, wl.q, wl.k, do, 0.0)
    check_latent_backward(mala, wl.q, wl.k, do, 0.0, r)
    qt = torch.tensor(host64(wl.q), requires_grad=True)
    kvt = torch.tensor(host64(wl.k), requires_grad=True)
    s = torch.einsum("bqhd,bkd->bhqk", qt, kvt[:, :, 0])
    legal = torch.arange(200)[None, :] <= torch.arange(200)[:, None]
    p = torch.softmax(s.masked_fill(~legal, float("-inf")), dim=-1)
    o = torch.einsum("bhqk,bkd->bqhd", p, kvt[:, :, 0, :DV])
    o.backward(torch.tensor(host64(do)))
    rep = type("R", (), {"err": {}})()
    assert rel_l2_only(host64(r["dq"]), qt.grad.numpy(), "dq", rep), rep.err
    assert rel_l2_only(host64(r["dkv"]), kvt.grad.numpy(), "dkv", rep), rep.err
    print(rep.err)
    assert (r["mb"].cpu().numpy() != 0).all()


def test_latent_backward_head_groups(mala):
    """Batch 4, 16 heads, N = 1024: enough key blocks that the key-major pass
    splits the heads into groups (fp32 partials summed in a fixed order);
    sampled key blocks and query blocks."""
    wl = workloads.latent_mqa(device="cuda", seed=13, batch=4, heads=16, n=1024, amplitude=24.0)
    do = latent_do(4, wl.q)
    r = run_latent_pass(mala, wl.q, wl.k, do, 0.05)
    prob = mala.make_problem(wl.q, wl.k, 0.05, 64, 64)
    assert mala.mala_bwd_latent_workspace_size(prob) > 4 * 16 * 1024 * 4 + 4 * 1024 * 576 * 4  # > 1 group
    kb = [(0, 0, 15), (3, 0, 14), (1, 0, 0)]
    qb = [0, 15]
    fwd = sorted({(b, h, i) for b in range(4) for h in range(16) for i in (0, 14, 15)})
    check_latent_backward(mala, wl.q, wl.k, do, 0.05, r, key_blocks=kb[:2], query_blocks=qb, fwd_blocks=fwd)
    assert torch.isfinite(r["dkv"].float()).all() and torch.isfinite(r["dq"].float()).all()


def test_latent_backward_deterministic(mala):
    wl = workloads.latent_mqa(device="cuda", seed=8, batch=1, heads=8, n=640, amplitude=12.0)
    do = latent_do(5, wl.q)
    r1 = run_latent_pass(mala, wl.q, wl.k, do, 0.05)
    r2 = run_latent_pass(mala, wl.q, wl.k, do, 0.05)
    assert torch.equal(r1["dq"], r2["dq"]) and torch.equal(r1["dkv"], r2["dkv"])
    assert torch.equal(r1["mb"], r2["mb"])


def test_latent_backward_full_size_sampled(mala):
    """The launch the bench times: batch 1, 16 heads, N = 4096, d_qk 576,
    d_v 512, tau 0.05; sampled key blocks (the last two) and query blocks."""
    wl = workloads.latent_mqa(device="cuda")
    do = latent_do(6, wl.q)
    r = run_latent_pass(mala, wl.q, wl.k, do, wl.tau)
    fwd = sorted({(0, h, i) for h in range(16) for i in (0, 62, 63)})
    check_latent_backward(mala, wl.q, wl.k, do, wl.tau, r, key_blocks=[(0, 0, 63), (0, 0, 62)], query_blocks=[0, 63],
                          fwd_blocks=fwd)
    check_backward_stats(r, 1, 16, 4096, 4096)
    assert torch.isfinite(r["dkv"].float()).all() and torch.isfinite(r["dq"].float()).all()
