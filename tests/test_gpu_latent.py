"""GPU parity of the latent (MLA-shaped) forward against the CPU oracle:
q [B, Nq, Hq, 576], one cached row per position kv [B, Nk, 1, 576], and the
value is the latent kv[..., :512] (mala_fwd_latent / mala_forward_latent)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_forward, forward_parity, fresh_mask, legal_tile_count, sample_blocks

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
    assert np.abs(o.double().cpu().numpy() - od).max() < 2e-2
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
