"""GPU parity of the operator-fidelity instrumentation (MALA page,
experiments: omitted mass, per-head relative L2, post-score slots per query,
Rademacher probe) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seed", [0, 1234567, (1 << 64) - 1])
def test_rademacher_bit_exact(mala, dtype, seed):
    n = (1 << 20) + 37  # several blocks and a ragged tail
    r = mala.mala_rademacher((n,), seed, dtype=dtype)
    torch.cuda.synchronize()
    assert np.array_equal(r.double().cpu().numpy(), oracle.rademacher(n, seed))


def test_omitted_mass_and_slot_histogram(mala):
    """Screened (tau 0.05) and screening-disabled (tau 0) forwards of the
    same inputs; omitted mass from the two z on the GPU vs the oracle's
    formula on the same z, and the GPU slot histogram of the screened mask vs
    the oracle's, bit for bit."""
    wl = workloads.local_band(device="cuda", seed=21, batch=2, heads=4, n=700, width=48.0,
                              amplitude=24.0)
    q, k, v = wl.q, wl.k, wl.v
    B, nq, hq, _ = q.shape
    bq = bk = 64
    mask = mala.new_tile_mask(B, hq, nq, nq, bq, bk, "cuda")
    stats = mala.new_stats("cuda")
    _, zs = mala.mala_fwd(q, k, v, 0.05, bq, bk, stats=stats, tile_mask=mask)
    _, zr = mala.mala_fwd(q, k, v, 0.0, bq, bk)
    om = mala.mala_omitted_mass(zs, zr)
    hist = mala.mala_slot_histogram(mask, nq, nq, bq, bk)
    torch.cuda.synchronize()
    ref = oracle.omitted_mass(host64(zs), host64(zr))
    got = host64(om)
    assert np.abs(got - ref).max() <= 1e-6 + 1e-5 * np.abs(ref).max()
    assert (ref > -1e-6).all()
    skipped = int(stats[0].item() - stats[1].item())
    print("tiles skipped", skipped, "of", int(stats[0].item()), "max omitted mass", ref.max())
    assert skipped > 0 and ref.max() > 0
    m = mask.cpu().numpy()
    h = hist.cpu().numpy()
    assert np.array_equal(h, oracle.slot_histogram(m, bq, nq))
    assert sum(c * bk * n for c, n in enumerate(h.tolist())) == int(stats[2].item())
    assert h.sum() == B * hq * nq


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_sq_err_heads(mala, dtype):
    g = torch.Generator(device="cuda").manual_seed(4)
    ref = torch.randn((2, 1000, 3, 128), generator=g, device="cuda").to(dtype)
    x = (ref.float() + 0.01 * torch.randn(ref.shape, generator=g, device="cuda")).to(dtype)
    sd, sr = mala.mala_sq_err_heads(x, ref)
    torch.cuda.synchronize()
    esd, esr = oracle.sq_err_heads(host64(x), host64(ref))
    assert np.allclose(sd.cpu().numpy(), esd, rtol=1e-11, atol=0)
    assert np.allclose(sr.cpu().numpy(), esr, rtol=1e-11, atol=0)
    sd2, _ = mala.mala_sq_err_heads(ref, ref)
    assert (sd2 == 0).all()
    # deterministic: a second call gives the same bits
    sd3, sr3 = mala.mala_sq_err_heads(x, ref)
    assert torch.equal(sd, sd3) and torch.equal(sr, sr3)


def test_backward_fidelity_with_rademacher_probe(mala):
    """The page's backward comparison: the same Rademacher dO through the
    screened and the screening-disabled backward; per-head relative L2 of dQ
    from the GPU sums equals the oracle's on the same tensors."""
    wl = workloads.local_band(device="cuda", seed=8, heads=2, n=384, width=48.0, amplitude=24.0)
    q, k, v = wl.q, wl.k, wl.v
    do = mala.mala_rademacher(q.shape, 7)
    o_s, z_s = mala.mala_fwd(q, k, v, 0.05, 64, 64)
    o_r, z_r = mala.mala_fwd(q, k, v, 0.0, 64, 64)
    dq_s, _, _ = mala.mala_bwd(q, k, v, o_s, do, z_s, 0.05, 64, 64)
    dq_r, _, _ = mala.mala_bwd(q, k, v, o_r, do, z_r, 0.0, 64, 64)
    sd, sr = mala.mala_sq_err_heads(dq_s, dq_r)
    torch.cuda.synchronize()
    assert np.array_equal(host64(do).ravel(), oracle.rademacher(do.numel(), 7))
    esd, esr = oracle.sq_err_heads(host64(dq_s), host64(dq_r))
    assert np.allclose(sd.cpu().numpy(), esd, rtol=1e-11)
    assert np.allclose(sr.cpu().numpy(), esr, rtol=1e-11)
    rel = np.sqrt(sd.cpu().numpy() / sr.cpu().numpy())
    print("per-head rel-L2 of dQ, tau 0.05 vs 0:", rel)
    assert (rel > 0).all() and (rel < 0.5).all()
