"""Pins of the oracle's latent (MLA-shaped) forward, ``mala_forward_latent``.

The value of latent attention is the cached latent itself: the first d_v
columns of each cached row (attention tutorial page, section "MLA: compress
the cached representation"). These tests check that reading against what the
pages and the mathematics fix, independently of the oracle's own code path:
dense brute force at tau = 0, the page's two-row worked example of moving the
value expansion after the weighted sum, and the from-scratch (linear-domain)
formulation of the MALA rule on a banded input that skips tiles.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _small(seed, n=160, heads=3, d_qk=40, d_v=32, amplitude=0.0, width=16.0):
    wl = workloads.latent_mqa(seed=seed, batch=1, heads=heads, n=n, d_qk=d_qk, d_v=d_v,
                              amplitude=amplitude, width=width, dtype=None)
    return wl.q.double().numpy(), wl.k.double().numpy(), d_v


@pytest.mark.parametrize("seed", [0, 233])
def test_tau_zero_is_dense_attention_over_the_latent(seed):
    q, kv, dv = _small(seed)
    res = oracle.mala_forward_latent(q, kv, dv, 0.0, 32, 32)
    o_ref, z_ref = oracle.dense_attention(q, kv, kv[..., :dv])
    assert res["o"].shape == (1, 160, 3, dv)
    np.testing.assert_allclose(res["o"], o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["z"], z_ref, rtol=0, atol=1e-12)
    legal = res["mask"] != 255
    assert (res["mask"][legal] == 1).all()


def test_two_row_absorption_example():
    """The tutorial page's example: one head, two cached rows, attention
    weights 0.25 and 0.75. Averaging the latent rows and then applying the
    value map gives the same vector as mapping each row and then averaging."""
    dv = 4
    c = np.array([[1.0, -2.0, 0.5, 3.0], [2.0, 1.0, -1.0, 0.0]])
    kv = np.zeros((1, 2, 1, dv + 2))
    kv[0, :, 0, :dv] = c
    kv[0, 1, 0, dv] = 1.0                 # positional column: s_1 - s_0 = log 3
    q = np.zeros((1, 2, 1, dv + 2))
    q[0, :, 0, dv] = math.log(3.0)
    w = np.array([[0.5, 1.0, 0.0], [2.0, -1.0, 1.0], [0.0, 0.5, 3.0], [1.0, 1.0, -2.0]])
    lat = oracle.mala_forward_latent(q, kv, dv, 0.05, 2, 2)
    exp = oracle.mala_forward(q, kv, kv[..., :dv] @ w, 0.05, 2, 2)
    avg = 0.25 * c[0] + 0.75 * c[1]
    np.testing.assert_allclose(lat["o"][0, 1, 0], avg, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lat["o"][0, 1, 0] @ w, exp["o"][0, 1, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(avg @ w, 0.25 * c[0] @ w + 0.75 * c[1] @ w, rtol=0, atol=1e-14)
    # row 0 sees only key 0
    np.testing.assert_allclose(lat["o"][0, 0, 0], c[0], rtol=0, atol=1e-15)
    assert lat["z"][0, 0, 1] == pytest.approx(math.log(1.0 + 3.0), abs=1e-14)


@pytest.mark.parametrize("tau", [0.05, 0.3])
def test_banded_latent_matches_the_from_scratch_rule(tau):
    """On a banded input (far tiles carry little mass) the latent forward
    skips tiles; every block's decisions, output and normalizer equal the
    linear-domain formulation that keeps the retained key sets explicitly."""
    q, kv, dv = _small(42, n=192, heads=2, d_qk=24, d_v=16, amplitude=40.0)
    bq = bk = 32
    res = oracle.mala_forward_latent(q, kv, dv, tau, bq, bk)
    skipped = 0
    for h in range(2):
        for i in range(oracle.num_blocks(192, bq)):
            rows, lastv, L, tiles = oracle.prefill_block_args(i, bq, bk, 192, 192, 0)
            o2, z2, dec2 = oracle.forward_block_from_scratch(q[0, rows, h], kv[0, :, 0],
                                                             kv[0, :, 0, :dv], lastv, L, tiles,
                                                             tau, bk)
            for j, d in dec2.items():
                assert res["mask"][0, h, i, j] == d
                skipped += d == 0
            np.testing.assert_allclose(res["o"][0, rows, h], o2, rtol=0, atol=1e-10)
            np.testing.assert_allclose(res["z"][0, h, rows], z2, rtol=0, atol=1e-10)
    assert skipped > 0


# ---------------------------------------------------------------------------
# decode on the latent cache
# ---------------------------------------------------------------------------

def _small_decode(seed, nk=300, heads=3, d_qk=40, d_v=32, amplitude=0.0):
    wl = workloads.latent_decode(seed=seed, batch=2, heads=heads, nk=nk, d_qk=d_qk, d_v=d_v,
                                 amplitude=amplitude, width=8.0, sink_score=2.0, dtype=None)
    return wl.q.double().numpy(), wl.k.double().numpy(), d_v


@pytest.mark.parametrize("splits", [1, 3])
def test_latent_decode_tau_zero_is_dense_attention(splits):
    q, kv, dv = _small_decode(7)
    res = oracle.mala_decode_latent(q, kv, dv, 0.0, 32, num_splits=splits)
    o_ref, z_ref = oracle.dense_attention(q, kv, kv[..., :dv])   # offset N_k - 1
    np.testing.assert_allclose(res["o"], o_ref[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["z"], z_ref[:, :, 0], rtol=0, atol=1e-12)
    assert (res["mask"] == 1).all()


def test_latent_decode_two_row_absorption_example():
    """The tutorial page's two-row example read by a decode step: the new
    token attends to two cached rows with weights 0.25 and 0.75, and the
    output is the same weighted average of the latents."""
    dv = 4
    c = np.array([[1.0, -2.0, 0.5, 3.0], [2.0, 1.0, -1.0, 0.0]])
    kv = np.zeros((1, 2, 1, dv + 2))
    kv[0, :, 0, :dv] = c
    kv[0, 1, 0, dv] = 1.0
    q = np.zeros((1, 1, 1, dv + 2))
    q[0, 0, 0, dv] = math.log(3.0)
    res = oracle.mala_decode_latent(q, kv, dv, 0.05, 2)
    np.testing.assert_allclose(res["o"][0, 0], 0.25 * c[0] + 0.75 * c[1], rtol=0, atol=1e-14)
    assert res["z"][0, 0] == pytest.approx(math.log(4.0), abs=1e-14)


def _logsumexp_combine(parts):
    zs = np.array([z for _, z in parts])
    z = np.log(np.sum(np.exp(zs)))
    return sum(np.exp(zp - z) * o for o, zp in parts), z


@pytest.mark.parametrize("tau,splits", [(0.05, 1), (0.05, 3), (0.3, 2)])
def test_latent_decode_matches_the_from_scratch_rule(tau, splits):
    """Each split runs the linear-domain formulation of the rule (explicit
    retained key sets, L_0 = N_k) over its own tiles, most recent first,
    from an empty state; the splits are merged by the plain logsumexp
    combination. Decisions, outputs and normalizers agree with the oracle,
    and the input skips tiles."""
    q, kv, dv = _small_decode(42, nk=320, heads=2, d_qk=24, d_v=16, amplitude=30.0)
    bk, nk = 32, 320
    T = nk // bk
    res = oracle.mala_decode_latent(q, kv, dv, tau, bk, num_splits=splits)
    skipped = 0
    for b in range(2):
        for h in range(2):
            parts = []
            for s in range(splits):
                lo, hi = s * T // splits, (s + 1) * T // splits
                o2, z2, dec2 = oracle.forward_block_from_scratch(
                    q[b, 0, h][None], kv[b, :, 0], kv[b, :, 0, :dv], [nk - 1], [nk],
                    list(range(hi - 1, lo - 1, -1)), tau, bk)
                for j, d in dec2.items():
                    assert res["mask"][b, h, j] == d
                    skipped += d == 0
                parts.append((o2[0], z2[0]))
            o_c, z_c = _logsumexp_combine(parts)
            np.testing.assert_allclose(res["o"][b, h], o_c, rtol=0, atol=1e-10)
            assert res["z"][b, h] == pytest.approx(z_c, abs=1e-10)
    assert skipped > 0


# ---------------------------------------------------------------------------
# backward on the latent cache
# ---------------------------------------------------------------------------

def _dense_latent_grads(q, kv, dv, do):
    """Gradients of dense causal attention over the latent value by torch
    autograd in float64: the cached row enters both the scores and (its
    first dv columns) the value, and autograd sums the two paths."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kvt = torch.tensor(kv, dtype=torch.float64, requires_grad=True)
    B, nq, hq, _ = q.shape
    nk = kv.shape[1]
    s = torch.einsum("bqhd,bkd->bhqk", qt, kvt[:, :, 0])
    legal = torch.arange(nk)[None, :] <= (torch.arange(nq) + nk - nq)[:, None]
    s = s.masked_fill(~legal, float("-inf"))
    o = torch.einsum("bhqk,bkd->bqhd", torch.softmax(s, dim=-1), kvt[:, :, 0, :dv])
    o.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kvt.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("seed", [0, 666])
def test_latent_backward_tau_zero_is_the_dense_gradient(seed):
    q, kv, dv = _small(seed, n=96, heads=3)
    do = np.random.default_rng(seed).standard_normal((1, 96, 3, dv))
    fwd = oracle.mala_forward_latent(q, kv, dv, 0.0, 32, 32)
    r = oracle.mala_backward_latent(q, kv, dv, fwd["o"], do, fwd["z"], 0.0, 32, 32)
    gq, gkv, o_ref = _dense_latent_grads(q, kv, dv, do)
    np.testing.assert_allclose(fwd["o"], o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dq"], gq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["dkv"], gkv, rtol=0, atol=1e-11)
    assert r["dkv"].shape == kv.shape


def test_latent_backward_value_path_by_finite_differences():
    """Central differences of <dO, O> in one latent column that is not part
    of the scores' dominant terms: the value path alone is d_v columns wide,
    the positional columns get only the score path."""
    q, kv, dv = _small(3, n=40, heads=2, d_qk=12, d_v=8)
    do = np.random.default_rng(3).standard_normal((1, 40, 2, dv))
    fwd = oracle.mala_forward_latent(q, kv, dv, 0.0, 16, 16)
    r = oracle.mala_backward_latent(q, kv, dv, fwd["o"], do, fwd["z"], 0.0, 16, 16)
    eps = 1e-6
    for (k, c) in [(5, 2), (17, 7), (33, 9), (39, 11)]:   # columns 9 and 11 are positional
        kp, km = kv.copy(), kv.copy()
        kp[0, k, 0, c] += eps
        km[0, k, 0, c] -= eps
        op = oracle.mala_forward_latent(q, kp, dv, 0.0, 16, 16)["o"]
        om = oracle.mala_forward_latent(q, km, dv, 0.0, 16, 16)["o"]
        fd = float(((op - om) * do).sum()) / (2 * eps)
        assert r["dkv"][0, k, 0, c] == pytest.approx(fd, rel=1e-6, abs=1e-8)
