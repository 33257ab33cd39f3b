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
