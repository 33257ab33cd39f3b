"""Pins of the oracle's short-query decode (``mala_decode_short``).

MALA page, "Fused decoding execution": decoding applies the forward rule with
a short query against a longer KV sequence, and under split-KV each split
keeps its own running state and tests against its partial normalizer; the
partial outputs are merged by the normalizer-aware reduction. The pins tie
the function to things fixed independently of it:

* one query token is the single-token decode (``mala_decode``);
* tau = 0 retains every tile, so any split count gives dense causal softmax
  attention with the query at the end of the cache (brute force);
* one split is the prefill forward rule on one query block of the Nq rows
  with causal offset N_k - Nq (``mala_forward``: its own row positions, L_q
  and diagonal-first tile order);
* a sequence of N_k(b) keys is the same call on the cache cut to N_k(b);
* rows at a negative position have no keys (o = 0, z = -inf).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _inputs(seed, B=2, hq=4, hkv=2, nq=4, nk=300, d=64, scale=3.0):
    q, k, v, _ = workloads.uniform(device="cpu", seed=seed, batch=B, heads_q=hq, heads_kv=hkv, nq=nq, nk=nk, d=d,
                                   scale=scale, dtype=torch.float32)
    return q.double().numpy(), k.double().numpy(), v.double().numpy()


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_one_token_is_single_token_decode(splits):
    q, k, v = _inputs(11, nq=1, nk=333)
    a = oracle.mala_decode_short(q, k, v, 0.05, 64, splits)
    b = oracle.mala_decode(q, k, v, 0.05, 64, splits)
    np.testing.assert_allclose(a["o"][:, 0], b["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a["z"][:, :, 0], b["z"], rtol=0, atol=1e-13)
    assert np.array_equal(a["mask"], b["mask"])


@pytest.mark.parametrize("nq,splits", [(1, 1), (3, 1), (4, 3), (7, 4)])
def test_tau_zero_is_dense_causal_attention(nq, splits):
    q, k, v = _inputs(12, nq=nq, nk=290)
    r = oracle.mala_decode_short(q, k, v, 0.0, 64, splits)
    o, z = oracle.dense_attention(q, k, v, causal_offset=k.shape[1] - nq)
    np.testing.assert_allclose(r["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["z"], z, rtol=0, atol=1e-12)
    T = oracle.num_blocks(k.shape[1], 64)
    assert (r["mask"][:, :, :T] == 1).all()


@pytest.mark.parametrize("nq,G,block_k,tau", [(2, 4, 64, 0.05), (4, 2, 64, 0.3), (4, 2, 32, 0.05), (3, 2, 64, 1.0)])
def test_one_split_is_the_prefill_rule_on_one_block(nq, G, block_k, tau):
    w = workloads.decode_cache(device="cpu", seed=17, batch=2, heads_q=2 * G, heads_kv=2, nk=1000, n_heavy=8, nq=nq)
    q, k, v = (t.double().numpy() for t in (w.q, w.k, w.v))
    nk = k.shape[1]
    r = oracle.mala_decode_short(q, k, v, tau, block_k, 1)
    f = oracle.mala_forward(q, k, v, tau, 64, block_k, causal_offset=nk - nq)
    np.testing.assert_allclose(r["o"], f["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["z"], f["z"], rtol=0, atol=1e-13)
    assert np.array_equal(r["mask"], f["mask"][:, :, 0, :])
    # the pin means something only if the rule skipped work here
    assert (r["mask"] == 0).any() and (r["mask"] == 1).any()


def test_shorter_sequences_are_cut_caches():
    q, k, v = _inputs(14, B=3, nq=4, nk=400, scale=5.0)
    lens = np.array([400, 257, 130])
    r = oracle.mala_decode_short(q, k, v, 0.05, 64, 3, seq_lens=lens)
    for b, n in enumerate(lens):
        c = oracle.mala_decode_short(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], 0.05, 64, 3)
        np.testing.assert_array_equal(r["o"][b], c["o"][0])
        np.testing.assert_array_equal(r["z"][b], c["z"][0])
        T = oracle.num_blocks(n, 64)
        assert np.array_equal(r["mask"][b, :, :T], c["mask"][0])
        assert (r["mask"][b, :, T:] == 255).all()


def test_rows_before_the_first_key_have_no_keys():
    q, k, v = _inputs(15, B=2, nq=4, nk=200)
    lens = np.array([2, 0])
    r = oracle.mala_decode_short(q, k, v, 0.05, 64, 1, seq_lens=lens)
    # sequence 0: tokens 0, 1 sit at positions -2, -1; tokens 2, 3 see keys 0 and 0..1
    assert (r["o"][0, :2] == 0).all() and np.isneginf(r["z"][0, :, :2]).all()
    o, z = oracle.dense_attention(q[:1, 2:], k[:1, :2], v[:1, :2], causal_offset=0)
    np.testing.assert_allclose(r["o"][0, 2:], o[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["z"][0, :, 2:], z[0], rtol=0, atol=1e-13)
    assert (r["o"][1] == 0).all() and np.isneginf(r["z"][1]).all()
    assert (r["mask"][1] == 255).all()


def test_split_rows_without_keys_leave_the_combine():
    # nk = 257, B_k = 64, 5 tiles, 5 splits: the last split holds key 256
    # only, which tokens 0..2 of 4 cannot see; their rows must still equal
    # the dense result at tau = 0
    q, k, v = _inputs(16, nq=4, nk=257)
    r = oracle.mala_decode_short(q, k, v, 0.0, 64, 5)
    o, z = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(r["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["z"], z, rtol=0, atol=1e-12)


def test_tile_margin_uses_each_rows_own_context():
    # two tiles: the most recent one is visited first from an empty state
    # and retained; the margin of the older tile is then, in closed form,
    # max over rows r of  max_k s_rk - log sum_{legal k in tile 1} e^{s_rk}
    #                      - (log tau - log L_r),  L_r = N_k - Nq + r + 1.
    # Token 0's query is made the sharpest, so the maximum is taken on a row
    # whose L_r differs from N_k (a rule using N_k for every row fails here).
    bk, nq, tau = 8, 6, 0.05
    q, k, v = _inputs(21, B=1, hq=2, hkv=1, nq=nq, nk=2 * bk, d=16, scale=2.0)
    q[:, 0] *= 4.0
    nk = 2 * bk
    r = oracle.decode_block_branches(q[0, :, 0], k[0, :, 0], v[0, :, 0], nk - nq + np.arange(nq), tau, bk, 1)
    (res,) = r[0]
    s = q[0, :, 0] @ k[0, :, 0].T
    pos = nk - nq + np.arange(nq)
    legal = np.arange(nk)[None, :] <= pos[:, None]
    t1 = np.where(legal[:, bk:], s[:, bk:], -np.inf)
    lse1 = np.log(np.exp(t1).sum(axis=1))
    rows1 = legal[:, bk:].any(axis=1)
    m0 = s[:, :bk].max(axis=1) - lse1 - (np.log(tau) - np.log(pos + 1))
    expect = m0[rows1].max()
    assert res.margin[1] == np.inf
    assert abs(res.margin[0] - expect) < 1e-12
    assert int(np.argmax(np.where(rows1, m0, -np.inf))) != nq - 1
