"""Pins of the oracle's packed-sequence forward."""

import numpy as np

import oracle


def test_equal_lengths_match_the_batched_layout():
    rng = np.random.default_rng(0)
    B, n, hq, hkv, d = 3, 70, 4, 2, 16
    q = rng.standard_normal((B, n, hq, d)) * 3 / np.sqrt(d)
    k = rng.standard_normal((B, n, hkv, d))
    v = rng.standard_normal((B, n, hkv, d))
    ref = oracle.mala_forward(q, k, v, 0.2, 16, 32)
    cu = np.arange(B + 1) * n
    r = oracle.mala_forward_varlen(q.reshape(B * n, hq, d), k.reshape(B * n, hkv, d),
                                   v.reshape(B * n, hkv, d), cu, cu, 0.2, 16, 32)
    assert np.array_equal(r["o"], ref["o"].reshape(B * n, hq, d))
    assert np.array_equal(r["z"], ref["z"].transpose(1, 0, 2).reshape(hq, B * n))
    assert np.array_equal(r["mask"], ref["mask"])


def test_chunked_prefill_and_empty_rows_at_tau_zero_are_dense():
    """tau = 0: each sequence equals dense bottom-right causal attention on
    its own rows; rows before the first key (N_k < N_q) are o = 0, z = -inf."""
    rng = np.random.default_rng(1)
    hq, hkv, d = 2, 1, 8
    nq_list, nk_list = [5, 40, 12, 9], [5, 100, 12, 4]  # plain, chunked prefill, plain, N_k < N_q
    cu_q = np.concatenate([[0], np.cumsum(nq_list)])
    cu_k = np.concatenate([[0], np.cumsum(nk_list)])
    q = rng.standard_normal((cu_q[-1], hq, d))
    k = rng.standard_normal((cu_k[-1], hkv, d))
    v = rng.standard_normal((cu_k[-1], hkv, d))
    r = oracle.mala_forward_varlen(q, k, v, cu_q, cu_k, 0.0, 16, 16)
    for b, (nq, nk) in enumerate(zip(nq_list, nk_list)):
        qs, ks = cu_q[b], cu_k[b]
        off = nk - nq
        for h in range(hq):
            for t in range(nq):
                if t + off < 0:
                    assert (r["o"][qs + t, h] == 0).all() and np.isneginf(r["z"][h, qs + t])
                    continue
                s = k[ks:ks + t + off + 1, 0] @ q[qs + t, h]
                p = np.exp(s - s.max())
                assert np.allclose(r["o"][qs + t, h], (p / p.sum()) @ v[ks:ks + t + off + 1, 0], atol=1e-12)
                assert np.isclose(r["z"][h, qs + t], s.max() + np.log(p.sum()), atol=1e-12)
