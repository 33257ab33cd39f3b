"""Pins of the oracle's paged decode: it must equal the contiguous decode of
the same keys (the page table only relocates rows), per sequence length."""

import numpy as np
import pytest
import torch

import oracle


def make_paged(rng, B, hq, hkv, d, lens, page_size, max_pages):
    n_pages = B * max_pages + 3
    kp = rng.standard_normal((n_pages, page_size, hkv, d))
    vp = rng.standard_normal((n_pages, page_size, hkv, d))
    perm = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages)  # scattered pages
    q = rng.standard_normal((B, 1, hq, d)) * 2.0 / np.sqrt(d)
    return q, kp, vp, perm.astype(np.int32), np.asarray(lens, np.int32)


@pytest.mark.parametrize("page_size,block_k,splits", [(16, 64, 1), (16, 64, 3), (32, 64, 2), (64, 128, 4)])
def test_paged_equals_contiguous(page_size, block_k, splits):
    rng = np.random.default_rng(page_size + splits)
    B, hq, hkv, d, max_pages = 3, 4, 2, 16, 12
    lens = [max_pages * page_size, 5 * page_size + 7, 130]
    q, kp, vp, table, seq = make_paged(rng, B, hq, hkv, d, lens, page_size, max_pages)
    r = oracle.mala_decode_paged(q, kp, vp, table, seq, page_size, 0.05, block_k, splits)
    for b in range(B):
        nk = lens[b]
        keys = np.arange(nk)
        kc = kp[table[b, keys // page_size], keys % page_size][None]
        vc = vp[table[b, keys // page_size], keys % page_size][None]
        T = -(-nk // block_k)
        s = min(splits, T)
        if s < splits:
            # fewer tiles than splits: the empty splits hold no keys, so the
            # result equals the decode with one split per tile
            s = T
        ref = oracle.mala_decode(q[b:b + 1], kc, vc, 0.05, block_k, s)
        assert np.allclose(r["o"][b], ref["o"][0], atol=1e-12, rtol=0)
        assert np.allclose(r["z"][b], ref["z"][0], atol=1e-12, rtol=0)
        if s == splits:
            assert np.array_equal(r["mask"][b, :, :T], ref["mask"][0])
        assert (r["mask"][b, :, T:] == 255).all()


def test_paged_tau_zero_is_dense_and_empty_sequence():
    rng = np.random.default_rng(1)
    B, hq, hkv, d, P, maxp = 2, 2, 1, 8, 16, 6
    q, kp, vp, table, seq = make_paged(rng, B, hq, hkv, d, [70, 0], P, maxp)
    r = oracle.mala_decode_paged(q, kp, vp, table, seq, P, 0.0, 64, 2)
    keys = np.arange(70)
    kc = kp[table[0, keys // P], keys % P][None]
    vc = vp[table[0, keys // P], keys % P][None]
    o, _ = oracle.dense_attention(torch.from_numpy(q[:1]), torch.from_numpy(kc), torch.from_numpy(vc),
                                  causal_offset=69)
    assert np.allclose(r["o"][0], np.asarray(o)[0, 0], atol=1e-12)
    assert (r["o"][1] == 0).all() and np.isneginf(r["z"][1]).all()
