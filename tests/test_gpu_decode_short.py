"""GPU parity of the HIP decode of a short query (N_q > 1 newest tokens, the
rows of a head forming one query block) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_decode, bf16_close, decode_short_parity, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def short_cache(seed, B=2, group=2, hkv=2, nq=4, nk=1000):
    wl = workloads.decode_cache(device="cuda", seed=seed, batch=B, heads_q=group * hkv, heads_kv=hkv, nk=nk,
                                n_heavy=8, nq=nq)
    return wl.q, wl.k, wl.v


def run(mala, q, k, v, tau, bk, splits):
    B, nq, hq, _ = q.shape
    T = oracle.num_blocks(k.shape[1], bk)
    mask = torch.full((B, hq, T), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_decode q {tuple(q.shape)} k {tuple(k.shape)} B_k {bk} splits {splits} tau {tau}", flush=True)
    o, z = mala.mala_decode(q, k, v, tau, bk, num_splits=splits, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    return o, z, mask, stats


def check_stats(stats, mask, B, hkv, group, nq, bk):
    s = stats.cpu().numpy()
    m = mask.cpu().numpy()
    T = m.shape[2]
    assert s[0] == m.size                              # every tile is legal for a head's block
    assert s[1] == int((m == 1).sum())                 # retained (head, tile) decisions
    assert s[2] == s[1] * bk * nq                      # post-score slots: the block's rows
    assert s[3] == (m.reshape(B, hkv, group, T) == 1).any(axis=2).sum()  # V tiles loaded


@pytest.mark.parametrize("group,nq", [(1, 4), (2, 4), (4, 4), (8, 2), (1, 16), (2, 8), (16, 1)])
@pytest.mark.parametrize("bk", [64, 256])
def test_heads_tokens_and_tiles(mala, group, nq, bk):
    hkv = 2
    q, k, v = short_cache(100 * group + nq + bk, group=group, hkv=hkv, nq=nq, nk=1003)
    T = oracle.num_blocks(1003, bk)
    for tau in (0.05, 0.5):
        for splits in sorted({1, 3, T}):
            o, z, mask, stats = run(mala, q, k, v, tau, bk, splits)
            rep = decode_short_parity(q, k, v, tau, bk, splits, o, z, mask)
            assert_decode(rep)
            check_stats(stats, mask, 2, hkv, group, nq, bk)


def sharp_cache(seed, B=2, group=2, hkv=2, nq=4, nk=4096, window=512):
    """Random rows (q ~ 4 N(0,1) / sqrt(d)) and one heavy key per (token,
    head), k = 4 q, placed among the last ``window`` keys: once a block has
    visited the recent tiles every row's normalizer is dominated by its heavy
    key, so the older tiles of a split that holds them are skipped."""
    hq = group * hkv
    q, k, v, _ = workloads.uniform(device="cuda", seed=seed, batch=B, heads_q=hq, heads_kv=hkv, nq=nq, nk=nk,
                                   d=128, scale=4.0, dtype=torch.float32)
    g = torch.Generator(device="cuda").manual_seed(seed)
    for b in range(B):
        for h in range(hq):
            for t in range(nq):
                pos = int(torch.randint(nk - window, nk - nq, (1,), generator=g, device="cuda"))
                k[b, pos, h // group] = 4.0 * q[b, t, h]
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


@pytest.mark.parametrize("group,nq", [(2, 4), (4, 4), (1, 16), (8, 2)])
def test_block_rule_with_skips(mala, group, nq):
    """Inputs on which the block rule skips most tiles of the split that
    holds the heavy keys: decisions, outputs and counters against the
    oracle, and the skips are really there."""
    q, k, v = sharp_cache(30 + group + nq, group=group, nq=nq)
    for splits in (1, 3, 8):
        o, z, mask, stats = run(mala, q, k, v, 0.05, 64, splits)
        assert_decode(decode_short_parity(q, k, v, 0.05, 64, splits, o, z, mask))
        check_stats(stats, mask, 2, 2, group, nq, 64)
        if splits == 1:
            m = mask.cpu().numpy()
            assert (m == 0).mean() > 0.5


def test_tau_zero_is_dense(mala):
    q, k, v = short_cache(8, group=2, nq=4, nk=777)
    for splits in (1, 5):
        o, z, mask, _ = run(mala, q, k, v, 0.0, 64, splits)
        od, zd = oracle.dense_attention(q, k, v, causal_offset=777 - 4)
        ok, err = bf16_close(host64(o), od)
        assert ok, err
        assert np.abs(host64(z) - zd).max() < 1e-4
        assert (mask.cpu().numpy() == 1).all()


def test_rows_without_keys_in_a_split(mala):
    # 257 keys, B_k 64: 5 tiles, 5 splits; the last split holds key 256,
    # which tokens 0..2 of 4 do not see
    q, k, v = short_cache(9, group=2, nq=4, nk=257)
    for tau in (0.0, 0.05):
        o, z, mask, _ = run(mala, q, k, v, tau, 64, 5)
        assert_decode(decode_short_parity(q, k, v, tau, 64, 5, o, z, mask))


def test_one_token_matches_the_single_token_layout(mala):
    q, k, v = short_cache(10, group=4, nq=1, nk=1000)
    o, z, mask, _ = run(mala, q, k, v, 0.05, 128, 3)
    assert z.shape == (2, 8)
    assert_decode(decode_short_parity(q, k, v, 0.05, 128, 3, o, z, mask))


def paged_from_contiguous(k, v, page_size, seed):
    """The first pages of every sequence scattered over a pool with spare
    pages (a permuted block table); plain copies, no arithmetic."""
    B, nk, hkv, d = k.shape
    per = -(-nk // page_size)
    g = torch.Generator(device="cuda").manual_seed(seed)
    n_pages = B * per + 3
    perm = torch.randperm(n_pages, generator=g, device="cuda")[:B * per].reshape(B, per)
    kp = torch.zeros((n_pages, page_size, hkv, d), dtype=k.dtype, device="cuda")
    vp = torch.zeros_like(kp)
    pad = per * page_size - nk
    kk = torch.nn.functional.pad(k, (0, 0, 0, 0, 0, pad)).reshape(B, per, page_size, hkv, d)
    vv = torch.nn.functional.pad(v, (0, 0, 0, 0, 0, pad)).reshape(B, per, page_size, hkv, d)
    kp[perm.reshape(-1)] = kk.reshape(-1, page_size, hkv, d)
    vp[perm.reshape(-1)] = vv.reshape(-1, page_size, hkv, d)
    return kp, vp, perm.to(torch.int32).contiguous()


@pytest.mark.parametrize("page_size,bk,splits", [(16, 64, 3), (64, 256, 2), (256, 128, 4)])
def test_paged_short_query(mala, page_size, bk, splits):
    q, k, v = short_cache(11, B=4, group=2, nq=4, nk=1024)
    kp, vp, table = paged_from_contiguous(k, v, page_size, 11)
    cap = table.shape[1] * page_size
    T = oracle.num_blocks(cap, bk)
    # full sequences: bit for bit the contiguous cache
    lens_full = torch.full((4,), 1024, dtype=torch.int32, device="cuda")
    mask_p = torch.full((4, 4, T), 255, dtype=torch.uint8, device="cuda")
    print(f"mala_decode_paged P {page_size} B_k {bk} splits {splits} (full lengths)", flush=True)
    op, zp = mala.mala_decode_paged(q, kp, vp, table, lens_full, 0.05, bk, splits, tile_mask=mask_p)
    o, z, mask, _ = run(mala, q, k, v, 0.05, bk, splits)
    assert torch.equal(op, o) and torch.equal(zp, z)
    assert torch.equal(mask_p[:, :, :mask.shape[2]], mask)
    # ragged lengths, one shorter than the query (rows before the first key)
    lens = torch.tensor([1024, 700, 65, 2], dtype=torch.int32, device="cuda")
    mask_p = torch.full((4, 4, T), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"mala_decode_paged P {page_size} B_k {bk} splits {splits} (ragged lengths)", flush=True)
    op, zp = mala.mala_decode_paged(q, kp, vp, table, lens, 0.05, bk, splits, stats=stats, tile_mask=mask_p)
    torch.cuda.synchronize()
    rep = decode_short_parity(q, k, v, 0.05, bk, splits, op, zp, mask_p, seq_lens=lens)
    assert_decode(rep)
    zz = zp.cpu().numpy()
    assert np.isneginf(zz[3, :, :2]).all() and (op[3, :2].float() == 0).all()


def test_short_query_invalid(mala):
    q, k, v = short_cache(12, group=4, nq=5, nk=256)
    with pytest.raises(mala.MalaError):  # 4 heads x 5 tokens > 16 columns
        mala.mala_decode(q, k, v, 0.05, 64, num_splits=1)


@pytest.mark.parametrize("splits", [4, 16])
def test_short_query_workload_full_size_sampled(mala, splits):
    """Batch 64, GQA 32/8, N_k = 131072, d 128, B_k 256, tau 0.05, the 4
    newest tokens per sequence: sampled (batch, head) rows against the
    oracle with the same split count."""
    wl = workloads.decode_cache(device="cuda", nq=4)
    o, z, mask, stats = run(mala, wl.q, wl.k, wl.v, wl.tau, 256, splits)
    heads = [(0, 0), (63, 31), (17, 12), (40, 7)]
    rep = decode_short_parity(wl.q, wl.k, wl.v, wl.tau, 256, splits, o, z, mask, heads=heads)
    print(rep)
    assert_decode(rep)
    assert torch.isfinite(o.float()).all()
    check_stats(stats, mask, 64, 8, 4, 4, 256)
