"""GPU parity of the HIP split-KV decode kernels against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_decode, bf16_close, decode_parity, host64, paged_decode_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def run_decode(mala, q, k, v, tau, bk, splits):
    B, _, hq, _ = q.shape
    T = oracle.num_blocks(k.shape[1], bk)
    mask = torch.full((B, hq, T), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_decode(q, k, v, tau, bk, num_splits=splits, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    return o, z, mask, stats


def small_cache(seed, B=2, hq=8, hkv=2, nk=1000, scale=4.0, heavy=True):
    q, k, v, _ = workloads.uniform(device="cuda", seed=seed, batch=B, heads_q=hq, heads_kv=hkv,
                                   nq=1, nk=nk, d=128, scale=scale, dtype=torch.float32)
    if heavy:  # a few keys aligned with a query, as in the decode workload
        g = torch.Generator(device="cuda").manual_seed(seed)
        for b in range(B):
            pos = torch.randint(0, nk, (6,), generator=g, device="cuda")
            hs = torch.randint(0, hq, (6,), generator=g, device="cuda")
            k[b, pos, hs // (hq // hkv)] = 4.0 * q[b, 0, hs]
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("bk", [64, 128, 256])
def test_group_and_tile_sizes(mala, group, bk):
    hkv = 2
    q, k, v = small_cache(group * 10 + bk, hq=group * hkv, hkv=hkv, nk=1000)
    T = oracle.num_blocks(1000, bk)
    for tau in (0.05, 1.0):
        for splits in sorted({1, 3, T}):
            o, z, mask, stats = run_decode(mala, q, k, v, tau, bk, splits)
            rep = decode_parity(q, k, v, tau, bk, splits, o, z, mask)
            assert_decode(rep)
            s = stats.cpu().numpy()
            m = mask.cpu().numpy()
            assert s[0] == m.size and s[1] == int((m == 1).sum()) and s[2] == s[1] * bk
            vl = (m.reshape(2, hkv, group, T) == 1).any(axis=2).sum()
            assert s[3] == vl


def test_tau_zero_dense(mala):
    q, k, v = small_cache(3, nk=777, heavy=False)
    for splits in (1, 4):
        o, z, mask, _ = run_decode(mala, q, k, v, 0.0, 64, splits)
        od, zd = oracle.dense_attention(q, k, v)
        ok, err = bf16_close(host64(o), od)
        assert ok, err
        assert np.abs(host64(z) - zd[:, :, 0]).max() < 1e-4
        assert (mask.cpu().numpy() == 1).all()


def test_split_support_vs_unsplit(mala):
    """Split decoding tests each tile against its split's partial
    normalizer, so it typically - not always - keeps at least the unsplit
    support (split-KV paragraph). Both runs must reproduce the oracle's
    decisions with their own split count; how many unsplit-retained
    decisions the split drops is reported, not asserted."""
    q, k, v = small_cache(4, nk=4096, scale=6.0)
    o1, z1, m1, _ = run_decode(mala, q, k, v, 0.5, 64, 1)
    o8, z8, m8, _ = run_decode(mala, q, k, v, 0.5, 64, 8)
    for S, o, z, m in ((1, o1, z1, m1), (8, o8, z8, m8)):
        assert_decode(decode_parity(q, k, v, 0.5, 64, S, o, z, m))
    a, b = m1.cpu().numpy(), m8.cpu().numpy()
    dropped = int(((a == 1) & (b == 0)).sum())
    extra = int(((a == 0) & (b == 1)).sum())
    print(f"8 splits vs 1: {extra} extra retained, {dropped} of {int((a == 1).sum())} unsplit-retained dropped")


def test_invalid_splits(mala):
    q, k, v = small_cache(5, nk=256, heavy=False)
    with pytest.raises(mala.MalaError):
        mala.mala_decode(q, k, v, 0.05, 64, num_splits=5)


@pytest.mark.parametrize("splits", [1, 4, 16])
def test_decode_workload_full_size_sampled(mala, splits):
    """Batch 64, GQA 32/8, N_k=131072, d=128, B_k=256, tau=0.05: sampled
    (batch, head) rows against the oracle with the same split count."""
    wl = workloads.decode_cache(device="cuda")
    o, z, mask, stats = run_decode(mala, wl.q, wl.k, wl.v, wl.tau, 256, splits)
    rows = [(0, 0), (0, 3), (63, 31), (17, 12), (40, 7)]
    rep = decode_parity(wl.q, wl.k, wl.v, wl.tau, 256, splits, o, z, mask, rows=rows)
    print(rep)
    assert_decode(rep)
    s = stats.cpu().numpy()
    print("per-head retain", s[1] / s[0], "V-tile load fraction", s[3] / (s[0] / 4))
    assert torch.isfinite(o.float()).all()


def paged_cache(seed, lens, page_size, hq=8, hkv=2, scale=4.0):
    """A paged cache: the sequences' pages are scattered over a pool with
    spare pages, the block table padded with pages no sequence uses."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    B = len(lens)
    max_pages = max(1, max(-(-n // page_size) for n in lens))
    n_pages = B * max_pages + 5
    q = scale * torch.randn((B, 1, hq, 128), generator=g, device="cuda") / 128 ** 0.5
    kp = torch.randn((n_pages, page_size, hkv, 128), generator=g, device="cuda")
    vp = torch.randn((n_pages, page_size, hkv, 128), generator=g, device="cuda")
    perm = torch.randperm(n_pages, generator=g, device="cuda")[:B * max_pages].reshape(B, max_pages)
    table = perm.to(torch.int32).contiguous()
    # a few heavy keys aligned with a query head of the group
    for b in range(B):
        for _ in range(4):
            if lens[b] == 0:
                break
            key = int(torch.randint(0, lens[b], (1,), generator=g, device="cuda"))
            h = int(torch.randint(0, hq, (1,), generator=g, device="cuda"))
            page = int(table[b, key // page_size])
            kp[page, key % page_size, h // (hq // hkv)] = 4.0 * q[b, 0, h]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bf = torch.bfloat16
    return q.to(bf), kp.to(bf), vp.to(bf), table, seq


@pytest.mark.parametrize("page_size,bk,splits", [(16, 64, 1), (16, 256, 4), (32, 128, 3), (64, 64, 8),
                                                 (256, 256, 2)])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 1)])
def test_paged_decode(mala, page_size, bk, splits, hq, hkv):
    """Scattered pages, per-sequence lengths (full capacity, ragged, shorter
    than one tile, fewer tiles than splits, one key, none)."""
    cap = 1536
    lens = [cap, 1000, 37, 2 * bk + 5, 1, 0]
    q, kp, vp, table, seq = paged_cache(page_size + bk + splits + hq, lens, page_size, hq=hq, hkv=hkv)
    max_pages = table.shape[1]
    B = len(lens)
    T = oracle.num_blocks(max_pages * page_size, bk)
    mask = torch.full((B, hq, T), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_decode_paged(q, kp, vp, table, seq, 0.05, bk, num_splits=splits, stats=stats,
                                  tile_mask=mask)
    torch.cuda.synchronize()
    rep = paged_decode_parity(q, kp, vp, table, seq, page_size, 0.05, bk, splits, o, z, mask)
    print(rep)
    assert_decode(rep)
    s = stats.cpu().numpy()
    m = mask.cpu().numpy()
    tiles = sum(oracle.num_blocks(n, bk) for n in lens)
    assert s[0] == tiles * hq == int((m != 255).sum())
    assert s[1] == int((m == 1).sum())


def test_paged_matches_contiguous_decode(mala):
    """The same keys as a contiguous cache and as scattered pages give the
    same bits (the page table only relocates rows)."""
    lens = [2048, 2048]
    q, kp, vp, table, seq = paged_cache(5, lens, 64)
    B, hkv = 2, kp.shape[2]
    kc = torch.stack([kp[table[b].long()].reshape(-1, hkv, 128) for b in range(B)])
    vc = torch.stack([vp[table[b].long()].reshape(-1, hkv, 128) for b in range(B)])
    for splits in (1, 8):
        o1, z1 = mala.mala_decode(q, kc.contiguous(), vc.contiguous(), 0.05, 256, num_splits=splits)
        o2, z2 = mala.mala_decode_paged(q, kp, vp, table, seq, 0.05, 256, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(z1, z2)
