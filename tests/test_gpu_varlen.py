"""GPU parity of the packed-sequence (variable-length) forward against the
CPU oracle: chunked prefill (N_q < N_k), ragged lengths, single-token
sequences and rows that see no key."""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_forward, bf16_close, forward_parity, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def packed(seed, nq_list, nk_list, hq=4, hkv=2, d=128, scale=5.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    tq, tk = sum(nq_list), sum(nk_list)
    q = (scale * torch.randn((tq, hq, d), generator=g, device="cuda") / d ** 0.5).bfloat16()
    k = torch.randn((tk, hkv, d), generator=g, device="cuda").bfloat16()
    v = torch.randn((tk, hkv, d), generator=g, device="cuda").bfloat16()
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(nq_list)]), dtype=torch.int32, device="cuda")
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(nk_list)]), dtype=torch.int32, device="cuda")
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("tau", [0.05, 1.0])
def test_varlen_chunked_prefill(mala, bq, bk, tau):
    nq_list = [1, 37, 64, 65, 300, 200]
    nk_list = [1, 37, 1064, 65, 300, 777]  # equal lengths and chunked prefill (cached context)
    q, k, v, cu_q, cu_k = packed(bq + bk, nq_list, nk_list)
    B, hq = len(nq_list), q.shape[1]
    mq, mk = max(nq_list), max(nk_list)
    mask = torch.full((B, hq, -(-mq // bq), -(-mk // bk)), 255, dtype=torch.uint8, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, mq, mk, tau, bq, bk, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    legal = 0
    for b, (nq, nk) in enumerate(zip(nq_list, nk_list)):
        qs, ks = int(cu_q[b]), int(cu_k[b])
        nqb, nkb = -(-nq // bq), -(-nk // bk)
        m_b = mask[b:b + 1, :, :nqb, :nkb].contiguous()
        rep = forward_parity(q[None, qs:qs + nq], k[None, ks:ks + nk], v[None, ks:ks + nk], tau, bq, bk,
                             nk - nq, o[None, qs:qs + nq].contiguous(),
                             z[None, :, qs:qs + nq].contiguous(), m_b)
        print(b, rep)
        assert_forward(rep, fp32=False)
        legal += int((m_b != 255).sum())
        # nothing written outside the sequence's own tiles
        assert (mask[b, :, nqb:] == 255).all() and (mask[b, :, :, nkb:] == 255).all()
    s = stats.cpu().numpy()
    assert s[0] == legal == int((mask != 255).sum())
    assert s[1] == int((mask == 1).sum())


def test_varlen_empty_rows(mala):
    """N_k < N_q: the first N_q - N_k rows see no key (o = 0, z = -inf); the
    others follow the rule with offset N_k - N_q. Also a sequence with no
    keys at all and one with no queries."""
    nq_list, nk_list = [100, 70, 0, 30], [40, 0, 50, 30]
    q, k, v, cu_q, cu_k = packed(3, nq_list, nk_list)
    o, z = mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, max(nq_list), max(nk_list), 0.05, 64, 64)
    torch.cuda.synchronize()
    ref = oracle.mala_forward_varlen(host64(q), host64(k), host64(v), cu_q.cpu().numpy(),
                                     cu_k.cpu().numpy(), 0.05, 64, 64)
    og, zg = host64(o), host64(z)
    empty = np.zeros(sum(nq_list), bool)
    empty[0:60] = True        # sequence 0: rows 0..59 see no key
    empty[100:170] = True     # sequence 1: no keys at all
    assert (og[empty] == 0).all() and np.isneginf(zg[:, empty]).all()
    assert np.isfinite(zg[:, ~empty]).all()
    ok, err = bf16_close(og[~empty], ref["o"][~empty])
    assert ok, err
    assert np.abs(zg[:, ~empty] - ref["z"][:, ~empty]).max() <= 1e-4


def test_varlen_matches_batched_layout_bitwise(mala):
    """Equal lengths: the packed call computes exactly what mala_fwd does on
    the batched layout."""
    B, n, hq, hkv, d = 3, 333, 4, 2, 128
    g = torch.Generator(device="cuda").manual_seed(9)
    q = (5 * torch.randn((B, n, hq, d), generator=g, device="cuda") / d ** 0.5).bfloat16()
    k = torch.randn((B, n, hkv, d), generator=g, device="cuda").bfloat16()
    v = torch.randn((B, n, hkv, d), generator=g, device="cuda").bfloat16()
    o1, z1 = mala.mala_fwd(q, k, v, 0.05, 64, 64)
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda") * n
    o2, z2 = mala.mala_fwd_varlen(q.view(B * n, hq, d), k.view(B * n, hkv, d), v.view(B * n, hkv, d), cu, cu,
                                  n, n, 0.05, 64, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(B * n, hq, d), o2)
    assert torch.equal(z1.permute(1, 0, 2).reshape(hq, B * n), z2)


def test_varlen_malformed_offsets_are_clamped(mala):
    """Decreasing or out-of-range prefix offsets are clamped to the packed
    tensors: the call completes (results for such a table are undefined)."""
    q, k, v, _, _ = packed(5, [64, 64], [64, 64])
    cu_q = torch.tensor([0, 100, 50], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, 1000, -5], dtype=torch.int32, device="cuda")
    o, z = mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, 128, 128, 0.05, 64, 64)
    torch.cuda.synchronize()
    assert o.shape == q.shape
