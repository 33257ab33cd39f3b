"""GPU parity of the HIP forward kernels against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (assert_forward, bf16_close, forward_parity, fresh_mask, legal_tile_count, sample_blocks,
                    v_copies_from_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def run_fwd(mala, q, k, v, tau, bq, bk, off=None):
    B, nq, hq, _ = q.shape
    nk = k.shape[1]
    off = nk - nq if off is None else off
    mask = fresh_mask(B, hq, nq, nk, bq, bk)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_fwd(q, k, v, tau, bq, bk, causal_offset=off, stats=stats, tile_mask=mask)
    torch.cuda.synchronize()
    return o, z, mask, stats, off


def check_stats(stats, mask, B, hq, nq, nk, bq, bk, off, bf16=True):
    s = stats.cpu().numpy()
    m = mask.cpu().numpy()
    assert s[0] == legal_tile_count(B, hq, nq, nk, bq, bk, off)
    assert s[0] == int((m != 255).sum())
    assert s[1] == int((m == 1).sum())
    assert s[2] == oracle.post_score_slots(m, bq, bk, nq)
    # V copies: one per (workgroup, tile) that some block of the workgroup
    # retains - two 64-row blocks share a copy
    assert s[3] == v_copies_from_mask(m, bq, bf16)
    if bq == 64 and bf16:
        assert s[1] >= s[3]


def test_fp32_small_workload(mala):
    """fp32, N=512, d=64, B_q=B_k=64, tau=0.05, heavy keys: every block."""
    wl = workloads.small_fp32(device="cuda")
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, wl.tau, 64, 64)
    rep = forward_parity(wl.q, wl.k, wl.v, wl.tau, 64, 64, off, o, z, mask)
    print(rep)
    assert_forward(rep, fp32=True)
    check_stats(stats, mask, 1, 1, 512, 512, 64, 64, 0, bf16=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bq,bk", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_gqa_all_blocks(mala, d, bq, bk, dtype):
    """N=600 (ragged tails in both block sizes), GQA 4/2, sharp rows, two
    tolerances; every query block compared."""
    q, k, v, _ = workloads.uniform(device="cuda", seed=d + bq + bk, batch=2, heads_q=4,
                                   heads_kv=2, nq=600, d=d, scale=6.0, dtype=dtype)
    for tau in (0.05, 1.0):
        o, z, mask, stats, off = run_fwd(mala, q, k, v, tau, bq, bk)
        rep = forward_parity(q, k, v, tau, bq, bk, off, o, z, mask)
        print(tau, rep)
        assert_forward(rep, fp32=dtype == torch.float32)
        check_stats(stats, mask, 2, 4, 600, 600, bq, bk, off, bf16=dtype == torch.bfloat16)


@pytest.mark.parametrize("bq,bk", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_late_sink_moves_reference(mala, bq, bk):
    """The largest score of each row arrives at its last tile (sink keys
    0-3, met last by the diagonal-first walk): by far for head 0, by about
    the online softmax's rescale threshold for head 1, so some rows move
    their reference at the final tile and others keep P up to ~2^8. Every
    query block compared, tau in {0, 0.05, 1}."""
    q, k, v, _ = workloads.late_sink(device="cuda")
    for tau in (0.0, 0.05, 1.0):
        o, z, mask, stats, off = run_fwd(mala, q, k, v, tau, bq, bk)
        rep = forward_parity(q, k, v, tau, bq, bk, off, o, z, mask)
        print(tau, rep)
        assert_forward(rep, fp32=False)
        check_stats(stats, mask, 1, 2, 700, 700, bq, bk, off)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tau_zero_is_dense(mala, dtype):
    q, k, v, _ = workloads.uniform(device="cuda", seed=3, batch=1, heads_q=2, nq=333, d=128,
                                   scale=4.0, dtype=dtype)
    o, z, mask, _, off = run_fwd(mala, q, k, v, 0.0, 64, 64)
    m = mask.cpu().numpy()
    assert ((m == 1) | (m == 255)).all()
    od, zd = oracle.dense_attention(q, k, v)
    if dtype == torch.float32:
        assert np.abs(o.double().cpu().numpy() - od).max() < 1e-4
    else:
        ok, err = bf16_close(o.double().cpu().numpy(), od)
        assert ok, err
    assert np.abs(z.double().cpu().numpy() - zd).max() < 1e-4


def test_offset_short_query(mala):
    """N_q < N_k (chunked prefill): row q sees keys <= q + N_k - N_q."""
    q, k, v, _ = workloads.uniform(device="cuda", seed=9, batch=1, heads_q=4, heads_kv=1,
                                   nq=200, nk=777, d=128, scale=5.0, dtype=torch.bfloat16)
    for off in (577, 300, 0):
        o, z, mask, stats, off = run_fwd(mala, q, k, v, 0.05, 64, 128, off=off)
        rep = forward_parity(q, k, v, 0.05, 64, 128, off, o, z, mask)
        assert_forward(rep, fp32=False)
        check_stats(stats, mask, 1, 4, 200, 777, 64, 128, off)


def test_single_row_and_tiny(mala):
    for n in (1, 2, 65):
        q, k, v, _ = workloads.uniform(device="cuda", seed=n, batch=1, heads_q=1, nq=n, d=64,
                                       scale=3.0, dtype=torch.bfloat16)
        o, z, mask, _, off = run_fwd(mala, q, k, v, 0.5, 64, 64)
        rep = forward_parity(q, k, v, 0.5, 64, 64, off, o, z, mask)
        assert_forward(rep, fp32=False)


def test_deterministic(mala):
    wl = workloads.mha_temperature(device="cuda", batch=1, heads=4, n=1024)
    a = run_fwd(mala, wl.q, wl.k, wl.v, 0.05, 128, 128)
    b = run_fwd(mala, wl.q, wl.k, wl.v, 0.05, 128, 128)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("tau", [0.01, 0.05, 0.2])
def test_mha_temperature_full_size_sampled(mala, tau):
    """Batch 2, 32 heads, N=4096, d=128, B_q=B_k=128, bf16 (the launch the
    bench times): sampled query blocks against the oracle, stats exact."""
    wl = workloads.mha_temperature(device="cuda", with_grad=False)
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, tau, 128, 128)
    blocks = sample_blocks(2, 32, 32, 10, seed=int(tau * 1000))
    rep = forward_parity(wl.q, wl.k, wl.v, tau, 128, 128, off, o, z, mask, blocks=blocks)
    print(tau, rep)
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 2, 32, 4096, 4096, 128, 128, 0)
    assert torch.isfinite(o.float()).all() and torch.isfinite(z).all()


def test_gqa_sink_window_full_size_sampled(mala):
    """Batch 1, GQA 32/8, N=16384, d=128, B_q=128, B_k=64, tau=0.05, sinks +
    local window: sampled query blocks, stats exact."""
    wl = workloads.gqa_sink_window(device="cuda")
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, wl.tau, 128, 64)
    blocks = sample_blocks(1, 32, 128, 6, seed=3)
    rep = forward_parity(wl.q, wl.k, wl.v, wl.tau, 128, 64, off, o, z, mask, blocks=blocks)
    print(rep)
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 1, 32, 16384, 16384, 128, 64, 0)


@pytest.mark.parametrize("bq,bk", [(64, 64), (128, 64), (128, 128)])
def test_local_band_skips(mala, bq, bk):
    """A diagonal-concentrated input (N=1000, ragged) on which most tiles are
    skipped: the skip path itself, every block compared, skip rate reported."""
    wl = workloads.local_band(device="cuda", seed=11, heads=2, n=1000, width=48.0, amplitude=24.0)
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, 0.05, bq, bk)
    rep = forward_parity(wl.q, wl.k, wl.v, 0.05, bq, bk, off, o, z, mask)
    print(rep)
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 1, 2, 1000, 1000, bq, bk, off)
    s = stats.cpu().numpy()
    print("skip rate", 1 - s[1] / s[0])
    assert s[1] < 0.5 * s[0]


@pytest.mark.parametrize("name", ["local_band", "page_band"])
def test_band_workloads_full_size_sampled(mala, name):
    """Batch 1, 16 heads, N = 8192, d = 128, 64 x 64 tiles, tau = 0.05: the
    inputs behind the bench's skip-path rows (the narrow band, ~190 slots per
    query, and the page-level band, ~1,000), in the launch the bench times;
    sampled query blocks against the oracle, counters exact."""
    if name == "local_band":
        wl = workloads.local_band(device="cuda", heads=16, n=8192, d=128, block=64)
    else:
        wl = workloads.page_band(device="cuda")
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, 0.05, 64, 64)
    blocks = sample_blocks(1, 16, 128, 8, seed=5)
    rep = forward_parity(wl.q, wl.k, wl.v, 0.05, 64, 64, off, o, z, mask, blocks=blocks)
    print(rep)
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 1, 16, 8192, 8192, 64, 64, 0)
    s = stats.cpu().numpy()
    print(name, "skip rate", 1 - s[1] / s[0], "slots per query", s[2] / (16 * 8192))
    assert s[1] < s[0]



def test_long_context_sampled(mala):
    """N = 65536 (1024 query and key blocks of 64), 4 heads, d 128, a
    diagonal band, 64 x 64 tiles: the longest prefill in the tests (row
    offsets up to 2^23 elements); sampled blocks at the start, middle and
    end against the oracle, counters exact over the whole mask."""
    wl = workloads.local_band(device="cuda", heads=4, n=65536, d=128, block=64)
    print("mala_fwd 1 x 4 x 65536, d 128, 64 x 64, tau 0.05", flush=True)
    o, z, mask, stats, off = run_fwd(mala, wl.q, wl.k, wl.v, 0.05, 64, 64)
    blocks = [(0, 0, 0), (0, 1, 511), (0, 2, 1023), (0, 3, 777)]
    rep = forward_parity(wl.q, wl.k, wl.v, 0.05, 64, 64, off, o, z, mask, blocks=blocks)
    print(rep)
    assert_forward(rep, fp32=False)
    check_stats(stats, mask, 1, 4, 65536, 65536, 64, 64, 0)
