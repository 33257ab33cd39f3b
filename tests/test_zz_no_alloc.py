"""The allocation-free decode entry point (mala_decode_noalloc) against
mala_decode through the C ABI: identical outputs, decisions and counters on
two calls in a row, the second with a smaller input, and the size limit
rejected on the host before any launch."""

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def run_both(mala, wl, splits):
    B, _, hq, _ = wl.q.shape
    T = -(-wl.k.shape[1] // wl.block_k)
    out = []
    for fn in (mala.mala_decode, mala.mala_decode_noalloc):
        mask = torch.full((B, hq, T), 255, dtype=torch.uint8, device="cuda")
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        print(f"{fn.__name__} B={B} hq={hq} nk={wl.k.shape[1]} B_k={wl.block_k} splits={splits}", flush=True)
        o, z = fn(wl.q, wl.k, wl.v, wl.tau, wl.block_k, splits, tile_mask=mask, stats=stats)
        torch.cuda.synchronize()
        out.append((o, z, mask, stats))
    return out


def test_noalloc_matches_workspace_decode(mala):
    # first call: 4 x (16 q / 4 kv heads), N_k 8192, 8 splits
    big = workloads.decode_cache(device="cuda", seed=71, batch=4, heads_q=16, heads_kv=4, nk=8192, n_heavy=8)
    (o1, z1, m1, s1), (o2, z2, m2, s2) = run_both(mala, big, 8)
    # second call, smaller: 2 x (8 q / 2 kv heads), N_k 3000 (ragged), 3 splits
    small = workloads.decode_cache(device="cuda", seed=72, batch=2, heads_q=8, heads_kv=2, nk=3000, n_heavy=4)
    (o3, z3, m3, s3), (o4, z4, m4, s4) = run_both(mala, small, 3)
    for a, b in ((o1, o2), (z1, z2), (m1, m2), (s1, s2), (o3, o4), (z3, z4), (m3, m4), (s3, s4)):
        assert torch.equal(a, b)
    assert np.isfinite(o4.float().cpu().numpy()).all()
    assert int(s4[0]) > 0 and int(s4[1]) > 0


def test_noalloc_rejects_oversized_problem(mala):
    # 64 x 32 query heads x d 128 at 64 splits needs 67.6 MB of partials (> 64 MiB)
    q = torch.zeros((64, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 64 * 64, 8, 128), dtype=torch.bfloat16, device="cuda")
    prob = mala.make_problem(q, k, 0.05, 1, 64, k.shape[1] - 1)
    assert mala.mala_decode_workspace_size(prob, 64) > mala.MALA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(mala.MalaError) as ei:
        mala.mala_decode_noalloc(q, k, k, 0.05, 64, 64)
    assert ei.value.status == mala.MALA_ETOOLARGE
