"""GPU parity of the HIP backward kernels against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import backward_parity, close_bf16, fresh_mask, host64, legal_tile_count, matched_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mala():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_causal_tile_amd as m
    m.load()
    return m


def run_pass(mala, q, k, v, do, tau, bq=64, bk=64, off=None):
    B, nq, hq, _ = q.shape
    nk = k.shape[1]
    off = nk - nq if off is None else off
    mf = fresh_mask(B, hq, nq, nk, bq, bk)
    mb = fresh_mask(B, hq, nq, nk, bq, bk)
    sf = torch.zeros(4, dtype=torch.int64, device="cuda")
    sb = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_fwd(q, k, v, tau, bq, bk, causal_offset=off, stats=sf, tile_mask=mf)
    dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, tau, bq, bk, causal_offset=off, stats=sb,
                               tile_mask=mb)
    torch.cuda.synchronize()
    return dict(o=o, z=z, dq=dq, dk=dk, dv=dv, mf=mf, mb=mb, sf=sf, sb=sb, off=off)


def check_all(q, k, v, do, tau, r, bq=64, bk=64, key_blocks=None, query_blocks=None,
              fwd_blocks=None):
    off = r["off"]
    o_ref, z_ref, ok = matched_forward(q, k, v, tau, bq, bk, off, r["mf"], blocks=fwd_blocks)
    assert ok, "forward decisions differ outside the band"
    rep, out = backward_parity(q, k, v, do, tau, bq, bk, off, o_ref, z_ref, r["dq"], r["dk"], r["dv"],
                               r["mb"], key_blocks=key_blocks, query_blocks=query_blocks)
    assert not rep.outband_mismatch, rep.outband_mismatch
    dq, dk, dv = host64(r["dq"]), host64(r["dk"]), host64(r["dv"])
    good = True
    if "kv" in out:
        _, dk_e, dv_e, _ = out["kv"]
        if key_blocks is None:
            good &= close_bf16(dk, dk_e, "dk", rep)
            good &= close_bf16(dv, dv_e, "dv", rep)
            if query_blocks is None:
                good &= close_bf16(dq, out["kv"][0], "dq", rep)
        else:
            sel = np.zeros(dk.shape, bool)
            for (b, g, j) in key_blocks:
                sel[b, j * bk:(j + 1) * bk, g] = True
            good &= close_bf16(dk, dk_e, "dk", rep, rows_mask=sel)
            good &= close_bf16(dv, dv_e, "dv", rep, rows_mask=sel)
    if "q" in out:
        dq_e = out["q"][0]
        sel = np.zeros(dq.shape, bool)
        for i in query_blocks:
            sel[:, i * bq:(i + 1) * bq] = True
        good &= close_bf16(dq, dq_e, "dq", rep, rows_mask=sel)
    print(rep)
    assert good, rep.err
    return rep


def check_stats(r, B, hq, nq, nk, bq, bk):
    sb, mb = r["sb"].cpu().numpy(), r["mb"].cpu().numpy()
    assert sb[0] == legal_tile_count(B, hq, nq, nk, bq, bk, r["off"]) == int((mb != 255).sum())
    assert sb[1] == int((mb == 1).sum()) == sb[3]
    assert sb[2] == oracle.post_score_slots(mb, bq, bk, nq)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tau", [0.05, 1.0, 3.0])
def test_ragged_gqa_all(mala, d, tau):
    q, k, v, do = workloads.uniform(device="cuda", seed=7 + d, batch=2, heads_q=4, heads_kv=2,
                                    nq=300, d=d, scale=6.0, dtype=torch.bfloat16)
    r = run_pass(mala, q, k, v, do, tau)
    check_all(q, k, v, do, tau, r)
    check_stats(r, 2, 4, 300, 300, 64, 64)
    # support nesting: backward retained implies forward retained (outside the band)
    mf, mb = r["mf"].cpu().numpy(), r["mb"].cpu().numpy()
    assert not ((mb == 1) & (mf == 0)).any()


def test_tau_zero_dense_gradients(mala):
    q, k, v, do = workloads.uniform(device="cuda", seed=5, batch=1, heads_q=2, nq=257, d=128,
                                    scale=3.0, dtype=torch.bfloat16)
    r = run_pass(mala, q, k, v, do, 0.0)
    mb = r["mb"].cpu().numpy()
    assert ((mb == 1) | (mb == 255)).all()
    gq, gk, gv = oracle.dense_attention_backward(q, k, v, do)

    class R:
        err = {}
    rep = R()
    assert close_bf16(host64(r["dq"]), gq, "dq", rep), rep.err
    assert close_bf16(host64(r["dk"]), gk, "dk", rep), rep.err
    assert close_bf16(host64(r["dv"]), gv, "dv", rep), rep.err
    # equal supports: every dS row sums to zero, so the dK rows sum to zero
    s = host64(r["dk"]).sum(axis=1)
    assert np.abs(s).max() < 0.05 * np.abs(gk).sum(axis=1).max()


def test_offset_short_query(mala):
    q, k, v, do = workloads.uniform(device="cuda", seed=11, batch=1, heads_q=2, heads_kv=1,
                                    nq=150, nk=400, d=128, scale=5.0, dtype=torch.bfloat16)
    for off in (250, 100):
        r = run_pass(mala, q, k, v, do, 0.05, off=off)
        check_all(q, k, v, do, 0.05, r)
        check_stats(r, 1, 2, 150, 400, 64, 64)


def test_unsupported(mala):
    q, k, v, do = workloads.uniform(device="cuda", seed=1, batch=1, heads_q=1, nq=128, d=128,
                                    dtype=torch.bfloat16)
    o, z = mala.mala_fwd(q, k, v, 0.05, 128, 128)
    with pytest.raises(mala.MalaError) as ei:
        mala.mala_bwd(q, k, v, o, do, z, 0.05, 128, 128)
    assert ei.value.status == mala.MALA_EUNSUPPORTED


def test_deterministic_masks(mala):
    q, k, v, do = workloads.uniform(device="cuda", seed=2, batch=1, heads_q=4, nq=512, d=128,
                                    scale=5.0, dtype=torch.bfloat16)
    a = run_pass(mala, q, k, v, do, 0.2)
    b = run_pass(mala, q, k, v, do, 0.2)
    # no atomics anywhere: the whole backward is bitwise reproducible
    for key in ("mb", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


def test_backward_workload_full_size_sampled(mala):
    """Batch 1, 16 heads, N=8192, d=128, B_q=B_k=64, tau=0.05 (the workload
    the bench times): full oracle forward, sampled key blocks for dK/dV and
    sampled query blocks for dQ."""
    wl = workloads.mha_backward(device="cuda")
    r = run_pass(mala, wl.q, wl.k, wl.v, wl.do, wl.tau)
    rng = np.random.default_rng(0)
    key_blocks = [(0, int(g), int(j)) for g, j in zip(rng.integers(16, size=4), rng.integers(128, size=4))]
    key_blocks += [(0, 0, 0), (0, 15, 127)]
    query_blocks = sorted({0, 127, *map(int, rng.integers(128, size=2))})
    rep = check_all(wl.q, wl.k, wl.v, wl.do, wl.tau, r, key_blocks=key_blocks,
                    query_blocks=query_blocks)
    check_stats(r, 1, 16, 8192, 8192, 64, 64)
    sb = r["sb"].cpu().numpy()
    print("bwd skip rate", 1 - sb[1] / sb[0], "fwd skip rate", 1 - r["sf"][1].item() / r["sf"][0].item())


def test_local_band_skips(mala):
    """Backward on a diagonal-concentrated input where most tiles are skipped
    in both passes (N=1000, ragged): every block compared."""
    wl = workloads.local_band(device="cuda", seed=12, heads=2, n=1000, width=48.0, amplitude=24.0)
    r = run_pass(mala, wl.q, wl.k, wl.v, wl.do, 0.05)
    check_all(wl.q, wl.k, wl.v, wl.do, 0.05, r)
    check_stats(r, 1, 2, 1000, 1000, 64, 64)
    sb = r["sb"].cpu().numpy()
    print("bwd skip rate", 1 - sb[1] / sb[0])
    assert sb[1] < 0.5 * sb[0]
