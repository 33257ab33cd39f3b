"""GPU parity of the HIP backward kernels against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_backward, fresh_mask, host64, legal_tile_count, rel_l2_only

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
    mq = fresh_mask(B, hq, nq, nk, bq, bk)
    sf = torch.zeros(4, dtype=torch.int64, device="cuda")
    sb = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, z = mala.mala_fwd(q, k, v, tau, bq, bk, causal_offset=off, stats=sf, tile_mask=mf)
    dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, tau, bq, bk, causal_offset=off, stats=sb,
                               tile_mask=mb, tile_mask_dq=mq)
    torch.cuda.synchronize()
    # the dQ pass decides every tile on its own: bit for bit the key-major decisions
    assert torch.equal(mb, mq)
    return dict(o=o, z=z, dq=dq, dk=dk, dv=dv, mf=mf, mb=mb, sf=sf, sb=sb, off=off)


def hip_bwd(mala, q, k, v, do, tau, bq, bk, off):
    """A launcher of the HIP backward on given (o, z) for ``check_backward``."""
    B, nq, hq, _ = q.shape
    nk = k.shape[1]

    def run(o, z):
        mb = fresh_mask(B, hq, nq, nk, bq, bk)
        mq = fresh_mask(B, hq, nq, nk, bq, bk)
        sb = torch.zeros(4, dtype=torch.int64, device="cuda")
        print(f"mala_bwd on the oracle forward B={B} nq={nq} nk={nk} hq={hq} tau={tau} off={off}", flush=True)
        dq, dk, dv = mala.mala_bwd(q, k, v, o, do, z, tau, bq, bk, causal_offset=off, stats=sb, tile_mask=mb,
                                   tile_mask_dq=mq)
        return dq, dk, dv, mb, mq, sb
    return run


def check_all(mala, q, k, v, do, tau, r, bq=64, bk=64, key_blocks=None, query_blocks=None,
              fwd_blocks=None):
    """Strict parity of the HIP backward on the oracle forward's o, z, and
    the end-to-end pass ``r`` (HIP forward, then HIP backward) by relative
    L2; returns the strict report and the strict run's outputs."""
    rep, rep2, res = check_backward(hip_bwd(mala, q, k, v, do, tau, bq, bk, r["off"]), q, k, v, do, tau, bq, bk,
                                    r["off"], r["mf"], e2e=(r["dq"], r["dk"], r["dv"], r["mb"]),
                                    key_blocks=key_blocks, query_blocks=query_blocks, fwd_blocks=fwd_blocks)
    return rep, res


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
    check_all(mala, q, k, v, do, tau, r)
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
    # tau = 0 retains every tile: strict parity on the oracle forward, and
    # the end-to-end pass against dense attention's gradients (autograd-free
    # closed form in float64) by relative L2
    _, (dq, dk, dv, mb_iso, _, _) = check_all(mala, q, k, v, do, 0.0, r)
    assert ((mb_iso.cpu().numpy() == 1) | (mb_iso.cpu().numpy() == 255)).all()
    gq, gk, gv = oracle.dense_attention_backward(q, k, v, do)

    class R:
        err = {}
    rep = R()
    assert rel_l2_only(host64(r["dq"]), gq, "dq", rep), rep.err
    assert rel_l2_only(host64(r["dk"]), gk, "dk", rep), rep.err
    assert rel_l2_only(host64(r["dv"]), gv, "dv", rep), rep.err
    print(rep.err)
    # equal supports: every dS row sums to zero, so the dK rows sum to zero
    s = host64(dk).sum(axis=1)
    assert np.abs(s).max() < 0.05 * np.abs(gk).sum(axis=1).max()


def test_offset_short_query(mala):
    q, k, v, do = workloads.uniform(device="cuda", seed=11, batch=1, heads_q=2, heads_kv=1,
                                    nq=150, nk=400, d=128, scale=5.0, dtype=torch.bfloat16)
    for off in (250, 100):
        r = run_pass(mala, q, k, v, do, 0.05, off=off)
        check_all(mala, q, k, v, do, 0.05, r)
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


def scaled(x, k):
    return (x.float() * 2.0 ** k).bfloat16()


@pytest.mark.parametrize("hq,hkv", [(8, 4), (2, 2)])
def test_single_key(mala, hq, hkv):
    """One query row and one key per sequence: P = 1, dS = dP - D = 0, so
    dQ and dK vanish (a zero reference) and dV is the sum of the group's dO."""
    q, k, v, do = workloads.uniform(device="cuda", seed=43, batch=2, heads_q=hq, heads_kv=hkv, nq=1, d=128,
                                    scale=3.0, dtype=torch.bfloat16)
    r = run_pass(mala, q, k, v, do, 0.01)
    check_all(mala, q, k, v, do, 0.01, r)
    check_stats(r, 2, hq, 1, 1, 64, 64)
    assert r["dq"].float().abs().max() < 1e-3 and r["dk"].float().abs().max() < 1e-3
    g = hq // hkv
    dv_ref = do.float().reshape(2, 1, hkv, g, 128).sum(dim=3).bfloat16()
    assert torch.equal(r["dv"], dv_ref)


def test_zero_and_tiny_value_tiles(mala):
    """Key blocks whose V rows are all zero, or 2^-100 times the others: the
    key-major role converts each V tile to fp16 with the exponent of its own
    maximum, so these tiles take the extreme exponents. The gradients stay
    finite and match the oracle."""
    q, k, v, do = workloads.uniform(device="cuda", seed=41, batch=1, heads_q=4, heads_kv=2, nq=300, d=128,
                                    scale=5.0, dtype=torch.bfloat16)
    v = v.clone()
    v[:, 64:128] = 0
    v[:, 128:192] = scaled(v[:, 128:192], -100)
    r = run_pass(mala, q, k, v, do, 0.05)
    for key in ("dq", "dk", "dv"):
        assert torch.isfinite(r[key].float()).all(), key
    check_all(mala, q, k, v, do, 0.05, r)
    check_stats(r, 1, 4, 300, 300, 64, 64)


@pytest.mark.parametrize("k", [-24, 12])
def test_gradients_follow_a_power_of_two_scale(mala, k):
    """dO -> dO 2^k scales every gradient by 2^k, and (V, O) -> (V, O) 2^k
    scales dQ and dK by 2^k and leaves dV, all bit for bit: the exponents
    the kernels pick for their 16-bit copies of dO and of the V tiles shift
    by k and the copies stay the same bits."""
    q, k_, v, do = workloads.uniform(device="cuda", seed=31, batch=1, heads_q=4, heads_kv=2, nq=300, d=128,
                                     scale=5.0, dtype=torch.bfloat16)
    o, z = mala.mala_fwd(q, k_, v, 0.05, 64, 64)
    print(f"mala_bwd, dO and (V, O) scaled by 2^{k}", flush=True)
    dq, dk, dv = mala.mala_bwd(q, k_, v, o, do, z, 0.05, 64, 64)
    dq2, dk2, dv2 = mala.mala_bwd(q, k_, v, o, scaled(do, k), z, 0.05, 64, 64)
    for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert torch.equal(a, scaled(b, k))
    dq3, dk3, dv3 = mala.mala_bwd(q, k_, scaled(v, k), scaled(o, k), do, z, 0.05, 64, 64)
    assert torch.equal(dq3, scaled(dq, k)) and torch.equal(dk3, scaled(dk, k))
    assert torch.equal(dv3, dv)


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
    rep, _ = check_all(mala, wl.q, wl.k, wl.v, wl.do, wl.tau, r, key_blocks=key_blocks,
                       query_blocks=query_blocks)
    check_stats(r, 1, 16, 8192, 8192, 64, 64)
    sb = r["sb"].cpu().numpy()
    print("bwd skip rate", 1 - sb[1] / sb[0], "fwd skip rate", 1 - r["sf"][1].item() / r["sf"][0].item())


def test_local_band_skips(mala):
    """Backward on a diagonal-concentrated input where most tiles are skipped
    in both passes (N=1000, ragged): every block compared."""
    wl = workloads.local_band(device="cuda", seed=12, heads=2, n=1000, width=48.0, amplitude=24.0)
    r = run_pass(mala, wl.q, wl.k, wl.v, wl.do, 0.05)
    check_all(mala, wl.q, wl.k, wl.v, wl.do, 0.05, r)
    check_stats(r, 1, 2, 1000, 1000, 64, 64)
    sb = r["sb"].cpu().numpy()
    print("bwd skip rate", 1 - sb[1] / sb[0])
    assert sb[1] < 0.5 * sb[0]


@pytest.mark.parametrize("name", ["local_band", "page_band"])
def test_band_workloads_backward_full_size_sampled(mala, name):
    """The training pass on the bench's skip-path inputs at full size
    (batch 1, 16 heads, N = 8192, d = 128, 64 x 64 tiles, tau = 0.05):
    sampled key blocks (dK, dV) and query blocks (dQ), the oracle forward on
    every row they depend on."""
    if name == "local_band":
        wl = workloads.local_band(device="cuda", heads=16, n=8192, d=128, block=64)
    else:
        wl = workloads.page_band(device="cuda")
    r = run_pass(mala, wl.q, wl.k, wl.v, wl.do, 0.05)
    key_blocks = [(0, 3, 127), (0, 9, 124), (0, 15, 120)]
    query_blocks = [0, 5, 127]
    fwd_blocks = sorted({(0, g, i) for (_, g, j) in key_blocks for i in range(j, 128)}
                        | {(0, h, i) for h in range(16) for i in query_blocks})
    check_all(mala, wl.q, wl.k, wl.v, wl.do, 0.05, r, key_blocks=key_blocks, query_blocks=query_blocks,
              fwd_blocks=fwd_blocks)
    check_stats(r, 1, 16, 8192, 8192, 64, 64)
    sb = r["sb"].cpu().numpy()
    print(name, "bwd skip rate", 1 - sb[1] / sb[0], "slots per query", sb[2] / (16 * 8192))
    assert sb[1] < sb[0]



def test_long_context_backward_sampled(mala):
    """The training pass at N = 65536 (1024 blocks of 64), 4 heads, d 128,
    on a diagonal band: sampled key blocks (dK, dV) near the end and query
    blocks (dQ) at both ends against the oracle, counters exact."""
    wl = workloads.local_band(device="cuda", heads=4, n=65536, d=128, block=64)
    print("mala_fwd + mala_bwd 1 x 4 x 65536, d 128, 64 x 64, tau 0.05", flush=True)
    r = run_pass(mala, wl.q, wl.k, wl.v, wl.do, 0.05)
    key_blocks = [(0, 1, 1023), (0, 2, 1000)]
    query_blocks = [0, 1023]
    fwd_blocks = sorted({(0, g, i) for (_, g, j) in key_blocks for i in range(j, 1024)}
                        | {(0, h, i) for h in range(4) for i in query_blocks})
    check_all(mala, wl.q, wl.k, wl.v, wl.do, 0.05, r, key_blocks=key_blocks, query_blocks=query_blocks,
              fwd_blocks=fwd_blocks)
    check_stats(r, 1, 4, 65536, 65536, 64, 64)
