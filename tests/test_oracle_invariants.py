"""Pins of the CPU oracle against invariants, closed forms and independent
routines (no GPU). Each check is chosen so that a plausible slip in the
oracle - a dropped term, a wrong sign or index, a transposed operand, the
wrong visiting order or tie rule - fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def rand_problem(rng, B=1, nq=8, nk=None, hq=2, hkv=None, d=4, scale=1.5):
    nk = nq if nk is None else nk
    hkv = hq if hkv is None else hkv
    q = scale * rng.standard_normal((B, nq, hq, d))
    k = rng.standard_normal((B, nk, hkv, d))
    v = rng.standard_normal((B, nk, hkv, d))
    do = rng.standard_normal((B, nq, hq, d))
    return q, k, v, do


def retained_keys(mask_row, bk, nk, last_visible):
    keys = []
    for j, m in enumerate(mask_row):
        if m == 1:
            keys += [kk for kk in range(j * bk, min((j + 1) * bk, nk)) if kk <= last_visible]
    return keys


# ---------------------------------------------------------------------------
# dense brute force vs independent library routines
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk,hq,hkv", [(7, 7, 2, 2), (5, 9, 4, 2), (6, 6, 4, 1)])
def test_dense_matches_torch_sdpa(nq, nk, hq, hkv):
    rng = np.random.default_rng(3)
    q, k, v, do = rand_problem(rng, B=2, nq=nq, nk=nk, hq=hq, hkv=hkv, d=5)
    off = nk - nq
    o, z = oracle.dense_attention(q, k, v)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    grp = hq // hkv
    # torch's own causal-masked attention in float64 on the CPU, KV heads
    # expanded to query heads, bottom-right aligned mask
    allowed = torch.arange(nk)[None, :] <= (torch.arange(nq) + off)[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(grp, dim=2).transpose(1, 2),
        tv.repeat_interleave(grp, dim=2).transpose(1, 2), attn_mask=allowed, scale=1.0)
    out = out.transpose(1, 2)
    assert np.allclose(o, out.detach().numpy(), atol=1e-13)
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv = oracle.dense_attention_backward(q, k, v, do)
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)
    # z is the log-normalizer of each row
    s = np.einsum("bqhd,bkhd->bhqk", q, np.repeat(k, grp, axis=2))
    s = np.where(allowed.numpy()[None, None], s, -np.inf)
    assert np.allclose(z, np.log(np.exp(s).sum(-1)), atol=1e-12)


def test_dense_gradient_finite_differences():
    """<dO, O> differentiated by central differences in every input entry."""
    rng = np.random.default_rng(11)
    q, k, v, do = rand_problem(rng, nq=6, hq=1, d=3)
    dq, dk, dv = oracle.dense_attention_backward(q, k, v, do)
    eps = 1e-6

    def f(q_, k_, v_):
        return float((oracle.dense_attention(q_, k_, v_)[0] * do).sum())

    for arr_idx, (g, name) in enumerate(((dq, "q"), (dk, "k"), (dv, "v"))):
        base = [q, k, v]
        x = base[arr_idx]
        num = np.zeros_like(x)
        for idx in itertools.product(*[range(s) for s in x.shape]):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p, args_m = list(base), list(base)
            args_p[arr_idx], args_m[arr_idx] = xp, xm
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert np.allclose(g, num, atol=1e-7), name


# ---------------------------------------------------------------------------
# tau -> 0 recovers FullAttn in both passes (I1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bq,bk,nq,nk", [(2, 2, 9, 9), (4, 2, 10, 10), (2, 4, 7, 11), (3, 3, 8, 8)])
def test_tau_zero_is_dense(bq, bk, nq, nk):
    rng = np.random.default_rng(bq * 100 + bk * 10 + nq)
    q, k, v, do = rand_problem(rng, nq=nq, nk=nk, hq=4, hkv=2, scale=3.0)
    o_d, z_d = oracle.dense_attention(q, k, v)
    r = oracle.mala_forward(q, k, v, 0.0, bq, bk)
    legal = r["mask"] != 255
    assert (r["mask"][legal] == 1).all()
    assert np.allclose(r["o"], o_d, atol=1e-13)
    assert np.allclose(r["z"], z_d, atol=1e-13)
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], 0.0, bq, bk)
    assert (rb["mask"][rb["mask"] != 255] == 1).all()
    for a, b in zip((rb["dq"], rb["dk"], rb["dv"]), oracle.dense_attention_backward(q, k, v, do)):
        assert np.allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------------------
# closed form given the mask (I3, I5), the ratio bound (I4), nesting (I6)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 42, 233, 666, 1234])
@pytest.mark.parametrize("tau", [0.05, 0.3, 1.0])
def test_closed_form_bound_nesting(seed, tau):
    rng = np.random.default_rng(seed)
    bq, bk = 4, 4
    q, k, v, do = rand_problem(rng, nq=27, nk=27, hq=2, d=6, scale=4.0)
    r = oracle.mala_forward(q, k, v, tau, bq, bk)
    o_d, z_d = oracle.dense_attention(q, k, v)
    nq = nk = 27
    for h in range(2):
        s = q[0, :, h] @ k[0, :, h].T
        for row in range(nq):
            i = row // bq
            keep = retained_keys(r["mask"][0, h, i], bk, nk, row)
            w = np.exp(s[row, keep] - s[row, keep].max())
            zq = s[row, keep].max() + math.log(w.sum())
            assert abs(r["z"][0, h, row] - zq) < 1e-12                          # I3
            assert np.allclose(r["o"][0, row, h], (w / w.sum()) @ v[0, keep, h], atol=1e-12)  # I5
            assert r["z"][0, h, row] <= z_d[0, h, row] + 1e-12
        # I4: every tested tile's block margin bounds the dense log-probability
        for i in range(oracle.num_blocks(nq, bq)):
            rows = np.arange(i * bq, min((i + 1) * bq, nq))
            thr = np.log(tau) - np.log(rows + 1.0)
            for j in range(i + 1):
                keys = np.arange(j * bk, min((j + 1) * bk, nk))
                legal = keys[None, :] <= rows[:, None]
                lp = np.where(legal, s[np.ix_(rows, keys)] - z_d[0, h, rows][:, None], -np.inf)
                bound = np.max(lp.max(axis=1) - thr)
                assert r["margin"][0, h, i, j] >= bound - 1e-12
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], tau, bq, bk)
    # I6: backward support nested in forward support
    assert not ((rb["mask"] == 1) & (r["mask"] == 0)).any()
    assert ((rb["mask"] == 255) == (r["mask"] == 255)).all()


def test_backward_retained_closed_form():
    """Backward result = the standard gradient formulas restricted to the
    backward-retained (q, k) entries with P = exp(S - z)."""
    rng = np.random.default_rng(5)
    bq, bk, n = 3, 2, 10
    q, k, v, do = rand_problem(rng, nq=n, hq=2, hkv=1, d=3, scale=3.0)
    r = oracle.mala_forward(q, k, v, 0.2, bq, bk)
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], 0.2, bq, bk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(2):
        s = q[0, :, h] @ k[0, :, 0].T
        D = (do[0, :, h] * r["o"][0, :, h]).sum(-1)
        sel = np.zeros((n, n), bool)
        for row in range(n):
            sel[row, retained_keys(rb["mask"][0, h, row // bq], bk, n, row)] = True
        p = np.where(sel, np.exp(s - r["z"][0, h][:, None]), 0.0)
        dp = do[0, :, h] @ v[0, :, 0].T
        ds = p * (dp - D[:, None])
        dq[0, :, h] = ds @ k[0, :, 0]
        dk[0, :, 0] += ds.T @ q[0, :, h]
        dv[0, :, 0] += p.T @ do[0, :, h]
    assert np.allclose(rb["dq"], dq, atol=1e-12)
    assert np.allclose(rb["dk"], dk, atol=1e-12)
    assert np.allclose(rb["dv"], dv, atol=1e-12)


# ---------------------------------------------------------------------------
# shift invariance (I7), uniform-row Jacobian (I8), zero dS row sum (I9)
# ---------------------------------------------------------------------------

def test_shift_invariance():
    """Adding c to every key adds q.c to a row's scores: O and the masks are
    unchanged, z shifts by q.c (tutorial: subtracting a row constant leaves
    softmax unchanged)."""
    rng = np.random.default_rng(7)
    q, k, v, do = rand_problem(rng, nq=16, hq=2, d=4, scale=3.0)
    c = rng.standard_normal(4)
    r1 = oracle.mala_forward(q, k, v, 0.1, 4, 4)
    r2 = oracle.mala_forward(q, k + c, v, 0.1, 4, 4)
    assert (r1["mask"] == r2["mask"]).all()
    assert np.allclose(r1["o"], r2["o"], atol=1e-12)
    assert np.allclose(r2["z"] - r1["z"], np.einsum("bqhd,d->bhq", q, c), atol=1e-12)
    b1 = oracle.mala_backward(q, k, v, r1["o"], do, r1["z"], 0.1, 4, 4)
    b2 = oracle.mala_backward(q, k + c, v, r2["o"], do, r2["z"], 0.1, 4, 4)
    assert (b1["mask"] == b2["mask"]).all()
    assert np.allclose(b1["dv"], b2["dv"], atol=1e-12)
    assert np.allclose(b1["dk"], b2["dk"], atol=1e-12)


def test_uniform_row_jacobian():
    """A zero query row attends uniformly over its n = q+1 keys; the softmax
    Jacobian there has diagonal (n-1)/n^2 and off-diagonal -1/n^2 (tutorial,
    'Variance, temperature and normalization'), so dS = J dP and
    dQ_q = dS K."""
    rng = np.random.default_rng(8)
    q, k, v, do = rand_problem(rng, nq=6, hq=1, d=3)
    row = 5
    q[0, row, 0] = 0.0
    r = oracle.mala_forward(q, k, v, 0.0, 2, 2)
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], 0.0, 2, 2)
    n = row + 1
    J = np.full((n, n), -1.0 / n**2) + np.eye(n) * (1.0 / n)
    assert np.allclose(np.diag(J), (n - 1) / n**2)
    dp = v[0, :n, 0] @ do[0, row, 0]
    ds = J @ dp
    assert np.allclose(rb["dq"][0, row, 0], ds @ k[0, :n, 0], atol=1e-13)


@pytest.mark.parametrize("tau", [0.0, 0.05])
def test_zero_ds_rowsum_when_supports_equal(tau):
    """When the backward support equals the forward support for every row,
    each row of dS sums to zero and hence sum_k dK_k = sum_q rowsum(dS) q = 0."""
    rng = np.random.default_rng(9)
    q, k, v, do = rand_problem(rng, nq=12, hq=1, d=4, scale=1.0)
    r = oracle.mala_forward(q, k, v, tau, 3, 3)
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], tau, 3, 3)
    if (rb["mask"] == r["mask"]).all():
        assert np.allclose(rb["dk"].sum(axis=1), 0.0, atol=1e-12)
    else:
        pytest.skip("supports differ for this draw")


# ---------------------------------------------------------------------------
# second formulation (from scratch) and brute force over tiny problems
# ---------------------------------------------------------------------------

def test_from_scratch_formulation_bruteforce():
    """Recomputing Z from the retained set at every test (no running max,
    no rescaling) reproduces the online oracle's decisions and outputs."""
    rng = np.random.default_rng(21)
    cases = 0
    for n in range(1, 9):
        for bq, bk in itertools.product((1, 2, 4), (1, 2, 4)):
            for tau in (0.05, 0.5, 1.0, 2.0):
                q, k, v, _ = rand_problem(rng, nq=n, hq=1, d=2, scale=2.0)
                r = oracle.mala_forward(q, k, v, tau, bq, bk)
                for i in range(oracle.num_blocks(n, bq)):
                    rows, lastv, L, tiles = oracle.prefill_block_args(i, bq, bk, n, n, 0)
                    o2, z2, dec2 = oracle.forward_block_from_scratch(
                        q[0, rows, 0], k[0, :, 0], v[0, :, 0], lastv, L, tiles, tau, bk)
                    for j, dcs in dec2.items():
                        assert r["mask"][0, 0, i, j] == dcs
                    assert np.allclose(r["o"][0, rows, 0], o2, atol=1e-12)
                    assert np.allclose(r["z"][0, 0, rows], z2, atol=1e-12)
                    cases += 1
    assert cases > 500


def test_first_legal_tile_always_retained_and_rows_nonempty():
    rng = np.random.default_rng(4)
    q, k, v, _ = rand_problem(rng, nq=20, hq=1, d=4, scale=8.0)
    for bq, bk in ((4, 2), (2, 4), (5, 3)):
        r = oracle.mala_forward(q, k, v, 5.0, bq, bk)
        for i in range(oracle.num_blocks(20, bq)):
            jmax = (min((i + 1) * bq, 20) - 1) // bk
            assert r["mask"][0, 0, i, jmax] == 1
            assert r["margin"][0, 0, i, jmax] == math.inf
        assert np.isfinite(r["z"]).all() and np.isfinite(r["o"]).all()


def test_rows_without_legal_key_keep_state():
    """B_q = 4, B_k = 2: rows 4i..4i+1 have no legal key in the diagonal key
    block 2i+1. They are not updated by it, so their outputs are as if that
    tile's keys did not exist for them (causality is kept)."""
    rng = np.random.default_rng(6)
    q, k, v, _ = rand_problem(rng, nq=8, hq=1, d=3, scale=2.0)
    r = oracle.mala_forward(q, k, v, 0.0, 4, 2)
    o_d, _ = oracle.dense_attention(q, k, v)
    assert np.allclose(r["o"], o_d, atol=1e-13)
    v2 = v.copy()
    v2[0, 5] += 100.0  # key 5 is future for row 4
    r2 = oracle.mala_forward(q, k, v2, 0.0, 4, 2)
    assert np.allclose(r2["o"][0, 4], r["o"][0, 4], atol=1e-13)


def test_ragged_and_offset():
    """N_q < N_k with a bottom-right offset equals the last N_q rows of the
    equal-length problem (row q sees k <= q + N_k - N_q)."""
    rng = np.random.default_rng(12)
    q, k, v, _ = rand_problem(rng, nq=13, nk=13, hq=2, d=4, scale=3.0)
    full = oracle.mala_forward(q, k, v, 0.0, 3, 4)
    part = oracle.mala_forward(q[:, 5:], k, v, 0.0, 3, 4)
    assert part["offset"] == 5
    assert np.allclose(part["o"], full["o"][:, 5:], atol=1e-13)
    assert np.allclose(part["z"], full["z"][:, :, 5:], atol=1e-13)


# ---------------------------------------------------------------------------
# in-band branching
# ---------------------------------------------------------------------------

def test_branches_cover_both_outcomes():
    """Put a tile exactly at the threshold: the rule retains it (tie), and
    the branch enumeration also yields the skipped outcome."""
    tau = 0.5
    L = 3
    thr = math.log(tau) - math.log(L)
    # one row at position 2, keys 0..2, B_k = 1, visited 2, 1, 0
    s2 = 1.0
    s1 = s2 + thr + 1e-5          # margin at key 1: s1 - s2 - thr = 1e-5
    s0 = -30.0
    q = np.ones((1, 1, 1, 1))
    k = np.array([s0, s1, s2]).reshape(1, 3, 1, 1)
    v = np.eye(3).reshape(1, 3, 1, 3)
    rows, lastv, Lr, tiles = oracle.prefill_block_args(0, 1, 1, 1, 3, 2)
    assert Lr[0] == L
    br = oracle.forward_block_branches(q[0, rows, 0], k[0, :, 0], v[0, :, 0], lastv, Lr,
                                       tiles, tau, 1, band=1e-3)
    decs = sorted(b.decision[1] for b in br)
    assert decs == [0, 1]
    plain = oracle.forward_block(q[0, rows, 0], k[0, :, 0], v[0, :, 0], lastv, Lr, tiles, tau, 1)
    assert plain.decision[1] == 1
    assert plain.inband == []


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tau", [0.0, 0.05, 1.0])
def test_decode_single_split_equals_prefill_last_row(tau):
    rng = np.random.default_rng(13)
    q, k, v, _ = rand_problem(rng, nq=1, nk=23, hq=4, hkv=2, d=4, scale=4.0)
    dec = oracle.mala_decode(q, k, v, tau, 4, num_splits=1)
    pre = oracle.mala_forward(q, k, v, tau, 1, 4)
    assert pre["offset"] == 22
    assert np.allclose(dec["o"], pre["o"][:, 0], atol=1e-13)
    assert np.allclose(dec["z"], pre["z"][:, :, 0], atol=1e-13)
    assert (dec["mask"] == pre["mask"][:, :, 0]).all()


@pytest.mark.parametrize("splits", [1, 2, 3, 6])
def test_decode_splits_dense_at_tau_zero(splits):
    rng = np.random.default_rng(14)
    q, k, v, _ = rand_problem(rng, nq=1, nk=23, hq=4, hkv=1, d=4, scale=4.0)
    dec = oracle.mala_decode(q, k, v, 0.0, 4, num_splits=splits)
    o_d, z_d = oracle.dense_attention(q, k, v)
    assert np.allclose(dec["o"], o_d[:, 0], atol=1e-13)
    assert np.allclose(dec["z"], z_d[:, :, 0], atol=1e-13)


def test_decode_split_support_typically_contains_unsplit():
    """A split usually tests against a smaller partial normalizer than the
    unsplit run at the same tile (it lacks the later splits' mass), so it
    typically keeps at least the unsplit support - the split-KV paragraph's
    "typically", not a guarantee: tiles the unsplit run skipped can raise a
    split's normalizer above the unsplit one when the later splits hold
    little mass. Checked: the split keeps extra work somewhere, and what it
    drops of the unsplit support stays a small fraction (reported)."""
    rng = np.random.default_rng(15)
    q, k, v, _ = rand_problem(rng, nq=1, nk=64, hq=4, hkv=2, d=4, scale=5.0)
    kept = dropped = extra = 0
    for tau in (0.05, 0.5, 2.0):
        r1 = oracle.mala_decode(q, k, v, tau, 4, num_splits=1)
        for s in (2, 4, 16):
            rs = oracle.mala_decode(q, k, v, tau, 4, num_splits=s)
            kept += int((r1["mask"] == 1).sum())
            dropped += int(((r1["mask"] == 1) & (rs["mask"] == 0)).sum())
            extra += int(((r1["mask"] == 0) & (rs["mask"] == 1)).sum())
    print(f"split runs: {extra} extra retained, {dropped} of {kept} unsplit-retained dropped")
    assert extra > 0
    assert dropped <= 0.01 * kept
    assert oracle.split_ranges(10, 3) == [(0, 3), (3, 6), (6, 10)]


def test_slots_metric():
    mask = np.full((1, 1, 3, 3), 255, np.uint8)
    mask[0, 0, 0, 0] = 1
    mask[0, 0, 1, :2] = [0, 1]
    mask[0, 0, 2, :3] = [1, 1, 0]
    # rows per block 4, 4, 2 (N_q = 10), B_k = 4
    assert oracle.post_score_slots(mask, 4, 4, 10) == 4 * 4 + 4 * 4 + 2 * 4 * 2
