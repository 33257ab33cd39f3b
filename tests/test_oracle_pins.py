"""Pins of the CPU oracle against the pages' worked examples.

Inputs come from the attention tutorial page (tests/golden); the expected
MALA outcomes (which tiles survive, the resulting output and log-normalizer)
are derived by hand below from the rules on the MALA page, written as closed
forms over the retained key set so that a mistake in the oracle's online
bookkeeping, visiting order, threshold or tie rule fails one of them.
"""

import math

import numpy as np
import pytest

import oracle

LN = math.log


def softmax_closed(scores, values, keep):
    """Closed form of a softmax renormalized over the kept keys."""
    w = {k: math.exp(scores[k]) for k in keep}
    zs = sum(w.values())
    out = sum(w[k] * np.asarray(values[k], dtype=float) for k in keep) / zs
    return out, LN(zs)


def one_row_problem(scores, values, pos=None):
    """A single query row whose scores against keys 0..n-1 are ``scores``:
    d = 1, q = [1], k = scores. The row sits at position n-1 of an n-token
    causal sequence (decode-style: N_q = 1, offset n-1, L = n)."""
    n = len(scores)
    q = np.ones((1, 1, 1, 1))
    k = np.asarray(scores, dtype=float).reshape(1, n, 1, 1)
    v = np.asarray(values, dtype=float).reshape(1, n, 1, -1)
    return q, k, v, (n - 1 if pos is None else pos)


# ---------------------------------------------------------------------------
# tutorial: one masked attention row
# ---------------------------------------------------------------------------

def test_masked_row_dense(golden):
    ex = golden["masked_row"]
    raw, dk = ex["raw_products"], ex["d_k"]
    scaled = [x / math.sqrt(dk) for x in raw]
    assert scaled == ex["scaled_scores"]  # the page's printed scaling
    # N_q = N_k = 4, K = identity, query row 2 carries the raw products with
    # 1/sqrt(d_k) folded in; V = identity so the output row is the weights.
    q = np.zeros((1, 4, 1, 4))
    q[0, 2, 0] = np.asarray(raw, dtype=float) / math.sqrt(dk)
    k = np.eye(4).reshape(1, 4, 1, 4)
    v = np.eye(4).reshape(1, 4, 1, 4)
    o, z = oracle.dense_attention(q, k, v)
    p = o[0, 2, 0]
    assert p[3] == 0.0  # the future key gets exactly zero weight
    e = [math.exp(s) for s in scaled[:3]]
    assert np.allclose(p[:3], [x / sum(e) for x in e], atol=1e-15)
    assert abs(p.sum() - 1.0) < 1e-15
    assert abs(z[0, 0, 2] - LN(sum(e))) < 1e-14
    # printed to six digits in the derivation: 0.766157, 0.170953, 0.062890
    assert np.allclose(p[:3], [0.766157, 0.170953, 0.062890], atol=1e-6)
    # MALA with any tau keeps the diagonal (first legal) tile; at tau=0 it is dense
    r = oracle.mala_forward(q, k, v, 0.0, 4, 4)
    assert np.allclose(r["o"][0, 2, 0], p, atol=1e-15)


# ---------------------------------------------------------------------------
# tutorial: the online accumulator example under MALA's rule
# ---------------------------------------------------------------------------

def _acc(golden):
    ex = golden["accumulator"]
    return ex["scores"], ex["values"]


def test_accumulator_dense_limit(golden):
    """The page: after all four keys u / l equals direct softmax. MALA with a
    vanishing tolerance keeps every tile and reproduces it (tau -> 0 limit)."""
    s, vals = _acc(golden)
    q, k, v, off = one_row_problem(s, vals)
    want, zwant = softmax_closed(s, vals, [0, 1, 2, 3])
    for tau in (0.0, 1e-9):
        r = oracle.mala_forward(q, k, v, tau, 1, 1, causal_offset=off)
        assert (r["mask"][0, 0, 0] == 1).all()
        assert np.allclose(r["o"][0, 0, 0], want, atol=1e-14)
        assert abs(r["z"][0, 0, 0] - zwant) < 1e-14
    assert np.allclose(want, [-0.699923, 0.268941], atol=1e-6)
    assert abs(zwant - 4.331412) < 1e-6


@pytest.mark.parametrize("tau,keep,bwd_keep", [
    # tau = 0.05, L = 4: thr = ln .05 - ln 4 = -4.382027.
    #   key3 first (empty state, retained); lse = 4
    #   key2: -1 - 4 + 4.382027 = -0.617973 -> skip
    #   key1:  3 - 4 + 4.382027 =  3.382027 -> keep; lse = 4 + ln(1 + e^-1)
    #   key0:  0 - 4.313262 + 4.382027 = 0.068765 -> keep
    # backward against z = ln(e^0 + e^3 + e^4) = 4.326563: s + 0.055464
    #   -> keys 0, 1, 3 kept; key2 margin -0.944536
    (0.05, [0, 1, 3], [0, 1, 3]),
    # tau = 1: thr = -1.386294. key3; key2 -3.613706 skip; key1 0.386294 keep;
    #   key0: 0 - 4.313262 + 1.386294 = -2.926968 skip.
    # backward against z = ln(e^3 + e^4) = 4.313262: s - 2.926968 ->
    #   key1 0.073032, key3 1.073032 kept.
    (1.0, [1, 3], [1, 3]),
    # tau = 0.02: thr = ln .005 = -5.298317. key2: -1 - 4 + 5.298317 = 0.298317 keep;
    #   key1 keep; key0: 0 - 4.318173 + 5.298317 = 0.980144 keep -> dense.
    # backward against the dense z = 4.331412: s + 0.966905 -> key2 at -0.033095
    #   is dropped: a strict subset of the forward support.
    (0.02, [0, 1, 2, 3], [0, 1, 3]),
])
def test_accumulator_mala(golden, tau, keep, bwd_keep):
    s, vals = _acc(golden)
    q, k, v, off = one_row_problem(s, vals)
    r = oracle.mala_forward(q, k, v, tau, 1, 1, causal_offset=off)
    got_keep = [j for j in range(4) if r["mask"][0, 0, 0, j] == 1]
    assert got_keep == keep
    want, zwant = softmax_closed(s, vals, keep)
    assert np.allclose(r["o"][0, 0, 0], want, atol=1e-14)
    assert abs(r["z"][0, 0, 0] - zwant) < 1e-14
    # margins of the tested tiles in visiting order 3, 2, 1, 0
    thr = LN(tau) - LN(4)
    lse = 4.0
    exp_margin = {}
    for j in (2, 1, 0):
        exp_margin[j] = s[j] - lse - thr
        if j in keep:
            lse = LN(math.exp(lse) + math.exp(s[j]))
    for j in (2, 1, 0):
        assert abs(r["margin"][0, 0, 0, j] - exp_margin[j]) < 1e-12
    assert r["margin"][0, 0, 0, 3] == math.inf
    # backward decisions against the finalized z
    do = np.ones((1, 1, 1, 2))
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], tau, 1, 1, causal_offset=off)
    got_bwd = [j for j in range(4) if rb["mask"][0, 0, 0, j] == 1]
    assert got_bwd == bwd_keep
    for j in range(4):
        assert abs(rb["margin"][0, 0, 0, j] - (s[j] - zwant - thr)) < 1e-12
    assert set(got_bwd) <= set(got_keep)  # support nesting


def test_accumulator_omitted_mass(golden):
    s, vals = _acc(golden)
    q, k, v, off = one_row_problem(s, vals)
    zref = LN(sum(math.exp(x) for x in s))
    for tau, keep in ((0.05, [0, 1, 3]), (1.0, [1, 3])):
        r = oracle.mala_forward(q, k, v, tau, 1, 1, causal_offset=off)
        om = oracle.omitted_mass(r["z"][0, 0, 0], zref)
        dropped = sum(math.exp(s[j]) for j in range(4) if j not in keep)
        assert abs(om - dropped / math.exp(zref)) < 1e-14
    r = oracle.mala_forward(q, k, v, 0.05, 1, 1, causal_offset=off)
    assert abs(oracle.omitted_mass(r["z"][0, 0, 0], zref) - 0.004837) < 1e-6


def test_accumulator_split_kv(golden):
    """Split-KV: two splits {0,1} | {2,3}, each from an empty state, L = 4.

    tau = 0.1, thr = ln(.025) = -3.688879.
    unsplit: key3; key2 -1.311121 skip; key1 2.688879 keep; key0
      0 - 4.313262 + 3.688879 = -0.624383 skip -> {1, 3}.
    split A (keys 1, 0): key1 retained (empty state), lse 3; key0
      0 - 3 + 3.688879 = 0.688879 -> keep: the smaller partial normalizer
      retains extra work.  split B (3, 2): key3; key2 skip.
    combined support {0, 1, 3}.  At tau = 0.05 and tau = 1 split == unsplit."""
    s, vals = _acc(golden)
    q, k, v, _ = one_row_problem(s, vals)
    for tau, keep1, keep2 in ((0.1, [1, 3], [0, 1, 3]), (0.05, [0, 1, 3], [0, 1, 3]),
                              (1.0, [1, 3], [1, 3])):
        r1 = oracle.mala_decode(q, k, v, tau, 1, num_splits=1)
        r2 = oracle.mala_decode(q, k, v, tau, 1, num_splits=2)
        assert [j for j in range(4) if r1["mask"][0, 0, j] == 1] == keep1
        assert [j for j in range(4) if r2["mask"][0, 0, j] == 1] == keep2
        for r, keep in ((r1, keep1), (r2, keep2)):
            want, zwant = softmax_closed(s, vals, keep)
            assert np.allclose(r["o"][0, 0], want, atol=1e-14)
            assert abs(r["z"][0, 0] - zwant) < 1e-14
    r2 = oracle.mala_decode(q, k, v, 0.1, 1, num_splits=2)
    assert abs(r2["margin"][0, 0, 0] - (0 - 3 - (LN(0.1) - LN(4)))) < 1e-12


# ---------------------------------------------------------------------------
# two-row tiles: "one row retains for all", and a skipped diagonal in backward
# ---------------------------------------------------------------------------

def two_row_problem(golden):
    """Rows 2 and 3 of a 4-token sequence: row 2 carries the masked-row
    example's scaled scores, row 3 the accumulator scores; K = identity so
    S = Q; values of the accumulator example. B_q = B_k = 2, so query block 1
    = rows {2, 3} sees key tiles J1 = {2, 3} (diagonal) then J0 = {0, 1}."""
    q = np.zeros((1, 4, 1, 4))
    q[0, 2, 0] = golden["masked_row"]["scaled_scores"]
    q[0, 3, 0] = golden["accumulator"]["scores"]
    q[0, 1, 0] = [0.3, -0.2, 0.0, 0.0]
    q[0, 0, 0] = [0.1, 0.0, 0.0, 0.0]
    k = np.eye(4).reshape(1, 4, 1, 4)
    v = np.asarray(golden["accumulator"]["values"], dtype=float).reshape(1, 4, 1, 2)
    return q, k, v


def test_two_row_tau1(golden):
    """tau = 1, thr_2 = ln(1/3), thr_3 = ln(1/4).
    J1 retained (empty state). J0: row 2 margin 2 - (-0.5) + 1.098612 =
    3.598612, row 3 margin 3 - 4.006715 + 1.386294 = 0.379579 -> retained.
    Backward: J0 max(0.832244, 0.054882), J1 max(-1.667756, 1.054882):
    both retained."""
    q, k, v = two_row_problem(golden)
    r = oracle.mala_forward(q, k, v, 1.0, 2, 2)
    assert list(r["mask"][0, 0, 1]) == [1, 1]
    s2, s3 = golden["masked_row"]["scaled_scores"], golden["accumulator"]["scores"]
    vals = golden["accumulator"]["values"]
    o2, z2 = softmax_closed(s2, vals, [0, 1, 2])
    o3, z3 = softmax_closed(s3, vals, [0, 1, 2, 3])
    assert np.allclose(r["o"][0, 2, 0], o2, atol=1e-14)
    assert np.allclose(r["o"][0, 3, 0], o3, atol=1e-14)
    assert np.allclose(o2, [0.829047, 0.233843], atol=1e-6)
    assert abs(z2 - 2.266368) < 1e-6
    lse2, lse3 = -0.5, LN(math.exp(4) + math.exp(-1))
    m_row2 = 2 - lse2 - LN(1 / 3)
    m_row3 = 3 - lse3 - LN(1 / 4)
    assert abs(r["margin"][0, 0, 1, 0] - max(m_row2, m_row3)) < 1e-12
    do = np.ones((1, 4, 1, 2))
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], 1.0, 2, 2)
    assert list(rb["mask"][0, 0, 1]) == [1, 1]
    assert abs(rb["margin"][0, 0, 1, 0] - (2 - z2 - LN(1 / 3))) < 1e-12
    assert abs(rb["margin"][0, 0, 1, 1] - (4 - z3 - LN(1 / 4))) < 1e-12


def test_two_row_tau3(golden):
    """tau = 3 (above 1 is allowed): thr_2 = 0, thr_3 = ln(3/4).
    Forward J0: row 2 margin 2.5, row 3 margin -0.719033: the tile is kept
    only because row 2 fails the skip test, and row 3 is updated with it.
    Backward: J0 max(-0.266368, -1.04373), J1 max(-2.766368, -0.04373):
    both skipped - the diagonal tile is not protected in backward, and the
    block's gradients vanish."""
    q, k, v = two_row_problem(golden)
    r = oracle.mala_forward(q, k, v, 3.0, 2, 2)
    assert list(r["mask"][0, 0, 1]) == [1, 1]
    s3 = golden["accumulator"]["scores"]
    lse3 = LN(math.exp(4) + math.exp(-1))
    assert 3 - lse3 - LN(3 / 4) < 0  # row 3 alone would skip J0
    assert abs(r["margin"][0, 0, 1, 0] - 2.5) < 1e-12
    o3, z3 = softmax_closed(s3, golden["accumulator"]["values"], [0, 1, 2, 3])
    assert np.allclose(r["o"][0, 3, 0], o3, atol=1e-14)
    do = np.ones((1, 4, 1, 2))
    rb = oracle.mala_backward(q, k, v, r["o"], do, r["z"], 3.0, 2, 2)
    assert list(rb["mask"][0, 0, 1]) == [0, 0]
    assert np.all(rb["dq"][0, 2:] == 0.0)
