"""Pins of the oracle's operator-fidelity functions (MALA page, experiments:
omitted mass, per-head relative L2, post-score slots per query, Rademacher
probe). CPU only."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")


def _ints(xs):
    return [int(x, 0) for x in xs]


def test_splitmix64_published_vectors():
    g = json.load(open(GOLDEN))
    assert oracle.splitmix64(1234567, 5).tolist() == _ints(g["seed_1234567"]["outputs"])
    assert oracle.splitmix64(0, 1).tolist() == _ints(g["seed_0"]["outputs"])


def test_splitmix64_counter_form_is_a_stream():
    # output i of a seed equals output 0 of the seed advanced by i gammas
    gamma = 0x9E3779B97F4A7C15
    xs = oracle.splitmix64(99, 6)
    for i in range(6):
        assert int(oracle.splitmix64((99 + i * gamma) % (1 << 64), 1)[0]) == int(xs[i])


def test_rademacher_signs_from_published_vector():
    g = json.load(open(GOLDEN))
    top = [1 if x >= (1 << 63) else 0 for x in _ints(g["seed_1234567"]["outputs"])]
    assert oracle.rademacher(5, 1234567).tolist() == [-1.0 if t else 1.0 for t in top]


def test_rademacher_is_balanced():
    n = 1 << 20
    r = oracle.rademacher(n, 42)
    assert set(np.unique(r).tolist()) == {-1.0, 1.0}
    assert abs(r.mean()) < 5.0 / np.sqrt(n)
    # neighbouring draws are uncorrelated
    assert abs((r[1:] * r[:-1]).mean()) < 5.0 / np.sqrt(n)


def test_slot_histogram_by_hand():
    # Nq = 5 rows in blocks of 2 (rows 2, 2, 1); Nk = 6 keys in blocks of 2.
    m = np.full((1, 1, 3, 3), 255, np.uint8)
    m[0, 0, 0, 0] = 1                 # block 0 retains 1 tile
    m[0, 0, 1, :2] = [0, 1]           # block 1 retains 1 tile (one skipped)
    m[0, 0, 2, :] = [1, 0, 1]         # block 2 (one row) retains 2 tiles
    assert oracle.slot_histogram(m, 2, 5).tolist() == [0, 4, 1, 0]


def test_slot_histogram_matches_slot_total_and_row_count():
    rng = np.random.default_rng(3)
    B, H, nq, bq, bk = 2, 3, 301, 64, 32
    nk = nq
    nqb, nkb = -(-nq // bq), -(-nk // bk)
    m = rng.integers(0, 2, size=(B, H, nqb, nkb)).astype(np.uint8)
    hist = oracle.slot_histogram(m, bq, nq)
    assert hist.sum() == B * H * nq
    slots = sum(c * bk * n for c, n in enumerate(hist.tolist()))
    assert slots == oracle.post_score_slots(m, bq, bk, nq)


def test_sq_err_heads_closed_forms():
    rng = np.random.default_rng(5)
    ref = rng.integers(-8, 8, size=(2, 7, 3, 4)).astype(np.float64)
    sd, sr = oracle.sq_err_heads(ref, ref)
    assert (sd == 0).all()
    sd, sr = oracle.sq_err_heads(ref + 0.5, ref)
    assert np.array_equal(sd, np.full((2, 3), 0.25 * 7 * 4))
    for b in range(2):
        for h in range(3):
            assert sr[b, h] == pytest.approx(np.linalg.norm(ref[b, :, h, :]) ** 2, rel=1e-15)
    x = ref * 1.5
    sd, sr = oracle.sq_err_heads(x, ref)
    assert np.sqrt(sd.sum() / sr.sum()) == pytest.approx(oracle.rel_l2(x, ref), rel=1e-12)
    assert np.allclose(np.sqrt(sd / sr), 0.5)


def test_omitted_mass_limits():
    z = np.array([1.0, 2.5, -3.0])
    assert np.array_equal(oracle.omitted_mass(z, z), np.zeros(3))
    # screened normalizer one nat below the reference: 1 - 1/e omitted
    assert oracle.omitted_mass(z - 1.0, z) == pytest.approx(np.full(3, 1.0 - np.exp(-1.0)), rel=1e-15)
