"""Pins of the oracle's use-side evaluation (KVSculpt, gist.science page,
section 2 "Problem Formulation" and "Loss Function").

The oracle takes one softmax over the concatenated cache.  The checks use
other routes: the LSE merge of per-chunk attention (pinned elsewhere against
scipy), hand arithmetic, and exact constructions whose compressed cache
carries the same attention mass and value sum as the full one.  A dropped
retain zone, a softmax over the wrong axis or a wrong normalisation of the
error fails at least one of them.
"""
import math

import numpy as np

from oracle import kvsculpt as O
from synth import WORKLOADS, make_use_batch


def test_full_cache_output_is_the_merge_of_its_two_chunks():
    rng = np.random.default_rng(1)
    nh, d, Z, m, k = 9, 6, 13, 5, 4
    Qh, Kz, Vz = rng.standard_normal((nh, d)), rng.standard_normal((Z, d)), rng.standard_normal((Z, d))
    Kr, Vr = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    Kc, Vc = rng.standard_normal((k, d)), rng.standard_normal((k, d))
    s = 1 / math.sqrt(d)
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, Kc, Vc, s)
    Yz, lz = O.reference_attention(Qh, Kz, Vz, s)
    Yr, lr = O.reference_attention(Qh, Kr, Vr, s)
    Yc, lc = O.reference_attention(Qh, Kc, Vc, s)
    full, _ = O.merge_attention(Yz, lz, Yr, lr)
    comp, _ = O.merge_attention(Yc, lc, Yr, lr)
    np.testing.assert_allclose(r["full"], full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["comp"], comp, rtol=0, atol=1e-13)
    D = comp - full
    assert abs(r["mse"] - np.mean(D ** 2)) <= 1e-15
    assert abs(r["rel"] - np.linalg.norm(D) / np.linalg.norm(full)) <= 1e-14


def test_hand_case_one_dimension():
    # scores q.k with q = 1, scale 1: exp-weights 1 and 3 (zone), 2 (retain)
    Qh = np.array([[1.0]])
    Kz, Vz = np.array([[0.0], [math.log(3.0)]]), np.array([[1.0], [5.0]])
    Kr, Vr = np.array([[math.log(2.0)]]), np.array([[2.0]])
    # one pair with the zone's mass (4) and mean value (1 + 15) / 4 = 4: lossless
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, np.array([[math.log(4.0)]]), np.array([[4.0]]), 1.0)
    assert abs(r["full"][0, 0] - 20.0 / 6.0) < 1e-14
    assert r["mse"] < 1e-28 and r["rel"] < 1e-14
    # a wrong value: output (12 + 4) / 6, error 4/6
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, np.array([[math.log(4.0)]]), np.array([[3.0]]), 1.0)
    assert abs(r["comp"][0, 0] - 16.0 / 6.0) < 1e-14
    assert abs(r["mse"] - (4.0 / 6.0) ** 2) < 1e-14
    assert abs(r["rel"] - 0.2) < 1e-14
    # a wrong mass (ln 3 instead of ln 4) with the right mean value: still an error
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, np.array([[math.log(3.0)]]), np.array([[4.0]]), 1.0)
    assert abs(r["comp"][0, 0] - (12.0 + 4.0) / 5.0) < 1e-14


def test_mass_preserving_merge_of_duplicate_keys_is_lossless():
    """Two equal keys merged into one key whose score is ln 2 higher for every
    query (queries carry a constant channel) and the mean value: the use-side
    output does not change.  Without the ln 2 shift it does."""
    rng = np.random.default_rng(2)
    nh, d, Z, m = 12, 5, 7, 3
    s = 1 / math.sqrt(d)
    Qh = rng.standard_normal((nh, d))
    Qh[:, -1] = 1.0
    Kz, Vz = rng.standard_normal((Z, d)), rng.standard_normal((Z, d))
    Kz[1] = Kz[0]
    Kr, Vr = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    Kc = np.delete(Kz, 1, axis=0)
    Vc = np.delete(Vz, 1, axis=0)
    Vc[0] = 0.5 * (Vz[0] + Vz[1])
    Kc[0, -1] += math.log(2.0) / s
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, Kc, Vc, s)
    assert r["rel"] < 1e-14
    Kc[0, -1] -= math.log(2.0) / s
    assert O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, Kc, Vc, s)["rel"] > 1e-3


def test_degenerate_cases():
    rng = np.random.default_rng(3)
    nh, d, Z, m = 6, 4, 9, 4
    s = 0.5
    Qh, Kz, Vz = rng.standard_normal((nh, d)), rng.standard_normal((Z, d)), rng.standard_normal((Z, d))
    Kr, Vr = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    # the compress zone itself: no error at all
    r = O.use_side_outputs(Qh, Kz, Vz, Kr, Vr, Kz, Vz, s)
    assert r["mse"] == 0.0 and r["rel"] == 0.0
    # no retain zone: plain chunk attention of each cache
    Kc, Vc = Kz[::3], Vz[::3]
    r = O.use_side_outputs(Qh, Kz, Vz, np.zeros((0, d)), np.zeros((0, d)), Kc, Vc, s)
    np.testing.assert_allclose(r["full"], O.reference_attention(Qh, Kz, Vz, s)[0], atol=1e-14)
    np.testing.assert_allclose(r["comp"], O.reference_attention(Qh, Kc, Vc, s)[0], atol=1e-14)
    # a retain key that dominates every score: both outputs are its value
    Q1 = Qh.copy()
    Q1[:, 0] = 1.0
    Kr1 = Kr.copy()
    Kr1[0] = 0.0
    Kr1[0, 0] = 200.0
    r = O.use_side_outputs(Q1, Kz, Vz, Kr1, Vr, Kc, Vc, s)
    np.testing.assert_allclose(r["full"], np.tile(Vr[0], (nh, 1)), atol=1e-12)
    assert r["mse"] < 1e-24


def test_held_out_queries_share_the_training_caches():
    """The held-out generator gives the same caches as the training one, and
    queries at future positions (not copies of training queries)."""
    from synth import make_batch
    w = WORKLOADS[0]
    u = make_use_batch(w, 0, per_head=16)
    b = make_batch(w, 0, with_retain=True)
    for key in ("Kz", "Vz", "Kr", "Vr"):
        assert np.array_equal(u[key], b[key])
    assert u["Qh"].shape == (1, w.g * 16, w.d)
    assert not np.isin(u["Qh"][0], b["Q"][0]).all(axis=1).any()
