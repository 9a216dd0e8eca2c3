"""Pins of the oracle's training-query construction (KVSculpt, gist.science
page, section 2 "Training Query Construction").

The checks do not reuse the oracle's rotation: the closed form writes each
channel pair as a complex number turned by exp(i * angle), with the
frequencies formed from exp/log rather than a power; the hand case uses
textbook trigonometric values; the layout checks compare copied rows bit for
bit.  A wrong pairing (interleaved instead of half-split), a sign flip of the
angle, a wrong frequency exponent, a wrong future position or a mixed-up row
order fails at least one of them.
"""
import math

import numpy as np
import pytest

from oracle import kvsculpt as O


def _freqs(d, theta):
    # theta ** (-2c/d) through exp/log
    return np.array([math.exp(-(2.0 * c / d) * math.log(theta)) for c in range(d // 2)])


def _rope_complex(u, pos, theta):
    """Rows of u turned by RoPE at pos, as complex channel pairs (c, c + d/2)."""
    d = u.shape[-1]
    h = d // 2
    z = u[..., :h] + 1j * u[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * _freqs(d, theta))
    return np.concatenate([z.real, z.imag], axis=-1)


def _context(rng, g, N, d, theta):
    """Context queries built from known content: Qctx[h, t] = RoPE(u[h, t], t)."""
    u = rng.standard_normal((g, N, d))
    return u, _rope_complex(u, np.arange(N)[None, :], theta)


@pytest.mark.parametrize("d,theta", [(8, 1e4), (64, 1e6), (128, 5e5)])
def test_future_rows_are_source_content_at_future_positions(d, theta):
    """Closed form: a future row is the source's content rotated at N + j."""
    rng = np.random.default_rng(d)
    g, N, m, F = 3, 50, 7, 11
    u, Qctx = _context(rng, g, N, d, theta)
    src = rng.integers(0, N, size=(g, F))
    Q = O.training_queries(Qctx, src, m, theta)
    assert Q.shape == (g * (m + F), d)
    for h in range(g):
        want = _rope_complex(u[h, src[h]], N + np.arange(F), theta)
        got = Q[g * m + h * F: g * m + (h + 1) * F]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-11)


def test_long_context_angles_stay_exact():
    """Positions near 35k (long-context workload) keep fp64 accuracy."""
    rng = np.random.default_rng(5)
    g, N, m, F, d, theta = 1, 32768, 4, 64, 16, 1e6
    u = rng.standard_normal((N, d))
    src = rng.integers(0, N, size=(1, F))
    # only the sampled rows matter: build them directly
    Qctx = np.zeros((g, N, d))
    Qctx[0, src[0]] = _rope_complex(u[src[0]], src[0], theta)
    Qctx[0, N - m:] = _rope_complex(u[N - m:], np.arange(N - m, N), theta)
    Q = O.training_queries(Qctx, src, m, theta)
    want = _rope_complex(u[src[0]], N + np.arange(F), theta)
    np.testing.assert_allclose(Q[m:], want, rtol=0, atol=1e-9)


def test_hand_case_d2_and_d4():
    """Textbook values: one channel pair at frequency 1 (and 0.1 for theta = 100)."""
    # d = 2: content (1, 0) seen at position 1 is (cos 1, sin 1); re-embedded at
    # position N = 3 it must read (cos 3, sin 3).
    Qctx = np.array([[[0.3, -0.2], [math.cos(1.0), math.sin(1.0)], [5.0, 5.0]]])
    Q = O.training_queries(Qctx, np.array([[1]]), 1, 1e4)
    np.testing.assert_allclose(Q[0], [5.0, 5.0], rtol=0, atol=0)        # retain row
    np.testing.assert_allclose(Q[1], [-0.9899924966004454, 0.1411200080598672],
                               rtol=0, atol=1e-15)
    # d = 4, theta = 100: pairs (0, 2) at frequency 1 and (1, 3) at 0.1.
    # content (1, 2, 0, 0) at position 0 is itself; at position N + 1 = 5 it is
    # (cos 5, 2 cos 0.5, sin 5, 2 sin 0.5).
    Qctx = np.zeros((1, 4, 4))
    Qctx[0, 0] = [1.0, 2.0, 0.0, 0.0]
    Q = O.training_queries(Qctx, np.array([[0, 0]]), 0, 100.0)
    np.testing.assert_allclose(Q[1], [0.28366218546322625, 1.7551651237807455,
                                      -0.9589242746631385, 0.958851077208406],
                               rtol=0, atol=1e-15)


def test_rotation_preserves_pair_norms_and_relative_scores():
    """RoPE turns each plane: pair norms are unchanged, and a future query's
    score with a key at position t equals its content's score with the key's
    content at position t - (N + j)."""
    rng = np.random.default_rng(11)
    g, N, m, F, d, theta = 2, 30, 5, 9, 16, 1e4
    u, Qctx = _context(rng, g, N, d, theta)
    src = rng.integers(0, N, size=(g, F))
    Q = O.training_queries(Qctx, src, m, theta)
    h = d // 2
    fut = Q[g * m:].reshape(g, F, d)
    for hh in range(g):
        a = np.hypot(fut[hh, :, :h], fut[hh, :, h:])
        b = np.hypot(u[hh, src[hh], :h], u[hh, src[hh], h:])
        np.testing.assert_allclose(a, b, rtol=1e-13)
    kc = rng.standard_normal(d)
    for t in (0, 13, 29):
        key = _rope_complex(kc, t, theta)
        for j in (0, 4, 8):
            lhs = fut[1, j] @ key
            rhs = u[1, src[1, j]] @ _rope_complex(kc, t - (N + j), theta)
            assert abs(lhs - rhs) < 1e-12


def test_retain_block_is_a_bit_exact_copy_in_head_order():
    rng = np.random.default_rng(3)
    g, N, m, F, d = 4, 20, 6, 3, 8
    Qctx = rng.standard_normal((g, N, d)).astype(np.float32)
    src = rng.integers(0, N, size=(g, F))
    Q = O.training_queries(Qctx, src, m, 1e4)
    for hh in range(g):
        assert np.array_equal(Q[hh * m:(hh + 1) * m], Qctx[hh, N - m:].astype(np.float64))


def test_degenerate_shapes():
    rng = np.random.default_rng(4)
    g, N, d = 2, 10, 8
    Qctx = rng.standard_normal((g, N, d))
    # no synthetic queries: the retain block only
    Q = O.training_queries(Qctx, np.zeros((g, 0), dtype=np.int64), 3, 1e4)
    assert Q.shape == (g * 3, d)
    # no retain queries: the future block only, and a source at position 0
    # re-embedded at N is the row turned by N
    Q = O.training_queries(Qctx, np.zeros((g, 2), dtype=np.int64), 0, 1e4)
    assert Q.shape == (g * 2, d)
    np.testing.assert_allclose(Q[0], _rope_complex(Qctx[0, 0], N, 1e4), atol=1e-13)
    np.testing.assert_allclose(Q[1], _rope_complex(Qctx[0, 0], N + 1, 1e4), atol=1e-13)
    with pytest.raises(ValueError):
        O.training_queries(Qctx, np.array([[0], [N]]), 1, 1e4)
