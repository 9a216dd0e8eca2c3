"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each check is independent of the oracle's own formulas: textbook routines
(scipy softmax/logsumexp, lstsq, dense BFGS recursion), closed forms, exact
special cases, finite differences and brute force.  A plausible slip in the
oracle (dropped term, wrong sign, transposed operand, wrong index) fails at
least one of them.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch, make_head, tiny_workload


def _rand_problem(rng, n=10, d=4, Z=12, peak=1.0):
    Q = rng.standard_normal((n, d)) * peak
    Kz = rng.standard_normal((Z, d))
    Vz = rng.standard_normal((Z, d))
    return Q, Kz, Vz


# ---------------------------------------------------------------- reference

def test_reference_attention_is_textbook_softmax_attention():
    rng = np.random.default_rng(1)
    Q, Kz, Vz = _rand_problem(rng, n=7, d=5, Z=9)
    s = 1 / math.sqrt(5)
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    S = np.einsum("id,jd->ij", Q, Kz) * s
    np.testing.assert_allclose(lse, logsumexp(S, axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(Y, softmax(S, axis=1) @ Vz, rtol=0, atol=1e-13)


def test_lse_composition_compress_plus_retain_equals_full_cache():
    """Chunk (Y, lse) of compress and retain zones merge into the full cache's."""
    w = tiny_workload(d=8, N=40, m=8, g=2, F=6)
    h = make_head(w, 0, 0)
    s = 1 / math.sqrt(w.d)
    fut = h["Q"][h["n_retain"]:]          # future queries see the whole cache
    Yz, lz = O.reference_attention(fut, h["Kz"], h["Vz"], s)
    Yr, lr = O.reference_attention(fut, h["Kr"], h["Vr"], s)
    Ym, lm = O.merge_attention(Yz, lz, Yr, lr)
    K = np.concatenate([h["Kz"], h["Kr"]])
    V = np.concatenate([h["Vz"], h["Vr"]])
    S = fut @ K.T * s
    np.testing.assert_allclose(lm, logsumexp(S, axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Ym, softmax(S, axis=1) @ V, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- loss

def test_loss_and_grad_vanish_when_compressed_cache_is_the_zone():
    w = tiny_workload(d=8, N=40, m=8, g=2, F=6)
    h = make_head(w, 0, 0)
    s = 1 / math.sqrt(w.d)
    Y, lse = O.reference_attention(h["Q"], h["Kz"], h["Vz"], s)
    L, g, _ = O.loss_grad(h["Q"], Y, lse, h["Kz"], h["Vz"], s)
    assert abs(L) < 1e-20
    assert np.abs(g).max() < 1e-12


def test_loss_invariant_under_joint_row_permutation():
    rng = np.random.default_rng(2)
    Q, Kz, Vz = _rand_problem(rng)
    s = 0.5
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    Kc, Vc = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    perm = rng.permutation(5)
    L1, g1, _ = O.loss_grad(Q, Y, lse, Kc, Vc, s)
    L2, g2, _ = O.loss_grad(Q, Y, lse, Kc[perm], Vc[perm], s)
    assert abs(L1 - L2) <= 1e-12 * L1
    np.testing.assert_allclose(g2, g1[perm], rtol=1e-11, atol=1e-13)


def test_loss_terms_by_hand():
    """Loss = sum of squared output errors + lam * sum of squared lse errors."""
    rng = np.random.default_rng(3)
    Q, Kz, Vz = _rand_problem(rng, n=4, d=3, Z=5)
    s = 0.7
    Y, lse = rng.standard_normal((4, 3)), rng.standard_normal(4)
    Kc, Vc = rng.standard_normal((2, 3)), rng.standard_normal((2, 3))
    tot = 0.0
    for i in range(4):
        sc = [s * sum(Q[i, c] * Kc[j, c] for c in range(3)) for j in range(2)]
        mx = max(sc)
        lh = mx + math.log(sum(math.exp(v - mx) for v in sc))
        a = [math.exp(v - lh) for v in sc]
        for c in range(3):
            yh = a[0] * Vc[0, c] + a[1] * Vc[1, c]
            tot += (yh - Y[i, c]) ** 2
        tot += 0.3 * (lh - lse[i]) ** 2
    assert abs(O.loss(Q, Y, lse, Kc, Vc, s, lam=0.3) - tot) < 1e-12 * tot


@pytest.mark.parametrize("peak", [1.0, 20.0])
@pytest.mark.parametrize("lam", [1.0, 0.0, 2.5])
def test_gradient_matches_central_finite_differences(peak, lam):
    rng = np.random.default_rng(4 + int(peak))
    n, d, Z, k = 10, 4, 12, 3
    Q, Kz, Vz = _rand_problem(rng, n=n, d=d, Z=Z)
    s = peak / math.sqrt(d)
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    Kc = Kz[[1, 5, 9]] + 0.1 * rng.standard_normal((k, d))
    Vc = rng.standard_normal((k, d))
    _, g, _ = O.loss_grad(Q, Y, lse, Kc, Vc, s, lam)
    fd = np.zeros_like(Kc)
    for j in range(k):
        for c in range(d):
            h = 1e-5 * max(1.0, abs(Kc[j, c]))
            xp, xm = Kc.copy(), Kc.copy()
            xp[j, c] += h
            xm[j, c] -= h
            fd[j, c] = (O.loss(Q, Y, lse, xp, Vc, s, lam) - O.loss(Q, Y, lse, xm, Vc, s, lam)) / (2 * h)
    assert np.linalg.norm(fd - g) <= 1e-6 * np.linalg.norm(g)


def test_gradient_k1_closed_form():
    """k = 1: Yhat_i = v for every query, so only the LSE term moves with kc."""
    rng = np.random.default_rng(5)
    Q, Kz, Vz = _rand_problem(rng, n=9, d=4, Z=7)
    s, lam = 0.5, 1.7
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    kc, v = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    L, g, _ = O.loss_grad(Q, Y, lse, kc, v, s, lam)
    want = 2 * lam * s * Q.T @ (s * Q @ kc[0] - lse)
    np.testing.assert_allclose(g[0], want, rtol=1e-12, atol=1e-12)
    want_L = ((v[0] - Y) ** 2).sum() + lam * ((s * Q @ kc[0] - lse) ** 2).sum()
    assert abs(L - want_L) < 1e-12 * want_L


# ---------------------------------------------------------------- ridge solve

def test_ridge_normal_equations_and_stacked_lstsq():
    w = tiny_workload(d=8, N=60, m=8, g=2, F=10)
    h = make_head(w, 0, 0)
    s = 1 / math.sqrt(w.d)
    Y, lse = O.reference_attention(h["Q"], h["Kz"], h["Vz"], s)
    Kc = h["Kz"][::4]
    Vc, mu, ok = O.ridge_values(h["Q"], Y, Kc, s)
    assert ok
    A = softmax(h["Q"] @ Kc.T * s, axis=1)
    k = Kc.shape[0]
    assert abs(mu - 1e-3 * np.sum(A * A) / k) < 1e-15
    M = A.T @ A + mu * np.eye(k)
    res = np.linalg.norm(M @ Vc - A.T @ Y) / np.linalg.norm(A.T @ Y)
    assert res <= 1e-10
    stacked = np.vstack([A, math.sqrt(mu) * np.eye(k)])
    rhs = np.vstack([Y, np.zeros((k, w.d))])
    ls = np.linalg.lstsq(stacked, rhs, rcond=None)[0]
    np.testing.assert_allclose(Vc, ls, rtol=1e-9, atol=1e-10)


def test_ridge_k1_closed_form():
    rng = np.random.default_rng(6)
    Q, Kz, Vz = _rand_problem(rng, n=11, d=3, Z=6)
    Y = rng.standard_normal((11, 3))
    Vc, mu, ok = O.ridge_values(Q, Y, rng.standard_normal((1, 3)), 0.6)
    assert ok and abs(mu - 1e-3 * 11) < 1e-15
    np.testing.assert_allclose(Vc[0], Y.sum(0) / (11 + 1e-3 * 11), rtol=1e-13)


# ---------------------------------------------------------------- top-k init

def test_importance_rows_sum_to_query_count_and_select_all():
    rng = np.random.default_rng(7)
    Q, Kz, Vz = _rand_problem(rng, n=13, d=4, Z=9)
    Y, lse = O.reference_attention(Q, Kz, Vz, 0.5)
    li = O.log_importance(Q, Kz, lse, 0.5)
    assert abs(np.exp(li).sum() - 13) < 1e-12
    assert list(O.select_topk(li, 9)) == list(range(9))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(8)
    for _ in range(50):
        vals = rng.integers(0, 6, size=17).astype(float)   # many exact ties
        k = int(rng.integers(1, 18))
        want = sorted(sorted(range(17), key=lambda j: (-vals[j], j))[:k])
        assert list(O.select_topk(vals, k)) == want


def test_select_fit_is_ridge_at_selected_keys():
    w = tiny_workload(d=8, N=60, m=8, g=2, F=10)
    h = make_head(w, 0, 0)
    s = 1 / math.sqrt(w.d)
    Y, lse = O.reference_attention(h["Q"], h["Kz"], h["Vz"], s)
    idx, Kc, Vc, ok = O.init_select_fit(h["Q"], h["Kz"], Y, lse, 6, s)
    imp = softmax(h["Q"] @ h["Kz"].T * s, axis=1).sum(0)
    assert list(idx) == sorted(np.argsort(-imp, kind="stable")[:6])
    np.testing.assert_array_equal(Kc, h["Kz"][idx])
    np.testing.assert_allclose(Vc, O.ridge_values(h["Q"], Y, Kc, s)[0], rtol=1e-14)


# ---------------------------------------------------------------- L-BFGS

def _dense_bfgs_inverse(hist, dim):
    s_n, y_n, _ = hist[-1]
    H = (s_n @ y_n) / (y_n @ y_n) * np.eye(dim)
    for s, y, rho in hist:                       # oldest first
        V = np.eye(dim) - rho * np.outer(y, s)
        H = V.T @ H @ V + rho * np.outer(s, s)
    return H


@pytest.mark.parametrize("m", [1, 3, 8])
def test_two_loop_equals_dense_bfgs_recursion(m):
    rng = np.random.default_rng(9 + m)
    dim = 8
    A = rng.standard_normal((dim, dim))
    A = A @ A.T + dim * np.eye(dim)               # SPD => s^T y > 0
    hist = []
    for _ in range(m):
        s = rng.standard_normal(dim)
        y = A @ s
        hist.append((s, y, 1.0 / (s @ y)))
    g = rng.standard_normal(dim)
    r = O.two_loop(g, hist)
    np.testing.assert_allclose(r, _dense_bfgs_inverse(hist, dim) @ g, rtol=1e-12, atol=1e-12)


def test_lbfgs_minimises_rosenbrock():
    def f(x):
        return float((1 - x[0]) ** 2 + 100 * (x[1] - x[0] ** 2) ** 2)

    def fg(x):
        g = np.array([-2 * (1 - x[0]) - 400 * x[0] * (x[1] - x[0] ** 2),
                      200 * (x[1] - x[0] ** 2)])
        return f(x), g

    st = O.lbfgs_minimize(f, fg, np.array([-1.2, 1.0]), 200)
    np.testing.assert_allclose(st.x, [1.0, 1.0], atol=1e-6)


def test_lbfgs_k1_convex_case_matches_lstsq():
    """k = 1 with fixed v: L(kc) = lam ||s Q kc - lse||^2 + const."""
    rng = np.random.default_rng(10)
    Q, Kz, Vz = _rand_problem(rng, n=20, d=4, Z=9)
    s, lam = 0.5, 1.0
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    v = rng.standard_normal((1, 4))
    f = lambda x: O.loss(Q, Y, lse, x, v, s, lam)
    fg = lambda x: O.loss_grad(Q, Y, lse, x, v, s, lam)[:2]
    st = O.lbfgs_minimize(f, fg, np.zeros((1, 4)), 60)
    want = np.linalg.lstsq(s * Q, lse, rcond=None)[0]
    np.testing.assert_allclose(st.x[0], want, rtol=1e-8, atol=1e-10)


def test_armijo_keeps_loss_non_increasing_between_value_solves():
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    opt = O.CompressOptions(iters=20)
    r = O.compress_problem(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"], opt, record=True)
    traj = r["traj"]
    for t in range(1, len(traj)):
        if t % opt.vc_every != 0:          # L-BFGS-only iterations
            assert traj[t] <= traj[t - 1]
    assert r["loss"] < 0.5 * r["init_loss"]
    assert r["flags"] == 0


def test_line_search_failure_flag_and_no_move():
    """c1 > 1 makes every Armijo test fail: no move, history cleared, flag set."""
    rng = np.random.default_rng(11)
    Q, Kz, Vz = _rand_problem(rng)
    s = 0.5
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    Vc = rng.standard_normal((3, 4))
    f = lambda x: O.loss(Q, Y, lse, x, Vc, s)
    fg = lambda x: O.loss_grad(Q, Y, lse, x, Vc, s)[:2]
    x0 = Kz[:3].copy()
    L0, g0 = fg(x0)
    st = O.LbfgsState(x=x0.copy(), L=L0, g=g0)
    ok = O.lbfgs_iteration(f, fg, st, O.LbfgsOptions(c1=2.0, max_backtracks=5))
    assert not ok and st.flags & O.FLAG_LINESEARCH
    np.testing.assert_array_equal(st.x, x0)


# ---------------------------------------------------------------- allocation

def test_allocation_hand_case_and_invariants():
    assert O.allocate_budget([1, 4, 9, 16], 100) == [10, 20, 30, 40]
    assert O.allocate_budget([4, 16, 36, 64], 100) == [10, 20, 30, 40]
    assert O.allocate_budget([2.0] * 8, 64) == [8] * 8
    assert O.allocate_budget([1, 2, 3, 4], 100, alpha=1.0) == [10, 20, 30, 40]


def test_allocation_bounds_sum_and_monotonicity():
    rng = np.random.default_rng(12)
    for _ in range(300):
        P = int(rng.integers(1, 40))
        mse = np.exp(rng.normal(0, 3, size=P))
        kmax = int(rng.integers(2, 50))
        kmin = int(rng.integers(1, kmax))
        K = int(rng.integers(P * kmin, P * kmax + 1))
        k = O.allocate_budget(list(mse), K, 0.5, kmin, kmax)
        assert sum(k) == K
        assert all(kmin <= v <= kmax for v in k)
        order = np.argsort(mse)
        ks = np.array(k)[order]
        assert np.all(np.diff(ks) >= -1)   # floors + remainders: monotone up to one unit
        # scaling every MSE by 4 scales every sqrt weight by exactly 2
        assert O.allocate_budget(list(mse * 4.0), K, 0.5, kmin, kmax) == k


def test_allocation_largest_remainder_ties_go_to_lower_index():
    assert O.allocate_budget([1.0, 1.0, 1.0], 4) == [2, 1, 1]
    assert O.allocate_budget([0.0, 0.0, 0.0, 0.0], 6) == [2, 2, 1, 1]


def test_allocation_rejects_infeasible_budget():
    with pytest.raises(ValueError):
        O.allocate_budget([1.0, 2.0], 10, k_max=4)


# ---------------------------------------------------------------- pins added for branches no other pin reaches

def test_output_mse_by_hand():
    """Output MSE = ||Yhat - Y||_F^2 / (n d), the LSE term excluded.

    Two equal keys give every query the weights (1/2, 1/2), so Yhat is the
    mean of the two value rows whatever the queries; the reference lse is
    far from lhat, so any LSE contribution would show."""
    Q = np.array([[0.3, -1.0], [2.0, 0.5]])
    Kc = np.array([[1.0, 1.0], [1.0, 1.0]])
    Vc = np.array([[1.0, 0.0], [3.0, 2.0]])          # mean row (2, 1)
    Y = np.array([[1.0, 2.0], [3.0, 4.0]])           # residuals (1,-1), (-1,-3): squares sum 12
    lse = np.array([100.0, -100.0])
    assert O.output_mse(Q, Y, lse, Kc, Vc, 0.7) == pytest.approx(12.0 / 4.0, rel=0, abs=1e-14)
    # one key: Yhat = v for every query; ||Y||^2 = 30 over n d = 4 entries
    assert O.output_mse(Q, Y, lse, Kc[:1], np.zeros((1, 2)), 0.7) == pytest.approx(7.5, abs=1e-14)
    # a rectangular case (n = 3, d = 2): the divisor is n d, not n or d
    Y3 = np.vstack([Y, [[0.0, 2.0]]])                # third residual (2, -1): 5 more
    Q3 = np.vstack([Q, [[1.0, 1.0]]])
    assert O.output_mse(Q3, Y3, np.zeros(3), Kc, Vc, 0.7) == pytest.approx(17.0 / 6.0, abs=1e-14)


def test_nondescent_direction_clears_history_and_flags():
    """A stored pair of negative curvature (which the curvature guard would
    never admit, planted here) turns the two-loop output into an ascent
    direction on f = |x|^2 / 2.  The iteration must flag it, drop the
    history, and take the steepest-descent step with the first step size
    1/max(1, ||g||); the accepted step then leaves exactly one pair.

    By hand: g = x0 = (1, 2, 3); with s = (1, 0, 0), y = (-1, 0, 0),
    rho = -1: a = rho s.g = -1, q = g - a y = (0, 2, 3), gamma = s.y / y.y = -1,
    r = gamma q = (0, -2, -3), b = rho y.r = 0, r += (a - b) s -> (-1, -2, -3),
    p = -r = g, so g.p = 14 > 0."""
    f = lambda x: 0.5 * float(x @ x)
    fg = lambda x: (f(x), x.copy())
    x0 = np.array([1.0, 2.0, 3.0])
    s, y = np.array([1.0, 0.0, 0.0]), np.array([-1.0, 0.0, 0.0])
    np.testing.assert_allclose(O.two_loop(x0, [(s, y, -1.0)]), -x0, rtol=0, atol=1e-15)
    st = O.LbfgsState(x=x0.copy(), L=f(x0), g=x0.copy(), hist=[(s, y, -1.0)])
    ok = O.lbfgs_iteration(f, fg, st, O.LbfgsOptions())
    assert ok
    assert st.flags == O.FLAG_NONDESCENT
    a0 = 1.0 / math.sqrt(14.0)
    assert st.last_alpha == a0 and st.trials == 1       # Armijo holds at once on this quadratic
    np.testing.assert_allclose(st.x, x0 * (1.0 - a0), rtol=0, atol=1e-15)
    assert len(st.hist) == 1
    s_new, y_new, rho_new = st.hist[0]
    np.testing.assert_allclose(s_new, -a0 * x0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(y_new, s_new, rtol=0, atol=1e-15)     # Hessian = I
    # an empty history is not a non-descent event: no flag
    st2 = O.LbfgsState(x=x0.copy(), L=f(x0), g=x0.copy())
    O.lbfgs_iteration(f, fg, st2, O.LbfgsOptions())
    assert st2.flags == 0


@pytest.mark.parametrize("alpha", [0.5, 1.0])
def test_pilot_allocate_wiring(alpha):
    """pilot_allocate = compress_problem for pilot_iters at uniform k0, its
    output MSE, then the (separately pinned) flat split of K_total = P k0
    with exponent alpha and bounds [1, Z].  The pilot MSEs differ enough that
    alpha = 0.5 and alpha = 1 give different budgets, checked by hand from
    the continuous shares."""
    w = tiny_workload(d=8, N=40, m=8, g=2, F=6, layers=1, kv_heads=3, k0=6)
    b = make_batch(w, 0)
    probs = [(b["Q"][p], b["Kz"][p], b["Vz"][p]) for p in range(3)]
    # widen the spread: scale the values of problems 1 and 2 up (pilot MSEs
    # about 0.049, 0.042, 0.025: shares 6.9/6.3/4.8 at alpha 0.5,
    # 7.7/6.5/3.8 at alpha 1, no bound binds)
    probs[1] = (probs[1][0], probs[1][1], probs[1][2] * 2.0)
    probs[2] = (probs[2][0], probs[2][1], probs[2][2] * 2.0)
    opt = O.CompressOptions()
    mse, ks, res = O.pilot_allocate(probs, w.k0, b["scale"], opt, pilot_iters=5, alpha=alpha)
    for p, (Q, Kz, Vz) in enumerate(probs):
        r = O.compress_problem(Q, Kz, Vz, w.k0, b["scale"], O.CompressOptions(iters=5))
        assert mse[p] == r["mse"]
        assert res[p]["traj"] == r["traj"]
    Z = w.Z
    assert ks == O.allocate_budget(mse, 3 * w.k0, alpha, 1, Z)
    assert sum(ks) == 18
    # by hand: continuous shares 18 w_p / sum w, w = mse**alpha, then floors
    # and largest remainders (no bound binds at these sizes)
    wts = [m ** alpha for m in mse]
    x = [18.0 * v / sum(wts) for v in wts]
    fl = [math.floor(v) for v in x]
    left = 18 - sum(fl)
    for p in sorted(range(3), key=lambda q: (-(x[q] - fl[q]), q))[:left]:
        fl[p] += 1
    assert ks == fl
    assert ks == ([7, 6, 5] if alpha == 0.5 else [8, 6, 4])
    other = O.pilot_allocate(probs, w.k0, b["scale"], opt, pilot_iters=5,
                             alpha=1.5 - alpha)[1]
    assert other != ks


def test_nonfinite_value_row_flags_and_freezes():
    """One NaN value row makes the zone's output NaN for every query (every
    weight is positive), so the loss at the start is NaN: FLAG_NONFINITE.
    Every Armijo test against a NaN loss is false, so every search fails:
    FLAG_LINESEARCH, and the keys stay at the Select+Fit choice.  The ridge
    solve passes the NaN right-hand side through instead of raising.  A
    finite problem keeps flags 0."""
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    Q, Kz = b["Q"][0], b["Kz"][0]
    Vz = b["Vz"][0].astype(np.float64).copy()
    Vz[7, :] = np.nan
    r = O.compress_problem(Q, Kz, Vz, w.k0, b["scale"], O.CompressOptions(iters=10))
    assert r["flags"] == O.FLAG_NONFINITE | O.FLAG_LINESEARCH
    assert np.isnan(r["loss"]) and np.isnan(r["init_loss"])
    np.testing.assert_array_equal(r["Kc"], Kz[r["idx"]].astype(np.float64))
    assert O.compress_problem(Q, Kz, b["Vz"][0], w.k0, b["scale"],
                              O.CompressOptions(iters=10))["flags"] == 0


def test_keys_f32_variant_is_the_schedule_at_float32_keys():
    """The sensitivity variant keeps every iterate float32-representable and
    reports the loss at those keys; with it off the schedule is unchanged."""
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    plain = O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=7))
    again = O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=7, keys_f32=False))
    assert plain["loss"] == again["loss"]
    r = O.compress_problem(Q, Kz, Vz, w.k0, s, O.CompressOptions(iters=7, keys_f32=True))
    assert np.array_equal(r["Kc"], r["Kc"].astype(np.float32).astype(np.float64))
    Y, l = O.reference_attention(Q, Kz, Vz, s)
    assert r["loss"] == O.loss(Q, Y, l, r["Kc"], r["Vc"], s)
    assert abs(r["loss"] / plain["loss"] - 1) < 0.05
