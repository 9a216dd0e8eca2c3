"""Pins of the oracle's optimizer ablations (KVSculpt, gist.science page,
section 4 "Optimizer Efficacy"): Adam in place of L-BFGS, and the search
over random restarts.

The Adam update is checked against torch.optim.Adam (a library routine, run
on the CPU in float64) and a closed form.  The Adam schedule without value
re-solves is checked against torch.optim.Adam driving the oracle's own
(separately pinned) loss gradient.  Restarts from given keys are checked
against the Select+Fit run that starts from the same keys.
"""
import numpy as np
import pytest

from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch, tiny_workload

torch = pytest.importorskip("torch")


def _torch_adam(x0, grad_fn, steps, a: O.AdamOptions):
    x = torch.tensor(np.array(x0, dtype=np.float64), requires_grad=True)
    opt = torch.optim.Adam([x], lr=a.lr, betas=(a.beta1, a.beta2), eps=a.eps)
    for _ in range(steps):
        opt.zero_grad()
        x.grad = torch.from_numpy(grad_fn(x.detach().numpy().copy()))
        opt.step()
    return x.detach().numpy()


def test_adam_step_matches_torch_adam_on_a_quadratic():
    rng = np.random.default_rng(0)
    A = rng.standard_normal((21, 21))
    H = A @ A.T / 21 + np.eye(21)
    c = rng.standard_normal(21)

    def grad(x):
        return (H @ x.reshape(-1) - c).reshape(x.shape)

    a = O.AdamOptions(lr=0.05)
    x0 = rng.standard_normal((7, 3))
    x, m, v = x0.copy(), np.zeros_like(x0), np.zeros_like(x0)
    for t in range(1, 61):
        x, m, v = O.adam_step(x, grad(x), m, v, t, a)
    np.testing.assert_allclose(x, _torch_adam(x0, grad, 60, a), rtol=0, atol=1e-12)


def test_adam_constant_gradient_closed_form():
    """With a fixed gradient the bias-corrected moments are g and g^2, so every
    step is lr * g / (|g| + eps)."""
    a = O.AdamOptions(lr=0.03, eps=1e-3)
    g = np.array([2.0, -0.5, 1e-3, 0.0])
    x, m, v = np.zeros(4), np.zeros(4), np.zeros(4)
    for t in range(1, 26):
        x, m, v = O.adam_step(x, g, m, v, t, a)
    np.testing.assert_allclose(x, -25 * a.lr * g / (np.abs(g) + a.eps), rtol=1e-13, atol=1e-16)


def test_adam_schedule_without_value_solves_is_torch_adam_on_the_loss():
    w = tiny_workload(d=8, N=40, m=8, g=2, F=6, k0=5)
    b = make_batch(w, 0)
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    opt = O.CompressOptions(iters=12, vc_every=100)
    a = O.AdamOptions(lr=0.02)
    r = O.compress_problem_adam(Q, Kz, Vz, 5, s, opt, a)
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    _, K0, V0, ok = O.init_select_fit(Q, Kz, Y, lse, 5, s)
    assert ok

    def grad(x):
        return O.loss_grad(Q, Y, lse, x, V0, s)[1]

    xt = _torch_adam(K0, grad, 12, a)
    np.testing.assert_allclose(r["Kc"], xt, rtol=0, atol=1e-11)
    assert abs(r["loss"] - O.loss(Q, Y, lse, xt, V0, s)) < 1e-10
    # no iterations: the Select+Fit loss
    r0 = O.compress_problem_adam(Q, Kz, Vz, 5, s, O.CompressOptions(iters=0), a)
    assert r0["loss"] == r0["init_loss"] == O.loss(Q, Y, lse, K0, V0, s)


def test_restart_from_top_k_keys_is_the_select_fit_run():
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    Q, Kz, Vz, s = b["Q"][0], b["Kz"][0], b["Vz"][0], b["scale"]
    opt = O.CompressOptions(iters=10)
    base = O.compress_problem(Q, Kz, Vz, 64, s, opt)
    rng = np.random.default_rng(1)
    sets = [Kz[np.sort(rng.choice(Kz.shape[0], 64, replace=False))] for _ in range(2)]
    sets.insert(1, Kz[base["idx"]])
    best, runs = O.restart_search(Q, Kz, Vz, 64, s, opt, sets)
    assert runs[1]["loss"] == base["loss"]
    np.testing.assert_array_equal(runs[1]["Kc"], base["Kc"])
    assert best == int(np.argmin([r["loss"] for r in runs]))
    # every run started from its own keys with ridge-fitted values
    Y, lse = O.reference_attention(Q, Kz, Vz, s)
    for K0, r in zip(sets, runs):
        V0, _, ok = O.ridge_values(Q, Y, K0, s)
        assert ok and abs(r["init_loss"] - O.loss(Q, Y, lse, K0, V0, s)) < 1e-9 * r["init_loss"]
