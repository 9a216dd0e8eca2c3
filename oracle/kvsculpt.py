"""Float64 CPU oracle of KVSculpt's per-(layer, KV-head) cache-distillation optimizer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it, and it shares no code with the HIP library: it is written
from the definitions on the pages, in NumPy/SciPy float64, one plain step at
a time, so that a reader can check it against the pages by eye.

Pages (cited by title and section):
  [abs]  KVSculpt: KV Cache Compression as Distillation -- arXiv abstract
         (mlsanity.com and arxiv.science pages).
  [gist] KVSculpt: KV Cache Compression as Distillation -- gist.science page,
         section 2 "Methodology" (subsections "Problem Formulation",
         "Loss Function", "Optimization Strategy (Alternating)",
         "Training Query Construction", "Adaptive Budget Allocation") and
         section 4 "Experimental Results".

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.  Textbook sources: L-BFGS two-loop
recursion and backtracking Armijo search follow Nocedal & Wright, Numerical
Optimization (2nd ed.), Algorithms 7.4/7.5 and 3.1.

Per-problem arrays are 2-D: Q [n, d], Y [n, d], lse [n], Kz/Vz [Z, d],
Kc/Vc [k, d].  ``scale`` is 1/sqrt(d).

Pins (tests/test_oracle_*.py): LSE composition identity, zero loss/gradient
at k = Z with the compress zone itself, permutation invariance, central
finite differences (plain and peaky logits), the k = 1 closed forms,
normal-equation residual and the stacked least-squares routine for the
ridge solve, dense BFGS inverse-Hessian recursion for the two-loop output,
Rosenbrock and convex least squares for the optimizer, brute-force search
on a tiny instance, and hand cases plus invariants for the allocator.
Training-query construction (tests/test_oracle_queries.py): a complex-
exponential closed form, textbook trigonometric values, norm and relative-
position invariants, layout.  Use-side evaluation (tests/test_oracle_use.py):
the LSE merge of per-chunk attention, hand arithmetic, a mass-preserving
exact merge of duplicate keys, degenerate caches.  Optimizer ablations
(tests/test_oracle_ablations.py): the Adam update against torch.optim.Adam
and a constant-gradient closed form, the Adam schedule without value solves
against torch.optim.Adam on the loss, restarts against the Select+Fit run.
Allocation variants (tests/test_oracle_alloc_variants.py): two-level split
by hand and by its reductions to the flat split; value-norm signal by hand
and invariances.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence

import numpy as np
from scipy.linalg import LinAlgError, cho_factor, cho_solve

# per-problem status bits (same meaning as the library's flags word)
FLAG_NONFINITE = 1
FLAG_CHOLESKY = 2
FLAG_LINESEARCH = 4
FLAG_NONDESCENT = 8


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# attention pieces
# --------------------------------------------------------------------------

def logits(Q, K, scale):
    """S = Q K^T * scale (scaled dot-product scores)."""
    return (_f64(Q) @ _f64(K).T) * scale


def row_logsumexp(S):
    """Natural-log log-sum-exp of each row, shifted by the row max."""
    m = S.max(axis=1)
    return m + np.log(np.exp(S - m[:, None]).sum(axis=1))


def reference_attention(Q, Kz, Vz, scale):
    """Attention of the training queries over the compress zone only.

    [gist] "Problem Formulation": the target is the attention output of the
    full cache for future queries; "Loss Function": the LSE term keeps the
    attention mass assigned to the context chunk right when it is combined
    with later tokens.  Reading: Y and lse are the chunk's output and
    log-sum-exp over the compress zone alone (no causal mask, every training
    query comes after the whole zone), so they merge with the retain zone
    by the usual log-sum-exp composition.
    Returns (Y [n, d], lse [n]).
    """
    S = logits(Q, Kz, scale)
    lse = row_logsumexp(S)
    A = np.exp(S - lse[:, None])
    return A @ _f64(Vz), lse


def merge_attention(Y1, l1, Y2, l2):
    """Combine two disjoint chunks' (output, lse) into the union's."""
    l = np.logaddexp(l1, l2)
    Y = np.exp(l1 - l)[:, None] * Y1 + np.exp(l2 - l)[:, None] * Y2
    return Y, l


# --------------------------------------------------------------------------
# initialisation: top-k attention importance (Select) + value fit
# --------------------------------------------------------------------------

def log_importance(Q, Kz, lse, scale):
    """log of each compress key's attention importance.

    [gist] "Optimization Strategy", Initialization: keys start at the top-k
    positions by attention importance.  Reading: importance_j is the sum over
    all training queries of the softmax weight of key j, i.e.
    sum_i exp(S_ij - lse_i); it is ranked through its logarithm, a column
    log-sum-exp, which cannot underflow.
    """
    S = logits(Q, Kz, scale) - _f64(lse)[:, None]
    m = S.max(axis=0)
    return m + np.log(np.exp(S - m[None, :]).sum(axis=0))


def select_topk(logimp, k):
    """Indices of the k largest log-importances; ties go to the lower position.

    Returned in ascending position order.
    """
    logimp = _f64(logimp)
    order = np.lexsort((np.arange(logimp.size), -logimp))
    return np.sort(order[:k]).astype(np.int64)


def softmax_rows(S):
    lse = row_logsumexp(S)
    return np.exp(S - lse[:, None]), lse


def ridge_values(Q, Y, Kc, scale, ridge_rel=1e-3):
    """Closed-form values for fixed keys.

    [gist] "Optimization Strategy": with the keys held fixed, the values
    have a closed-form ridge-regression (least-squares) solution given the
    current keys' attention weights; the arXiv abstract [abs] says the same.
    Reading: A = softmax(Q Kc^T scale) over the k compressed keys, ridge
    constant mu = ridge_rel * trace(A^T A) / k, and
    (A^T A + mu I) Vc = A^T Y solved by Cholesky and two triangular solves.
    The ridge term only regularises this solve; it is not part of the loss.
    Returns (Vc [k, d], mu, ok).
    """
    A, _ = softmax_rows(logits(Q, Kc, scale))
    Gm = A.T @ A
    k = Gm.shape[0]
    mu = ridge_rel * np.trace(Gm) / k
    try:
        c = cho_factor(Gm + mu * np.eye(k), lower=True, check_finite=True)
    except (LinAlgError, ValueError):
        return None, mu, False
    # plain arithmetic: a non-finite right-hand side gives non-finite values
    return cho_solve(c, A.T @ _f64(Y), check_finite=False), mu, True


def init_select_fit(Q, Kz, Y, lse, k, scale, ridge_rel=1e-3):
    """Select+Fit warm start: top-k keys by importance, values by ridge fit.

    [abs] Select+Fit is attention-score eviction with least-squares value
    fitting; [gist] "Optimization Strategy" uses the top-k positions as the
    keys' warm start.  Returns (idx, Kc, Vc, ok).
    """
    idx = select_topk(log_importance(Q, Kz, lse, scale), k)
    Kc = _f64(Kz)[idx]
    Vc, _, ok = ridge_values(Q, Y, Kc, scale, ridge_rel)
    return idx, Kc, Vc, ok


# --------------------------------------------------------------------------
# loss and gradient
# --------------------------------------------------------------------------

def loss_terms(Q, Y, lse, Kc, Vc, scale, lam=1.0):
    """Two-term distillation loss.

    [gist] "Loss Function": output term ||Yhat - Y||_F^2 and LSE term
    ||lhat - l||^2.  Reading: plain sums over every training query (retain
    and future rows weighted alike), the LSE term weighted by lam (1.0),
    natural logarithm.
    """
    S = logits(Q, Kc, scale)
    lh = row_logsumexp(S)
    A = np.exp(S - lh[:, None])
    Yh = A @ _f64(Vc)
    R = Yh - _f64(Y)
    e = lh - _f64(lse)
    out = float((R * R).sum())
    lterm = float((e * e).sum())
    return out + lam * lterm, dict(out=out, lse_term=lterm, Yh=Yh, lh=lh, A=A, R=R, e=e)


def loss(Q, Y, lse, Kc, Vc, scale, lam=1.0):
    return loss_terms(Q, Y, lse, Kc, Vc, scale, lam)[0]


def loss_grad(Q, Y, lse, Kc, Vc, scale, lam=1.0):
    """Loss and its gradient with respect to the compressed keys.

    Chain rule through Yhat = softmax(S) Vc and lhat = LSE(S):
      G = 2 (Yhat - Y), dA = G Vc^T, delta_i = G_i . Yhat_i,
      dS = A * (dA - delta 1^T + 2 lam (lhat - l) 1^T),
      dL/dKc = dS^T Q * scale.
    Returns (L, grad [k, d], aux).
    """
    L, aux = loss_terms(Q, Y, lse, Kc, Vc, scale, lam)
    G = 2.0 * aux["R"]
    dA = G @ _f64(Vc).T
    delta = (G * aux["Yh"]).sum(axis=1)
    dS = aux["A"] * (dA - delta[:, None] + 2.0 * lam * aux["e"][:, None])
    grad = (dS.T @ _f64(Q)) * scale
    return L, grad, aux


def output_mse(Q, Y, lse, Kc, Vc, scale):
    """Per-problem output MSE ||Yhat - Y||_F^2 / (n d) (the pilot signal)."""
    _, aux = loss_terms(Q, Y, lse, Kc, Vc, scale, 0.0)
    n, d = np.shape(Y)
    return aux["out"] / (n * d)


# --------------------------------------------------------------------------
# L-BFGS on the keys
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LbfgsOptions:
    history: int = 10
    c1: float = 1e-4
    shrink: float = 0.5
    max_backtracks: int = 30
    curvature_eps: float = 1e-10


@dataclasses.dataclass
class LbfgsState:
    x: np.ndarray
    L: float
    g: np.ndarray
    hist: list = dataclasses.field(default_factory=list)   # [(s, y, rho)], oldest first
    flags: int = 0
    last_alpha: float = 0.0
    trials: int = 0


def two_loop(g, hist):
    """L-BFGS two-loop recursion (Nocedal & Wright, Algorithm 7.4).

    hist holds (s, y, rho) oldest first; H0 = gamma I with
    gamma = s_new^T y_new / y_new^T y_new.  Returns r ~= H g.
    """
    q = g.copy()
    alphas = []
    for s, y, rho in reversed(hist):
        a = rho * float(np.vdot(s, q))
        q -= a * y
        alphas.append(a)
    s_n, y_n, _ = hist[-1]
    r = (float(np.vdot(s_n, y_n)) / float(np.vdot(y_n, y_n))) * q
    for (s, y, rho), a in zip(hist, reversed(alphas)):
        b = rho * float(np.vdot(y, r))
        r += (a - b) * s
    return r


def lbfgs_iteration(f: Callable, fg: Callable, st: LbfgsState, opt: LbfgsOptions):
    """One L-BFGS iteration: direction, backtracking Armijo search, history update.

    [gist] "Optimization Strategy": the keys are optimised by L-BFGS.  The
    pages fix no constants; reading taken (textbook defaults): history 10,
    gamma-scaled initial matrix, step 1 (or 1/max(1, ||g||) with an empty
    history), Armijo constant c1 = 1e-4, halving, at most 30 trials, a pair is
    kept only if s^T y > 1e-10 ||s|| ||y||, and a non-descent direction or a
    failed search clears the history.
    """
    g = st.g
    if st.hist:
        p = -two_loop(g, st.hist)
        a0 = 1.0
    else:
        p = -g
        a0 = 1.0 / max(1.0, float(np.linalg.norm(g)))
    gtp = float(np.vdot(g, p))
    if not gtp < 0.0:
        if st.hist:
            st.flags |= FLAG_NONDESCENT
        st.hist.clear()
        p = -g
        a0 = 1.0 / max(1.0, float(np.linalg.norm(g)))
        gtp = float(np.vdot(g, p))
    alpha = a0
    accepted = False
    trials = 0
    for _ in range(opt.max_backtracks):
        trials += 1
        xt = st.x + alpha * p
        Lt = f(xt)
        if Lt <= st.L + opt.c1 * alpha * gtp:
            accepted = True
            break
        alpha *= opt.shrink
    st.trials = trials
    if not accepted:
        st.hist.clear()
        st.flags |= FLAG_LINESEARCH
        st.last_alpha = 0.0
        return False
    Lt, gt = fg(xt)
    s = xt - st.x
    y = gt - g
    sy = float(np.vdot(s, y))
    if sy > opt.curvature_eps * float(np.linalg.norm(s)) * float(np.linalg.norm(y)):
        st.hist.append((s, y, 1.0 / sy))
        if len(st.hist) > opt.history:
            st.hist.pop(0)
    st.x, st.L, st.g = xt, Lt, gt
    st.last_alpha = alpha
    if not (np.isfinite(Lt) and np.all(np.isfinite(gt))):
        st.flags |= FLAG_NONFINITE
    return True


def lbfgs_minimize(f, fg, x0, iters, opt: Optional[LbfgsOptions] = None):
    """Plain L-BFGS over ``iters`` iterations (used by the optimizer pins)."""
    opt = opt or LbfgsOptions()
    L0, g0 = fg(x0)
    st = LbfgsState(x=_f64(x0).copy(), L=L0, g=g0)
    for _ in range(iters):
        lbfgs_iteration(f, fg, st, opt)
    return st


# --------------------------------------------------------------------------
# the alternating schedule and the pilot
# --------------------------------------------------------------------------

@dataclasses.dataclass
class CompressOptions:
    iters: int = 20
    vc_every: int = 5
    lam: float = 1.0
    ridge_rel: float = 1e-3
    lbfgs: LbfgsOptions = dataclasses.field(default_factory=LbfgsOptions)
    # sensitivity variant: round the keys to float32 at the start and after
    # every iteration (the loss and gradient are then taken at the rounded
    # keys).  Not part of the method; it measures how far the schedule's
    # result moves under perturbations of float32 size.
    keys_f32: bool = False


def compress_problem(Q, Kz, Vz, k, scale, opt: CompressOptions, Y=None, lse=None,
                     init=None, record=False, init_keys=False):
    """KVSculpt on one (layer, KV-head) problem.

    [abs] keys by L-BFGS, values in closed form, alternating every few steps;
    [gist] "Optimization Strategy".  Reading: one iteration is one L-BFGS
    iteration on Kc with Vc fixed; after iterations vc_every, 2*vc_every, ...
    Vc is re-solved and the loss and gradient are recomputed at the same Kc,
    keeping the L-BFGS history.  Flags: FLAG_NONFINITE whenever the loss or
    gradient at the current keys is not finite (at the start, after an
    accepted step, after a value re-solve); such a problem then fails every
    search and does not move.  ``init``: None = Select+Fit; a (Kc, Vc)
    pair; or, with ``init_keys``, starting keys Kc whose values are the ridge
    fit (a failed fit starts from zero values and sets FLAG_CHOLESKY).
    """
    if Y is None:
        Y, lse = reference_attention(Q, Kz, Vz, scale)
    if init is None:
        idx, Kc, Vc, ok = init_select_fit(Q, Kz, Y, lse, k, scale, opt.ridge_rel)
    elif init_keys:
        idx, Kc = None, _f64(init)
        Vc, _, ok = ridge_values(Q, Y, Kc, scale, opt.ridge_rel)
        if not ok:
            Vc = np.zeros_like(Kc)
    else:
        idx, (Kc, Vc), ok = None, init, True
    flags = 0 if ok else FLAG_CHOLESKY
    Kc = _f64(Kc).copy()
    if opt.keys_f32:
        Kc = Kc.astype(np.float32).astype(np.float64)
    Vc = _f64(Vc).copy() if Vc is not None else np.zeros_like(Kc)

    def make_f(Vc_):
        return (lambda x: loss(Q, Y, lse, x, Vc_, scale, opt.lam),
                lambda x: loss_grad(Q, Y, lse, x, Vc_, scale, opt.lam)[:2])

    def finite(L, g):
        return bool(np.isfinite(L) and np.all(np.isfinite(g)))

    f, fg = make_f(Vc)
    L0, g0 = fg(Kc)
    st = LbfgsState(x=Kc, L=L0, g=g0, flags=flags)
    if not finite(L0, g0):
        st.flags |= FLAG_NONFINITE
    traj = [L0]
    for t in range(1, opt.iters + 1):
        lbfgs_iteration(f, fg, st, opt.lbfgs)
        if opt.keys_f32:
            xr = st.x.astype(np.float32).astype(np.float64)
            if not np.array_equal(xr, st.x):
                st.x = xr
                st.L, st.g = fg(st.x)
        if t % opt.vc_every == 0:
            Vn, _, ok = ridge_values(Q, Y, st.x, scale, opt.ridge_rel)
            if ok:
                Vc = Vn
            else:
                st.flags |= FLAG_CHOLESKY
            f, fg = make_f(Vc)
            st.L, st.g = fg(st.x)
            if not finite(st.L, st.g):
                st.flags |= FLAG_NONFINITE
        if record:
            traj.append(st.L)
    mse = output_mse(Q, Y, lse, st.x, Vc, scale)
    return dict(Kc=st.x, Vc=Vc, loss=st.L, init_loss=L0, flags=st.flags, idx=idx,
                mse=mse, traj=traj, Y=Y, lse=lse)


def allocate_budget(mse: Sequence[float], K_total: int, alpha: float = 0.5,
                    k_min: int = 1, k_max: int = 1 << 30) -> List[int]:
    """Split K_total compressed pairs over problems in proportion to MSE**alpha.

    [gist] "Adaptive Budget Allocation": the total budget is redistributed in
    proportion to the square root of the pilot MSE, at layer and KV-head
    granularity.  Reading: one flat pool over all problems; weights
    w = sqrt(mse) (alpha = 0.5, correctly rounded sqrt; other alpha via pow);
    bounded water-filling x_p = clamp(t w_p, k_min, k_max) with sum K_total,
    found by fixing, each round, the violators that the clamped total proves
    final;
    floors plus largest remainders, ties to the lower problem index.  All
    arithmetic is IEEE double with sums in problem order, so any
    implementation doing the same operations agrees bit for bit.
    """
    P = len(mse)
    if P == 0:
        return []
    if K_total < P * k_min or K_total > P * k_max:
        raise ValueError("infeasible budget")
    w = []
    for v in mse:
        v = float(v)
        if not (v >= 0.0) or math.isinf(v):
            raise ValueError("mse must be finite and >= 0")
        w.append(math.sqrt(v) if alpha == 0.5 else (v if alpha == 1.0 else math.pow(v, alpha)))
    total = 0.0
    for x in w:
        total += x
    if total == 0.0:
        w = [1.0] * P
    fixed = [None] * P
    x = [0.0] * P
    while True:
        R = float(K_total)
        for p in range(P):
            if fixed[p] is not None:
                R -= float(fixed[p])
        S = 0.0
        for p in range(P):
            if fixed[p] is None:
                S += w[p]
        free = [p for p in range(P) if fixed[p] is None]
        if not free:
            break
        for p in free:
            x[p] = (R * w[p]) / S if S > 0.0 else R / len(free)
        hi = [p for p in free if x[p] > k_max]
        lo = [p for p in free if x[p] < k_min]
        if not hi and not lo:
            break
        # The clamped total says on which side the final multiplier lies:
        # over budget -> it is smaller, so today's lower violators stay at the
        # lower bound; under budget -> today's upper violators stay at the top.
        C = 0.0
        for p in free:
            C += float(k_max) if x[p] > k_max else (float(k_min) if x[p] < k_min else x[p])
        if C > R:
            fix = [(p, k_min) for p in lo]
        elif C < R:
            fix = [(p, k_max) for p in hi]
        else:
            fix = [(p, k_max) for p in hi] + [(p, k_min) for p in lo]
        for p, v in fix:
            fixed[p] = v
    k = [0] * P
    frac = []
    used = 0
    for p in range(P):
        if fixed[p] is not None:
            k[p] = int(fixed[p])
        else:
            fl = math.floor(x[p])
            k[p] = int(fl)
            frac.append((-(x[p] - fl), p))
        used += k[p]
    left = K_total - used
    frac.sort()
    for _, p in frac:
        if left <= 0:
            break
        if k[p] < k_max:
            k[p] += 1
            left -= 1
    return k


def allocate_budget_two_level(mse: Sequence[float], layers: int, heads: int, K_total: int,
                              alpha: float = 0.5, k_min: int = 1, k_max: int = 1 << 30) -> List[int]:
    """Two-level split: layers first, then the heads of each layer.

    [gist] "Adaptive Budget Allocation": allocation is done at both the layer
    and the KV-head level.  Reading: problem p = layer * heads + head; a
    layer's signal is the mean of its heads' MSE (the MSE of the layer's
    concatenated head outputs), summed in head order and divided by
    ``heads``; the layer budgets split K_total by :func:`allocate_budget`
    with bounds [heads * k_min, min(heads * k_max, K_total)]; each layer's
    budget is then split over its heads by :func:`allocate_budget` on the
    heads' own MSE.  Same exponent alpha at both levels.
    """
    if layers < 1 or heads < 1 or len(mse) != layers * heads:
        raise ValueError("mse must hold layers * heads entries")
    lmse = []
    for l in range(layers):
        acc = 0.0
        for h in range(heads):
            acc += float(mse[l * heads + h])
        lmse.append(acc / heads)
    lmax = min(heads * k_max, K_total)
    if lmax > (1 << 31) - 1:
        raise ValueError("per-layer bound too large")
    kl = allocate_budget(lmse, K_total, alpha, heads * k_min, lmax)
    out = []
    for l in range(layers):
        out += allocate_budget(mse[l * heads:(l + 1) * heads], kl[l], alpha, k_min, k_max)
    return out


def value_norm_signal(Vz):
    """Static allocation signal: the mean Euclidean norm of the compress
    zone's value rows.  [gist] "Adaptive Budget Allocation" compares the
    pilot MSE against static per-head signals, value norms among them;
    reading: this per-problem mean, used as the allocation weight in place of
    the pilot MSE."""
    V = _f64(Vz)
    return float(np.mean(np.sqrt(np.sum(V * V, axis=1))))


def pilot_allocate(problems, k0, scale, opt: CompressOptions, pilot_iters=60,
                   alpha=0.5, k_min=1, k_max=None):
    """Pilot run at uniform k0, then per-head budgets.

    [gist] "Adaptive Budget Allocation": a short compression run (60 steps)
    at uniform allocation gives a per-component MSE, and the total budget is
    redistributed in proportion to MSE^0.5.  ``problems`` is a list of
    (Q, Kz, Vz) per problem.  Returns (mse list, k list, pilot results).
    """
    popt = dataclasses.replace(opt, iters=pilot_iters)
    res, mse = [], []
    for (Q, Kz, Vz) in problems:
        r = compress_problem(Q, Kz, Vz, k0, scale, popt)
        res.append(r)
        mse.append(r["mse"])
    Z = problems[0][1].shape[0]
    kmax = Z if k_max is None else k_max
    ks = allocate_budget(mse, k0 * len(problems), alpha, k_min, kmax)
    return mse, ks, res


# --------------------------------------------------------------------------
# training-query construction
# --------------------------------------------------------------------------

def rotary(x, pos, theta):
    """Rotary position embedding of the rows of ``x`` at integer positions ``pos``.

    [gist] "Training Query Construction" speaks of RoPE'd queries without
    fixing the convention.  Reading: the half-split pairing of the Llama /
    Qwen families -- channel c and channel c + d/2 (c < d/2) form a plane,
    turned counter-clockwise by pos * theta**(-2c/d), positions 0-based.
    ``x`` is [..., d]; ``pos`` broadcasts against x's leading axes.
    """
    x = _f64(x)
    d = x.shape[-1]
    h = d // 2
    freq = np.power(float(theta), -2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)))
    out[..., :h] = a * cos - b * sin
    out[..., h:] = a * sin + b * cos
    return out


def de_rotary(x, pos, theta):
    """Remove the rotary embedding applied at ``pos`` (the De-RoPE step)."""
    return rotary(x, -np.asarray(pos, dtype=np.float64), theta)


def training_queries(Qctx, src, m, theta):
    """Training queries of one KV head from its query heads' context queries.

    [gist] "Training Query Construction": the real queries of the recent
    context, plus synthetic future queries whose content is taken from the
    context by undoing RoPE and which are embedded again at future positions,
    the sources drawn uniformly over the context.  Readings:
      * ``Qctx`` [g][N][d] holds the RoPE'd queries of the g query heads that
        share the KV head, at context positions 0..N-1;
      * retain queries are the rows at the retain-zone positions N-m..N-1
        ([gist] "Problem Formulation": the most recent m pairs);
      * ``src`` [g][F] holds the uniformly drawn source positions (the draw is
        an input); synthetic query j of head h is the row at src[h][j] with its
        rotation at src[h][j] removed, rotated again at position N + j;
      * rows are ordered: retain block (head 0's m rows, head 1's, ...), then
        the future block (head 0's F rows, head 1's, ...).
    Returns Q [g(m+F)][d] in float64.
    """
    Qctx = _f64(Qctx)
    src = np.asarray(src, dtype=np.int64)
    g, N, d = Qctx.shape
    F = src.shape[1] if src.ndim == 2 else 0
    if src.size and (src.min() < 0 or src.max() >= N):
        raise ValueError("source positions must lie in [0, N)")
    retain = [Qctx[h, N - m:N] for h in range(g)]
    future = []
    for h in range(g):
        content = de_rotary(Qctx[h, src[h]], src[h], theta)     # De-RoPE at the source
        future.append(rotary(content, N + np.arange(F), theta))  # future positions
    rows = retain + future
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, d))


# --------------------------------------------------------------------------
# use-side evaluation
# --------------------------------------------------------------------------

def use_side_outputs(Qh, Kz, Vz, Kr, Vr, Kc, Vc, scale):
    """Attention outputs at use time over the full and the compressed cache.

    [gist] "Problem Formulation": the compressed cache (k free pairs in place
    of the compress zone, retain zone unchanged) should give the full cache's
    attention output for future queries; "Loss Function": the LSE term keeps
    the chunk's attention mass right when it is combined with the other
    tokens.  Reading: a use-time query attends over [Kz; Kr] (full cache) or
    [Kc; Kr] (compressed cache) in one softmax -- the plain definition, no
    chunk merging -- with scores scale * q.k and no mask (every held-out
    query comes after the whole context).  ``Kr`` may have zero rows.
    Returns dict(full [nh, d], comp [nh, d], mse, rel) with
    mse = ||comp - full||_F^2 / (nh d) and rel = ||comp - full||_F / ||full||_F.
    """
    Qh = _f64(Qh)
    d = Qh.shape[1]
    Kr = _f64(Kr).reshape(-1, d)
    Vr = _f64(Vr).reshape(-1, d)

    def attend(K, V):
        W, _ = softmax_rows(logits(Qh, K, scale))
        return W @ V

    full = attend(np.concatenate([_f64(Kz), Kr]), np.concatenate([_f64(Vz), Vr]))
    comp = attend(np.concatenate([_f64(Kc), Kr]), np.concatenate([_f64(Vc), Vr]))
    D = comp - full
    sq = float(np.sum(D * D))
    nf = float(np.sqrt(np.sum(full * full)))
    return dict(full=full, comp=comp, mse=sq / D.size, rel=math.sqrt(sq) / nf if nf > 0 else 0.0)


# --------------------------------------------------------------------------
# optimizer ablations
# --------------------------------------------------------------------------

def restart_search(Q, Kz, Vz, k, scale, opt: CompressOptions, key_sets):
    """The best of several runs of the schedule from different starting keys.

    [gist] section 4 "Optimizer Efficacy" compares a single L-BFGS run with
    an oracle search over 100 random restarts.  Reading: a restart starts
    from k keys of the compress zone taken at uniformly drawn distinct
    positions (``key_sets``: one [k, d] array per restart, the draw is an
    input), with ridge-fitted values, and runs the same schedule; the search
    keeps the lowest final loss.  Returns (best index, list of run results).
    """
    Y, lse = reference_attention(Q, Kz, Vz, scale)
    runs = [compress_problem(Q, Kz, Vz, k, scale, opt, Y=Y, lse=lse, init=K0, init_keys=True)
            for K0 in key_sets]
    best = int(np.argmin([r["loss"] for r in runs]))
    return best, runs


@dataclasses.dataclass
class AdamOptions:
    lr: float = 1e-2
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8


def adam_step(x, g, m, v, t, a: AdamOptions):
    """One Adam update at step t >= 1 (Kingma & Ba, "Adam: A Method for
    Stochastic Optimization", 2015, Algorithm 1): first and second moment
    averages, their bias corrections, and the step lr * mhat / (sqrt(vhat) + eps).
    Returns (x, m, v)."""
    m = a.beta1 * m + (1.0 - a.beta1) * g
    v = a.beta2 * v + (1.0 - a.beta2) * (g * g)
    mhat = m / (1.0 - a.beta1 ** t)
    vhat = v / (1.0 - a.beta2 ** t)
    return x - a.lr * mhat / (np.sqrt(vhat) + a.eps), m, v


def compress_problem_adam(Q, Kz, Vz, k, scale, opt: CompressOptions, adam: AdamOptions,
                          Y=None, lse=None, init=None, init_keys=False):
    """The alternating schedule with Adam in place of L-BFGS on the keys.

    [gist] section 4 "Optimizer Efficacy": replacing L-BFGS by Adam raises the
    per-layer MSE 17-95x; section 2 "Optimization Strategy" says first-order
    methods get trapped.  Reading: the same start (Select+Fit, or ``init`` as
    in :func:`compress_problem`), the same value re-solves after iterations
    vc_every, 2*vc_every, ..., one Adam step on Kc per iteration at the
    gradient of the current (Kc, Vc), moments kept across value solves.  The
    pages give no Adam constants: Kingma & Ba's defaults, step size lr
    (parameter, 1e-2 here).
    """
    if Y is None:
        Y, lse = reference_attention(Q, Kz, Vz, scale)
    flags = 0
    if init is None:
        idx, Kc, Vc, ok = init_select_fit(Q, Kz, Y, lse, k, scale, opt.ridge_rel)
        if not ok:
            flags |= FLAG_CHOLESKY
    elif init_keys:
        idx, Kc = None, _f64(init)
        Vc, _, ok = ridge_values(Q, Y, Kc, scale, opt.ridge_rel)
        if not ok:
            Vc, flags = np.zeros_like(Kc), flags | FLAG_CHOLESKY
    else:
        idx, (Kc, Vc) = None, init
    x = _f64(Kc).copy()
    Vc = _f64(Vc).copy()
    m = np.zeros_like(x)
    v = np.zeros_like(x)
    L0 = loss(Q, Y, lse, x, Vc, scale, opt.lam)
    for t in range(1, opt.iters + 1):
        _, g = loss_grad(Q, Y, lse, x, Vc, scale, opt.lam)[:2]
        if not np.all(np.isfinite(g)):
            flags |= FLAG_NONFINITE
            break
        x, m, v = adam_step(x, g, m, v, t, adam)
        if t % opt.vc_every == 0:
            Vn, _, ok = ridge_values(Q, Y, x, scale, opt.ridge_rel)
            if ok:
                Vc = Vn
            else:
                flags |= FLAG_CHOLESKY
    L = loss(Q, Y, lse, x, Vc, scale, opt.lam)
    return dict(Kc=x, Vc=Vc, loss=L, init_loss=L0, flags=flags, idx=idx,
                mse=output_mse(Q, Y, lse, x, Vc, scale), Y=Y, lse=lse)
