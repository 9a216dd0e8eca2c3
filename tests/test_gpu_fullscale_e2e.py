"""End-to-end GPU parity at the full sizes of the large workloads, against
oracle runs stored by tests/golden/make_golden.py (oracle only).

- kvs_pilot_allocate on the whole 56-problem full cache, 60 iterations,
  r = 0.3, 0.5 and 0.7, bounds [1, Z] (Z binds at 0.5 and 0.7):
  * the budgets equal the oracle allocator fed the GPU's pilot MSEs, bit for
    bit (the allocation contract: the same MSE vector in, the same k out);
  * the final pilot losses against the oracle's own 60-iteration pilot.
    The schedule is chaotic at float32 precision, so a head's final loss is
    not a unique result: two perturbations at the level of one float32
    rounding measure its spread, the oracle's run with its keys rounded to
    float32 after every iteration (2 to 4 of these 56 heads move by more
    than 2%, up to 4.4%) and the GPU run again with every query element
    moved by one ulp; a head's spread is the larger of the two.  The GPU's
    relative deviations from the float64 run must have a signed mean within
    0.5% (no systematic bias), and be no more than twice the spread in the
    bulk and the tail: median at most max(0.5%, twice the median spread), at
    most 2 n + 2 heads beyond 2% (n: heads whose spread is beyond 2%), the
    worst at most max(2%, twice the largest spread).  The pilot MSEs, one of the two
    terms the optimizer trades, are compared and reported;
  * against the oracle's own allocation (its own MSEs) each head's budget may
    move only as far as the MSE differences move its continuous share, plus
    the two units that rounding can add: |dk_p| < |dx_p| + 2, where x_p are
    the continuous bounded shares (computed here independently, by
    bisection on the multiplier).  The number of heads that differ and the
    smallest distance of a fractional part to the rounding cut are printed.
- kvs_compress with the bench's launch shapes (the whole batch at uniform
  k0: 256 llama3-8b problems, T = 200; 112 long-context problems, T = 150):
  problem 0's Select+Fit loss within 1e-4 of the oracle's, its final loss
  within 2% of the oracle's run of the same schedule, or within twice the
  problem's spread, whichever is larger; llama3-8b problem 0 also alone at
  k = 4680, the largest budget the pilot hands out on that cache.  For a
  single problem one perturbation samples its spread once, so here the
  GPU's part of the spread is the largest move under three one-rounding
  perturbations (the queries by one ulp in either alternating pattern, the
  compress-zone keys in one), beside the oracle's float32-key run.
- kvs_compress on the whole llama3-8b batch at seeded ragged budgets (the main
  run after a reallocation), eight seeded problems against the oracle, each
  to the single-problem bar.
"""
import json
import math
import os

import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch
from tests.gpu_common import empty, host, say, to_gpu, workspace

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def band_err(x, a, b):
    """Relative distance of x to the interval [min(a, b), max(a, b)]."""
    lo, hi = min(a, b), max(a, b)
    return 0.0 if lo <= x <= hi else (lo - x) / lo if x < lo else (x - hi) / hi


def ulp_perturbed(x, phase=0):
    """x with every element moved by one float32 ulp, up at even flat
    positions and down at odd ones (phase 1: the other way round): a
    perturbation at the level of one float32 rounding."""
    f = np.asarray(x, dtype=np.float32).ravel().copy()
    up = np.arange(f.size) % 2 == phase
    f[up] = np.nextafter(f[up], np.float32(np.inf))
    f[~up] = np.nextafter(f[~up], np.float32(-np.inf))
    return f.reshape(np.shape(x))


def _shares(mse, K_total, alpha, kmin, kmax):
    """Continuous bounded shares x_p = clamp(t w_p, kmin, kmax), sum K_total."""
    w = np.asarray(mse, dtype=np.float64) ** alpha
    if w.sum() == 0:
        w = np.ones_like(w)
    lo, hi = 0.0, 1.0
    while np.clip(hi * w, kmin, kmax).sum() < K_total:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.clip(mid * w, kmin, kmax).sum() < K_total:
            lo = mid
        else:
            hi = mid
    return np.clip(hi * w, kmin, kmax)


@pytest.mark.parametrize("ratio", [0.3, 0.5, 0.7])
def test_pilot_full_cache(ratio):
    gold = json.load(open(os.path.join(GOLD, "oracle_pilot_qwen2.5-1.5b-full-cache.json")))
    g = gold["ratios"][str(ratio)]
    w = WORKLOADS[2].with_ratio(ratio)
    assert g["k0"] == w.k0
    b = make_batch(w, gold["seed"], workers=8)
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    pilot = gold["pilot_iters"]
    o = K.opts(iters=pilot)
    bt = K.Batch(P, d, Z, n, k=[w.k0] * P, scale=b["scale"])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt, o))
    pm = empty((P,))
    Qg, Kzg, Vzg = to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"])
    say(f"[pilot full cache] r={ratio} P={P} k0={w.k0} Z={Z} pilot={pilot}")
    k_out = np.asarray(K.kvs_pilot_allocate(ctx, bt, o, pilot, 0.5, 1, Z, Qg, Kzg, Vzg, pm, ws))
    mg = host(pm).astype(np.float64)
    # the same pilot run through kvs_compress, for its final losses
    Kc, Vc = empty((w.k0 * P, d)), empty((w.k0 * P, d))
    loss, mse2, l0 = empty((P,)), empty((P,)), empty((P,))
    fl = to_gpu(np.zeros(P, np.int32))
    K.kvs_compress(ctx, bt, o, Qg, Kzg, Vzg, Kc, Vc, loss, mse2, l0, fl, ws)
    lg = host(loss).astype(np.float64)
    assert host(mse2).astype(np.float64).tobytes() == mg.tobytes()
    # and with the queries moved by one ulp, for the spread
    K.kvs_compress(ctx, bt, o, to_gpu(ulp_perturbed(b["Q"])), Kzg, Vzg, Kc, Vc, loss, mse2, l0, fl, ws)
    lu = host(loss).astype(np.float64)
    mo = np.asarray(g["mse"], dtype=np.float64)
    lo = np.asarray(g["loss"], dtype=np.float64)
    l32 = np.asarray(g["loss_f32keys"], dtype=np.float64)
    Kt = w.k0 * P
    assert k_out.tolist() == O.allocate_budget(list(mg), Kt, 0.5, 1, Z)
    err = np.abs(mg - mo) / mo
    lerr = np.abs(lg - lo) / lo
    bias = float(np.mean((lg - lo) / lo))
    berr = np.array([band_err(lg[p], lo[p], l32[p]) for p in range(P)])
    oerr = np.abs(l32 - lo) / lo
    uerr = np.abs(lu - lg) / lg
    spread = np.maximum(oerr, uerr)
    nsp, ngpu = int(np.sum(spread > 0.02)), int(np.sum(lerr > 0.02))
    say(f"   pilot loss: rel diff to the float64 oracle median {np.median(lerr):.2e} max {lerr.max():.2e} "
        f"signed mean {bias:.2e} ({ngpu} heads > 2%); outside the float64 / float32-key interval: "
        f"{int(np.sum(berr > 0))} heads, max {berr.max():.2e}; spread under the oracle's float32 keys median "
        f"{np.median(oerr):.2e} max {oerr.max():.2e}, under the GPU's one-ulp queries median {np.median(uerr):.2e} "
        f"max {uerr.max():.2e} ({nsp} heads > 2% under either); pilot MSE: worst {err.max():.2e} "
        f"(median {np.median(err):.2e}); flags {int(np.count_nonzero(host(fl)))}")
    ko = np.asarray(g["k"])
    xg, xo = _shares(mg, Kt, 0.5, 1, Z), _shares(mo, Kt, 0.5, 1, Z)
    dk, dx = np.abs(k_out - ko), np.abs(xg - xo)
    frac = xo - np.floor(xo)
    free = (xo > 1) & (xo < Z)
    cut = np.sort(frac[free])[::-1]
    left = Kt - int(np.floor(xo).sum())
    margin = float(cut[left - 1] - cut[left]) if 0 < left < len(cut) else float("nan")
    say(f"   k: {int(np.count_nonzero(dk))} of {P} heads differ from the oracle's own allocation, "
        f"max |dk| {int(dk.max())}, max |dx| {dx.max():.3f}; k at Z: {int(np.sum(k_out == Z))}; "
        f"fractional-part gap at the rounding cut {margin:.2e}")
    assert np.median(lerr) <= max(0.005, 2.0 * np.median(spread)) and abs(bias) <= 0.005
    assert ngpu <= 2 * nsp + 2 and lerr.max() <= max(0.02, 2.0 * spread.max())
    assert np.all(dk < dx + 2)
    assert int(k_out.sum()) == Kt and k_out.min() >= 1 and k_out.max() <= Z


def _compress(b, ks, T, Q=None, Kz=None):
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    o = K.opts(iters=T)
    bt = K.Batch(P, d, Z, n, k=ks, scale=b["scale"])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt, o))
    kt = int(sum(ks))
    Kc, Vc = empty((kt, d)), empty((kt, d))
    loss, mse, l0 = empty((P,)), empty((P,)), empty((P,))
    flags = to_gpu(np.zeros(P, np.int32))
    K.kvs_compress(ctx, bt, o, to_gpu(b["Q"] if Q is None else Q), to_gpu(b["Kz"] if Kz is None else Kz),
                   to_gpu(b["Vz"]), Kc, Vc, loss, mse, l0, flags, ws)
    return host(loss).astype(np.float64), host(l0).astype(np.float64), host(flags)


def _gpu_spread(b, ks, T, lg):
    """Per problem, the largest relative move of the GPU's final loss under
    three one-rounding perturbations of its inputs (the queries moved by one
    ulp in either alternating pattern, the compress-zone keys in one): one
    perturbation samples a chaotic head's spread once, three bound it more
    tightly.  Returns (spread, losses of the first perturbation)."""
    runs = [_compress(b, ks, T, Q=ulp_perturbed(b["Q"]))[0],
            _compress(b, ks, T, Q=ulp_perturbed(b["Q"], 1))[0],
            _compress(b, ks, T, Kz=ulp_perturbed(b["Kz"]))[0]]
    return np.max([np.abs(r - lg) / lg for r in runs], axis=0), runs[0]


E2E = {
    "llama3-8b-batch-k2381": ("llama3-8b-cache", 3, 2381, "batch"),
    "llama3-8b-alone-k4680": ("llama3-8b-cache", 3, 4680, "alone"),
    "qwen2.5-7b-long-batch-k3226": ("qwen2.5-7b-long-context", 4, 3226, "batch"),
}


@pytest.mark.parametrize("name", list(E2E))
def test_compress_full_schedule(name):
    wname, cid, k, how = E2E[name]
    gold = json.load(open(os.path.join(GOLD, f"oracle_compress_{wname}_p0.json")))
    run = next(r for r in gold["runs"] if r["k"] == k)
    w = WORKLOADS[cid]
    T = gold["iters"]
    b = make_batch(w, gold["seed"], problems=None if how == "batch" else [0], workers=16)
    P = b["Q"].shape[0]
    say(f"[full schedule] {name}: P={P} k={k} T={T}")
    lg, l0g, fg = _compress(b, [k] * P, T)
    ub, lu = _gpu_spread(b, [k] * P, T, lg)
    lo, l32 = run["final_loss"], run["final_loss_f32keys"]
    dev = abs(lg[0] - lo) / lo
    spread = max(abs(l32 - lo) / lo, ub[0])
    be = band_err(lg[0], lo, l32)
    say(f"   p=0 init gpu={l0g[0]:.7g} oracle={run['init_loss']:.7g}; final gpu={lg[0]:.7g} "
        f"oracle={lo:.7g} (float32 keys {l32:.7g}; gpu with one-ulp queries {lu[0]:.7g}; GPU spread over three "
        f"one-rounding perturbations {ub[0]:.2e}) deviation {dev:.2e}, spread {spread:.2e}, distance to the "
        f"float64 / float32-key interval {be:.2e}; flags={fg[0]}; batch final/init median "
        f"{np.median(lg / l0g):.4f}, GPU spread over the batch median {np.median(ub):.2e} max {ub.max():.2e}, "
        f"flagged {int(np.count_nonzero(fg))}")
    assert abs(l0g[0] - run["init_loss"]) <= 1e-4 * run["init_loss"]
    assert dev <= max(0.02, 2.0 * spread)
    assert fg[0] & ~K.KVS_FLAG_NONDESCENT == 0 and run["flags"] & ~O.FLAG_NONDESCENT == 0
    assert np.all(np.isfinite(lg))


def test_compress_ragged_batch():
    """kvs_compress on the whole llama3-8b-shaped batch (256 problems) at
    seeded ragged budgets (log-uniform in [700, 4680], the spread a
    reallocation produces there), T = 200; eight seeded problems against the
    oracle's runs of the same schedule: Select+Fit loss within 1e-4, final
    loss within max(2%, twice the problem's spread), the spread measured as
    for the single-problem runs (the oracle with float32 keys, the GPU with
    one-ulp queries)."""
    gold = json.load(open(os.path.join(GOLD, "oracle_compress_llama3-8b-cache_ragged.json")))
    w = WORKLOADS[3]
    ks, T = gold["k"], gold["iters"]
    b = make_batch(w, gold["seed"], workers=16)
    P = b["Q"].shape[0]
    assert len(ks) == P
    say(f"[ragged batch] {w.name}: P={P} k {min(ks)}..{max(ks)} (sum {sum(ks)}) T={T}")
    lg, l0g, fg = _compress(b, ks, T)
    ub, lu = _gpu_spread(b, ks, T, lg)
    devs, bad = [], []
    for run in gold["runs"]:
        p = run["p"]
        lo, l32 = run["final_loss"], run["final_loss_f32keys"]
        dev = abs(lg[p] - lo) / lo
        spread = max(abs(l32 - lo) / lo, ub[p])
        devs.append(dev)
        say(f"   p={p} k={ks[p]} init gpu={l0g[p]:.7g} oracle={run['init_loss']:.7g}; final gpu={lg[p]:.7g} "
            f"oracle={lo:.7g} (float32 keys {l32:.7g}; gpu with one-ulp queries {lu[p]:.7g}) deviation "
            f"{dev:.2e} spread {spread:.2e}; flags={fg[p]}")
        if not abs(l0g[p] - run["init_loss"]) <= 1e-4 * run["init_loss"]:
            bad.append((p, "init"))
        if not dev <= max(0.02, 2.0 * spread):
            bad.append((p, "final"))
        if not (fg[p] & ~K.KVS_FLAG_NONDESCENT == 0 and run["flags"] & ~O.FLAG_NONDESCENT == 0):
            bad.append((p, "flags"))
    say(f"   sampled deviations median {np.median(devs):.2e} max {max(devs):.2e}; batch final/init median "
        f"{np.median(lg / l0g):.4f}, GPU spread over the batch median {np.median(ub):.2e} max {ub.max():.2e}, "
        f"flagged {int(np.count_nonzero(fg))}")
    assert not bad, bad
    assert np.all(np.isfinite(lg))
