"""GPU parity: use-side evaluation through the C ABI.

Bar: both outputs within 1e-4 relative Frobenius error of the float64 oracle
on identical float32 inputs.  The error figures mse and rel are a difference
of two outputs, so their error is amplified by ||Ofull|| / ||Ocomp - Ofull||.
Each output carries ~1e-6 relative error (float32 scores and accumulation),
so mse is held to 1e-4 relative only where that ratio is below 20; the
cases here compress coarsely (ratio 2-10, printed).  The uncompressed case
k = Z, Kc = Kz is held to an absolute bound instead.
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_use_batch, tiny_workload
from tests.gpu_common import empty, host, pack, rel, row_err, say, to_gpu, workspace

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _subset(u, ks, seed):
    """Compressed caches for the test: k_p sorted random rows of the zone, values
    scaled by 1.1 (a coarse, lossy stand-in for an optimised cache)."""
    rng = np.random.default_rng(seed)
    Kc, Vc = [], []
    for p, k in enumerate(ks):
        idx = np.sort(rng.choice(u["Kz"].shape[1], size=k, replace=False))
        Kc.append(u["Kz"][p, idx])
        Vc.append(1.1 * u["Vz"][p, idx])
    return pack(ks, Kc).astype(np.float32), pack(ks, Vc).astype(np.float32)


def _run(u, ks, Kc, Vc, m, outputs=True):
    P, n, d = u["Qh"].shape
    Z = u["Kz"].shape[1]
    bt = K.Batch(P, d, Z, n, k=ks)
    ctx = K.Context()
    ws = workspace(K.use_eval_workspace_bytes(bt, m))
    Of = empty((P, n, d)) if outputs else None
    Oc = empty((P, n, d)) if outputs else None
    mse, rl = empty((P,)), empty((P,))
    Kr = to_gpu(u["Kr"]) if m else None
    Vr = to_gpu(u["Vr"]) if m else None
    K.kvs_use_eval(ctx, bt, m, to_gpu(u["Qh"]), to_gpu(u["Kz"]), to_gpu(u["Vz"]), Kr, Vr,
                   to_gpu(Kc), to_gpu(Vc), Of, Oc, mse, rl, ws)
    return (host(Of) if outputs else None, host(Oc) if outputs else None, host(mse), host(rl))


def _cases():
    t64 = tiny_workload(d=64, N=300, m=20, g=3, F=23, layers=3, kv_heads=1)
    return {
        "qwen-one-layer": (WORKLOADS[1], None, None, None),
        "ragged-d64": (t64, None, [5, 117, 280], None),
        "no-retain-d128": (tiny_workload(d=128, N=200, m=0, g=2, F=40, layers=1, kv_heads=2),
                           None, [33, 150], None),
        "long-context-1-problem": (WORKLOADS[4], [0], None, 64),
    }


@pytest.mark.parametrize("name", list(_cases()))
def test_use_eval_matches_oracle(name):
    w, probs, ks, per_head = _cases()[name]
    u = make_use_batch(w, 3, probs, per_head)
    P, n, d = u["Qh"].shape
    ks = [w.k0] * P if ks is None else ks
    say(f"[use-eval] case={name} P={P} n={n} Z={w.Z} m={w.m} d={d} k={ks}")
    Kc, Vc = _subset(u, ks, 7)
    Of, Oc, mse, rl = _run(u, ks, Kc, Vc, w.m)
    Kcs = np.split(Kc, np.cumsum(ks)[:-1])
    Vcs = np.split(Vc, np.cumsum(ks)[:-1])
    for p in range(P):
        r = O.use_side_outputs(u["Qh"][p], u["Kz"][p], u["Vz"][p], u["Kr"][p], u["Vr"][p],
                               Kcs[p], Vcs[p], u["scale"])
        ef, ec = row_err(Of[p], r["full"]), row_err(Oc[p], r["comp"])
        amp = 1.0 / max(r["rel"], 1e-30)
        em, er = abs(mse[p] - r["mse"]) / r["mse"], abs(rl[p] - r["rel"]) / r["rel"]
        say(f"   p={p} rowOf={ef:.2e} rowOc={ec:.2e} mse={r['mse']:.3e} rel={r['rel']:.3f} "
            f"(amplification {amp:.1f}) err mse={em:.2e} rel={er:.2e}")
        assert ef <= TOL and ec <= TOL
        assert amp < 20
        assert em <= TOL and er <= TOL


def test_uncompressed_cache_has_no_use_error_and_outputs_are_optional():
    w = WORKLOADS[1]
    u = make_use_batch(w, 4, None, 100)
    P, n, d = u["Qh"].shape
    ks = [w.Z] * P
    Kc = u["Kz"].reshape(-1, d).copy()
    Vc = u["Vz"].reshape(-1, d).copy()
    say(f"[use-eval] k = Z = {w.Z}, Kc = Kz: P={P} n={n}")
    Of, Oc, mse, rl = _run(u, ks, Kc, Vc, w.m)
    for p in range(P):
        ms = float(np.mean(Of[p].astype(np.float64) ** 2))
        say(f"   p={p} mse={mse[p]:.3e} (mean square output {ms:.3e}) rel={rl[p]:.2e}")
        assert mse[p] <= 1e-10 * ms and rl[p] <= 1e-5
    Kc2, Vc2 = _subset(u, [700, 900], 1)
    a = _run(u, [700, 900], Kc2, Vc2, w.m, outputs=True)
    b = _run(u, [700, 900], Kc2, Vc2, w.m, outputs=False)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])


def test_use_eval_single_query_single_pair():
    """n = 1 held-out query and k = 1 compressed pair per problem."""
    w = tiny_workload(d=64, N=50, m=6, g=1, F=1, layers=1, kv_heads=3)
    u = make_use_batch(w, 8, None, 1)
    P, n, d = u["Qh"].shape
    assert n == 1
    ks = [1] * P
    say(f"[use-eval] degenerate n=1, k=1, P={P}")
    Kc, Vc = _subset(u, ks, 3)
    Of, Oc, mse, rl = _run(u, ks, Kc, Vc, w.m)
    for p in range(P):
        r = O.use_side_outputs(u["Qh"][p], u["Kz"][p], u["Vz"][p], u["Kr"][p], u["Vr"][p],
                               Kc[p:p + 1], Vc[p:p + 1], u["scale"])
        assert row_err(Of[p], r["full"]) <= TOL and row_err(Oc[p], r["comp"]) <= TOL
        assert abs(mse[p] - r["mse"]) <= TOL * r["mse"]
