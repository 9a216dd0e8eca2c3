"""GPU parity of the optimizer ablations through the C ABI.

- kvs_compress_adam: the keys after one Adam step within 1e-5 (relative to
  1 + |Kc|) of the oracle's step from the same start.  Elements whose float64
  gradient is below 1e-4 of the largest are skipped: there the sign of a
  near-zero gradient decides the direction of a full lr step.  Final loss after the whole schedule
  within 2% of the oracle's (the same bar as kvs_compress); the loss at the
  start within 1e-4.
- kvs_compress_from_keys: started from the Select+Fit keys it reproduces
  kvs_compress bit for bit.  Started from random key draws (batched restarts,
  one problem per restart) each final loss is within 2% of the oracle's run
  from the same draw.
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch, tiny_workload
from tests.gpu_common import empty, host, pack, say, to_gpu, workspace

pytestmark = pytest.mark.gpu


def _alloc(bt, o, ktot, d, P):
    ws = workspace(K.workspace_bytes(bt, o))
    return ws, empty((ktot, d)), empty((P,)), empty((P,)), empty((P,)), to_gpu(np.zeros(P, np.int32))


def _adam_gpu(b, k, o, a, Kc0=None):
    P, n, d = b["Q"].shape
    bt = K.Batch(P, d, b["Kz"].shape[1], n, k=[k] * P, scale=b["scale"])
    ws, Vc, loss, mse, l0, flags = _alloc(bt, o, k * P, d, P)
    Kc = to_gpu(Kc0) if Kc0 is not None else empty((k * P, d))
    K.kvs_compress_adam(K.Context(), bt, o, a, Kc0 is not None, to_gpu(b["Q"]), to_gpu(b["Kz"]),
                        to_gpu(b["Vz"]), Kc, Vc, loss, mse, l0, flags, ws)
    return host(Kc), host(Vc), host(loss), host(l0), host(flags)


def test_adam_first_step_matches_oracle():
    w = WORKLOADS[1]
    b = make_batch(w, 0)
    a = K.adam_opts(lr=1e-2)
    o = K.opts(iters=1, vc_every=100)
    say(f"[adam] one step, {w.name} P={b['Q'].shape[0]} k={w.k0}")
    Kc, _, _, _, flags = _adam_gpu(b, w.k0, o, a)
    assert not flags.any()
    Kcs = np.split(Kc, b["Q"].shape[0])
    for p in range(b["Q"].shape[0]):
        Q, Kz, Vz, s = b["Q"][p], b["Kz"][p], b["Vz"][p], b["scale"]
        Y, lse = O.reference_attention(Q, Kz, Vz, s)
        _, K0, V0, ok = O.init_select_fit(Q, Kz, Y, lse, w.k0, s)
        g = O.loss_grad(Q, Y, lse, K0, V0, s)[1]
        x1, _, _ = O.adam_step(K0, g, np.zeros_like(g), np.zeros_like(g), 1,
                               O.AdamOptions(lr=1e-2))
        sel = np.abs(g) > 1e-4 * np.abs(g).max()
        err = (np.abs(Kcs[p] - x1) / (1.0 + np.abs(x1)))[sel].max()
        say(f"   p={p} checked {sel.mean():.3f} of the elements, max |dKc|/(1+|Kc|) {err:.2e}")
        assert err <= 1e-5


ADAM_CASES = {
    "single-head-d64": (WORKLOADS[0], 20),
    "qwen-one-layer-40it": (WORKLOADS[1], 40),
}


@pytest.mark.parametrize("name", list(ADAM_CASES))
def test_adam_schedule_final_loss(name):
    w, T = ADAM_CASES[name]
    b = make_batch(w, 0)
    P = b["Q"].shape[0]
    o = K.opts(iters=T)
    say(f"[adam] schedule {name} P={P} k={w.k0} T={T}")
    _, _, loss, l0, flags = _adam_gpu(b, w.k0, o, K.adam_opts())
    assert not flags.any()
    for p in range(P):
        r = O.compress_problem_adam(b["Q"][p], b["Kz"][p], b["Vz"][p], w.k0, b["scale"],
                                    O.CompressOptions(iters=T), O.AdamOptions())
        lb = O.compress_problem(b["Q"][p], b["Kz"][p], b["Vz"][p], w.k0, b["scale"],
                                O.CompressOptions(iters=T))
        say(f"   p={p} init {l0[p]:.5g} / {r['init_loss']:.5g}; Adam final {loss[p]:.5g} / "
            f"{r['loss']:.5g}; L-BFGS final (oracle) {lb['loss']:.5g}")
        assert abs(l0[p] - r["init_loss"]) <= 1e-4 * r["init_loss"]
        assert abs(loss[p] - r["loss"]) <= 0.02 * r["loss"]


def test_compress_from_select_fit_keys_is_compress():
    w = WORKLOADS[1]
    b = make_batch(w, 1)
    P, n, d = b["Q"].shape
    o = K.opts(iters=12)
    bt = K.Batch(P, d, w.Z, n, k=[w.k0] * P, scale=b["scale"])
    say(f"[from-keys] Select+Fit keys vs kvs_compress, {w.name} T=12")
    ctx = K.Context()
    Q, Kz, Vz = to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"])
    ws, Vc, loss, mse, l0, flags = _alloc(bt, o, w.k0 * P, d, P)
    Kc = empty((w.k0 * P, d))
    K.kvs_compress(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)
    ref = [host(t).copy() for t in (Kc, Vc, loss, l0)]
    # the Select+Fit keys, gathered by the library itself
    Y, lse = empty((P, n, d)), empty((P, n))
    K.kvs_reference_attn(ctx, bt, Q, Kz, Vz, Y, lse, ws)
    idx = empty((w.k0 * P,), "i32")
    K.kvs_init_topk(ctx, bt, Q, Kz, Y, lse, idx, Kc, Vc, flags, ws)
    Kc0 = host(Kc).copy()
    Kc = to_gpu(Kc0)
    K.kvs_compress_from_keys(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)
    got = [host(t) for t in (Kc, Vc, loss, l0)]
    for name, x, y in zip(("Kc", "Vc", "loss", "init_loss"), got, ref):
        assert np.array_equal(x, y), name


def test_batched_random_restarts_match_oracle_runs():
    w = tiny_workload(d=64, N=200, m=16, g=2, F=40, k0=24)
    b = make_batch(w, 0)
    R = 4
    rng = np.random.default_rng(5)
    draws = [np.sort(rng.choice(w.Z, w.k0, replace=False)) for _ in range(R)]
    Q = np.repeat(b["Q"], R, axis=0)
    Kz = np.repeat(b["Kz"], R, axis=0)
    Vz = np.repeat(b["Vz"], R, axis=0)
    Kc0 = pack([w.k0] * R, [b["Kz"][0][ix] for ix in draws])
    P, n, d = Q.shape
    T = 15
    o = K.opts(iters=T)
    bt = K.Batch(P, d, w.Z, n, k=[w.k0] * P, scale=b["scale"])
    say(f"[restarts] {R} restarts of one problem as a batch, Z={w.Z} k={w.k0} T={T}")
    ws, Vc, loss, mse, l0, flags = _alloc(bt, o, w.k0 * P, d, P)
    Kc = to_gpu(Kc0)
    K.kvs_compress_from_keys(K.Context(), bt, o, to_gpu(Q), to_gpu(Kz), to_gpu(Vz), Kc, Vc, loss,
                             mse, l0, flags, ws)
    lg, l0g = host(loss), host(l0)
    best, runs = O.restart_search(b["Q"][0], b["Kz"][0], b["Vz"][0], w.k0, b["scale"],
                                  O.CompressOptions(iters=T), [b["Kz"][0][ix] for ix in draws])
    for r in range(R):
        say(f"   restart {r}: init {l0g[r]:.5g} / {runs[r]['init_loss']:.5g}, final {lg[r]:.5g} / "
            f"{runs[r]['loss']:.5g}")
        assert abs(l0g[r] - runs[r]["init_loss"]) <= 1e-4 * runs[r]["init_loss"]
        assert abs(lg[r] - runs[r]["loss"]) <= 0.02 * runs[r]["loss"]
    assert abs(lg.min() - runs[best]["loss"]) <= 0.02 * runs[best]["loss"]
