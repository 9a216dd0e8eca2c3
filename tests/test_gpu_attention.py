"""GPU parity: reference attention and loss/gradient through the C ABI.

Bar (relative Frobenius error against the float64 oracle on identical float32
inputs): 1e-4 for Y, lse, loss, gradient and output MSE.
"""
import math

import numpy as np
import pytest

import attention_distillation_amd as K
from oracle import kvsculpt as O
from synth import WORKLOADS, make_batch, tiny_workload
from tests.gpu_common import empty, host, rel, say, to_gpu, workspace

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _cases():
    return {
        "single-head-d64": (WORKLOADS[0], None),
        "qwen-one-layer": (WORKLOADS[1], None),
        "tiny64-ragged": (tiny_workload(d=64, N=80, m=10, g=1, F=40, layers=3, kv_heads=1), None),
        "tiny128-ragged": (tiny_workload(d=128, N=150, m=6, g=3, F=11, layers=1, kv_heads=2), None),
    }


def _ref_gpu(w, b):
    P, n, Z, d = b["Q"].shape[0], b["Q"].shape[1], b["Kz"].shape[1], b["Q"].shape[2]
    bt = K.Batch(P, d, Z, n)
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt))
    Y, lse = empty((P, n, d)), empty((P, n))
    K.kvs_reference_attn(ctx, bt, to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"]), Y, lse, ws)
    return host(Y), host(lse)


@pytest.mark.parametrize("name", list(_cases()))
def test_reference_attention_matches_oracle(name):
    w, _ = _cases()[name]
    b = make_batch(w, 0)
    say(f"[ref-attn] case={name} P={b['Q'].shape[0]} n={b['Q'].shape[1]} Z={b['Kz'].shape[1]} d={w.d}")
    Yg, lg = _ref_gpu(w, b)
    for p in range(b["Q"].shape[0]):
        Y, l = O.reference_attention(b["Q"][p], b["Kz"][p], b["Vz"][p], b["scale"])
        ey, el = rel(Yg[p], Y), rel(lg[p], l)
        say(f"   p={p} relY={ey:.2e} rel_lse={el:.2e}")
        assert ey <= TOL and el <= TOL


def _loss_case(name, state):
    """Per-problem fp32 inputs (Q, Y, lse, Kc, Vc) at a given optimizer state."""
    w, _ = _cases()[name]
    b = make_batch(w, 0)
    P = b["Q"].shape[0]
    s = b["scale"]
    rng = np.random.default_rng(5)
    probs = []
    for p in range(P):
        Q, Kz, Vz = b["Q"][p], b["Kz"][p], b["Vz"][p]
        Y, l = O.reference_attention(Q, Kz, Vz, s)
        Y32, l32 = Y.astype(np.float32), l.astype(np.float32)
        Z = Kz.shape[0]
        k = w.k0 if name in ("single-head-d64", "qwen-one-layer") else [1, 17, Z, 33][p % 4]
        k = min(k, Z)
        if state == "init":
            idx, Kc, Vc, ok = O.init_select_fit(Q, Kz, Y32, l32, k, s)
        elif state == "perturbed":
            idx, Kc, Vc, ok = O.init_select_fit(Q, Kz, Y32, l32, k, s)
            Kc = Kc + 1e-2 * rng.standard_normal(Kc.shape)
        else:
            t = int(state[1:])
            r = O.compress_problem(Q, Kz, Vz, k, s, O.CompressOptions(iters=t),
                                   Y=Y32.astype(np.float64), lse=l32.astype(np.float64))
            Kc, Vc = r["Kc"], r["Vc"]
        probs.append((Q, Y32, l32, Kc.astype(np.float32), Vc.astype(np.float32)))
    return w, b, probs


LOSS_CASES = [("single-head-d64", "init"), ("single-head-d64", "perturbed"), ("single-head-d64", "t5"), ("single-head-d64", "t20"),
              ("qwen-one-layer", "init"), ("tiny64-ragged", "init"), ("tiny128-ragged", "perturbed")]


@pytest.mark.parametrize("name,state", LOSS_CASES)
def test_loss_grad_matches_oracle(name, state):
    w, b, probs = _loss_case(name, state)
    P, n, d = b["Q"].shape
    Z = b["Kz"].shape[1]
    ks = [pr[3].shape[0] for pr in probs]
    say(f"[loss-grad] case={name} state={state} P={P} n={n} d={d} k={ks}")
    bt = K.Batch(P, d, Z, n, k=ks, scale=b["scale"])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt))
    Kc = to_gpu(np.concatenate([pr[3] for pr in probs]))
    Vc = to_gpu(np.concatenate([pr[4] for pr in probs]))
    Yt = to_gpu(np.stack([pr[1] for pr in probs]))
    lt = to_gpu(np.stack([pr[2] for pr in probs]))
    loss, mse = empty((P,)), empty((P,))
    grad = empty((sum(ks), d))
    K.kvs_loss_grad(ctx, bt, to_gpu(b["Q"]), Yt, lt, Kc, Vc, loss, grad, mse, ws)
    lg, gg, mg = host(loss), host(grad), host(mse)
    off = 0
    for p, (Q, Y32, l32, Kc32, Vc32) in enumerate(probs):
        L, g, aux = O.loss_grad(Q, Y32, l32, Kc32, Vc32, b["scale"])
        m = aux["out"] / (n * d)
        k = Kc32.shape[0]
        eL, eg, em = rel(lg[p], L), rel(gg[off:off + k], g), rel(mg[p], m)
        say(f"   p={p} k={k} L={L:.6g} relL={eL:.2e} relgrad={eg:.2e} relmse={em:.2e}")
        assert eL <= TOL and eg <= TOL and em <= TOL
        off += k


def test_loss_grad_zero_at_compress_zone():
    """k = Z with the zone's own keys and values: loss ~ 0 up to fp32 rounding."""
    w = WORKLOADS[0]
    b = make_batch(w, 0)
    Q, Kz, Vz = b["Q"][0], b["Kz"][0], b["Vz"][0]
    Y, l = O.reference_attention(Q, Kz, Vz, b["scale"])
    P, n, d = b["Q"].shape
    Z = Kz.shape[0]
    bt = K.Batch(1, d, Z, n, k=[Z])
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt))
    loss, grad = empty((1,)), empty((Z, d))
    K.kvs_loss_grad(ctx, bt, to_gpu(b["Q"]), to_gpu(Y.astype(np.float32)[None]),
                    to_gpu(l.astype(np.float32)[None]), to_gpu(Kz), to_gpu(Vz), loss, grad, None, ws)
    Lg = float(host(loss)[0])
    say(f"[zero] L={Lg:.3e} |Y|^2={float((Y ** 2).sum()):.3e}")
    assert 0 <= Lg <= 1e-9 * float((Y ** 2).sum())
