"""GPU check of the forward that reads stored scores.

After a value re-solve the keys have not moved, so kvs_compress takes the
loss at the new values from the scores stored by the last forward at those
keys instead of forming them again.  A stored score is exactly the float the
score product produced, so that loss must equal, bit for bit, the loss that
kvs_loss_grad computes at the returned (Kc, Vc) with the full forward.
"""
import numpy as np
import pytest

import attention_distillation_amd as K
from synth import WORKLOADS, make_batch, tiny_workload
from tests.gpu_common import empty, host, say, to_gpu, workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,w,T", [
    ("qwen-one-layer", WORKLOADS[1], 10),
    ("ragged-d64", tiny_workload(d=64, N=300, m=20, g=2, F=30, layers=2, kv_heads=2, k0=100), 15),
])
def test_loss_after_value_solve_equals_full_forward(name, w, T):
    b = make_batch(w, 0)
    P, n, d = b["Q"].shape
    ks = [w.k0] * P if name == "qwen-one-layer" else [40, 100, 150, 280]
    bt = K.Batch(P, d, w.Z, n, k=ks, scale=b["scale"])
    o = K.opts(iters=T)            # T a multiple of 5: the call ends with a value solve
    ctx = K.Context()
    ws = workspace(K.workspace_bytes(bt, o))
    Q, Kz, Vz = to_gpu(b["Q"]), to_gpu(b["Kz"]), to_gpu(b["Vz"])
    ktot = sum(ks)
    Kc, Vc = empty((ktot, d)), empty((ktot, d))
    loss, mse, l0 = empty((P,)), empty((P,)), empty((P,))
    flags = to_gpu(np.zeros(P, np.int32))
    say(f"[score-reuse] case={name} P={P} k={ks} T={T}")
    K.kvs_compress(ctx, bt, o, Q, Kz, Vz, Kc, Vc, loss, mse, l0, flags, ws)
    lc, mc = host(loss).copy(), host(mse).copy()
    Y, lse = empty((P, n, d)), empty((P, n))
    K.kvs_reference_attn(ctx, bt, Q, Kz, Vz, Y, lse, ws)
    l2, m2 = empty((P,)), empty((P,))
    K.kvs_loss_grad(ctx, bt, Q, Y, lse, Kc, Vc, l2, None, m2, ws)
    lf, mf = host(l2), host(m2)
    say(f"   compress loss {lc.tolist()} / full forward {lf.tolist()}")
    assert np.array_equal(lc, lf) and np.array_equal(mc, mf)
